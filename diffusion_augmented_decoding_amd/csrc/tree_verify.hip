// Psi-Spec tree verify (per-node rejection over a prefix tree) for gfx950.
//
// Method: Uno summary (hyper.ai, arXiv 2609.04010), section "方法", last
// paragraph -- the tree sampler verifies several candidates as a prefix tree,
// losslessly.  Read as multi-candidate speculative sampling (SpecInfer, Miao
// et al. 2023): siblings are tried in ascending node id; a rejected sibling
// replaces the running target r by max(0, r - q_d) / sum.
//
// Re-organisation for the GPU (same results up to rounding): with the
// siblings of one node sharing the draft marginal q, the target after j
// rejections has the closed form
//     r_j = max(0, p - c_j q) / D_j,   c_0 = 0, D_0 = 1,
//     c_{j+1} = c_j + D_j,             D_j = sum_v max(0, p_v - c_j q_v),
// (a zero mass D_j keeps (c, D) of step j-1, as the sequential rule keeps r).
// It depends only on j, not on the rejected tokens, so the masses of every
// node are computed in parallel before the walk instead of on its critical
// path.  Three launches:
//  1. tree_stats: softmax statistics of every AR row and draft row;
//  2. tree_residual: one workgroup per node, one streaming pass per child,
//     giving (c_j, D_j) after each child's rejection;
//  3. tree_walk_draw: one workgroup per tree; wave 0 walks the tree with
//     gathered probabilities and the (c, D) table, then the workgroup draws
//     the correction or bonus token by inverse CDF (block_draw).
#include "sampler_common.h"

namespace uno {

namespace {

constexpr int kMaxTree = 1024;

struct TreeCD {
  float c;
  float d;
};

size_t ws_stats_bytes(int batch, int n, int dmax) {
  return align_up(size_t(batch) * (n + dmax) * sizeof(RowStat), 256);
}

template <typename T>
__global__ __launch_bounds__(kStatThreads) void tree_stats_kernel(TreeVerifyArgs a, RowStat* stats) {
  const int rpb = a.n_tree + a.max_depth;
  const int row = blockIdx.x;
  const int b = row / rpb, j = row - b * rpb;
  const T* base = (j < a.n_tree)
                      ? static_cast<const T*>(a.p) + (int64_t(b) * a.n_tree + j) * a.vocab
                      : static_cast<const T*>(a.q) + (int64_t(b) * a.max_depth + (j - a.n_tree)) * a.vocab;
  row_stats_body<T>(base, a.vocab, a.scale_log2, -1, stats + row);
}

// Depth of node i, or -1 if the parent chain is malformed.
__device__ int node_depth(const int* par, int n, int i) {
  int d = 0;
  int j = i;
  while (j > 0) {
    const int pj = par[j];
    if (pj < 0 || pj >= j) return -1;
    j = pj;
    ++d;
  }
  return (j == 0 && par[0] == -1) ? d : -1;
}

template <typename T>
__global__ __launch_bounds__(kDrawThreads) void tree_residual_kernel(TreeVerifyArgs a, const RowStat* stats,
                                                                     TreeCD* cd) {
  __shared__ int par[kMaxTree];
  __shared__ float wsum[kDrawWaves];
  __shared__ int sh_depth;
  const int n = a.n_tree;
  const int b = blockIdx.x / n, i = blockIdx.x - (blockIdx.x / n) * n;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid / kWave;
  for (int v = tid; v < n; v += kDrawThreads) par[v] = a.parent[int64_t(b) * n + v];
  __syncthreads();
  if (tid == 0) sh_depth = node_depth(par, n, i);
  __syncthreads();
  const int depth = sh_depth;
  if (depth < 0 || depth >= a.max_depth) return;   // malformed, or no q row for children

  const int rpb = n + a.max_depth;
  const RowStat sp = stats[int64_t(b) * rpb + i];
  const RowStat sq = stats[int64_t(b) * rpb + n + depth];
  DrawRows<T> d;
  d.prow = static_cast<const T*>(a.p) + (int64_t(b) * n + i) * a.vocab;
  d.qrow = static_cast<const T*>(a.q) + (int64_t(b) * a.max_depth + depth) * a.vocab;
  d.mp = sp.m;
  d.inv_sp = 1.f / sp.s;
  d.mq = sq.m;
  d.inv_sq = 1.f / sq.s;
  d.vec_p = (reinterpret_cast<uintptr_t>(d.prow) & 15u) == 0;
  d.vec_q = (reinterpret_cast<uintptr_t>(d.qrow) & 15u) == 0;
  const float sl2 = a.scale_log2;
  const int vocab = a.vocab;

  float c_prev = 0.f, d_prev = 1.f;      // (c_{j-1}, D_{j-1})
  bool frozen = false;
  for (int ch = i + 1; ch < n; ++ch) {
    if (par[ch] != i) continue;
    float cj = c_prev + d_prev, dj = d_prev;
    if (!frozen) {
      d.c = cj;
      float s = 0.f;
      for (int e0 = tid * kEPT; e0 < vocab; e0 += kDrawTile) {
        float w[8];
        weights8<T>(d, e0, vocab, sl2, w);
#pragma unroll
        for (int j = 0; j < 8; ++j) s += w[j];
      }
      s = wave_sum(s);
      if (lane == 0) wsum[wave] = s;
      __syncthreads();
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < kDrawWaves; ++w) tot += wsum[w];
      __syncthreads();
      if (tot > 0.f) {
        dj = tot;
      } else {
        frozen = true;
        cj = c_prev;
        dj = d_prev;
      }
    } else {
      cj = c_prev;
      dj = d_prev;
    }
    if (tid == 0) cd[int64_t(b) * n + ch] = TreeCD{cj, dj};
    c_prev = cj;
    d_prev = dj;
  }
}

template <typename T>
__device__ __forceinline__ float prob_at(const T* row, int t, const RowStat& s, float sl2) {
  return fast_exp2(fmaf(load_logit<T>(row, t), sl2, -s.m)) / s.s;
}

template <typename T>
__global__ __launch_bounds__(kDrawThreads) void tree_walk_draw_kernel(TreeVerifyArgs a, const RowStat* stats,
                                                                      const TreeCD* cd) {
  __shared__ int par[kMaxTree];
  __shared__ DrawShared sh;
  __shared__ int sh_bad, sh_cur, sh_depth, sh_L, sh_haskids;
  __shared__ float sh_c;
  __shared__ int path[64];
  const int n = a.n_tree;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid / kWave;
  if (tid == 0) sh_bad = 0;
  __syncthreads();
  for (int v = tid; v < n; v += kDrawThreads) {
    const int pv = a.parent[int64_t(b) * n + v];
    par[v] = pv;
    const bool ok = (v == 0) ? (pv == -1) : (pv >= 0 && pv < v);
    if (!ok) sh_bad = 1;
  }
  __syncthreads();
  if (sh_bad) {
    if (tid < a.max_depth) a.out_path[int64_t(b) * a.max_depth + tid] = -1;
    if (tid == 0) {
      a.out_len[b] = -1;
      a.out_tok[b] = -1;
    }
    return;
  }

  const float sl2 = a.scale_log2;
  const int rpb = n + a.max_depth;
  const RowStat* st = stats + int64_t(b) * rpb;
  if (wave == 0) {
    int cur = 0, depth = 0, L = 0;
    float c = 0.f, dd = 1.f;
    bool haskids = false, bad = false;
    while (true) {
      bool accepted = false;
      haskids = false;
      c = 0.f;
      dd = 1.f;
      for (int base = cur + 1; base < n && !accepted; base += kWave) {
        const int v = base + lane;
        uint64_t mask = wave_ballot(v < n && par[v] == cur);
        while (mask && !accepted) {
          const int ch = base + int(__builtin_ctzll(mask));
          mask &= mask - 1;
          haskids = true;
          if (depth >= a.max_depth) {
            bad = true;
            break;
          }
          const int t = a.tokens[int64_t(b) * n + ch];
          const T* prow = static_cast<const T*>(a.p) + (int64_t(b) * n + cur) * a.vocab;
          const T* qrow = static_cast<const T*>(a.q) + (int64_t(b) * a.max_depth + depth) * a.vocab;
          float pt = 0.f, qt = 0.f;
          if (t >= 0 && t < a.vocab) {
            pt = prob_at<T>(prow, t, st[cur], sl2);
            qt = prob_at<T>(qrow, t, st[n + depth], sl2);
          }
          const float rt = fmaxf(fmaf(-c, qt, pt), 0.f) / dd;
          const float u = a.u_acc[int64_t(b) * n + ch];
          if (t >= 0 && t < a.vocab && u * qt < rt) {
            if (lane == 0) path[L] = ch;
            ++L;
            cur = ch;
            ++depth;
            accepted = true;
          } else {
            const TreeCD e = cd[int64_t(b) * n + ch];
            c = e.c;
            dd = e.d;
          }
        }
        if (bad) break;
      }
      if (!accepted || bad) break;
    }
    if (lane == 0) {
      sh_cur = cur;
      sh_depth = depth;
      sh_L = bad ? -1 : L;
      sh_haskids = haskids ? 1 : 0;
      sh_c = haskids ? c : 0.f;
    }
  }
  __syncthreads();
  const int L = sh_L;
  if (L < 0) {
    if (tid < a.max_depth) a.out_path[int64_t(b) * a.max_depth + tid] = -1;
    if (tid == 0) {
      a.out_len[b] = -1;
      a.out_tok[b] = -1;
    }
    return;
  }
  const int cur = sh_cur, depth = sh_depth;
  DrawRows<T> d;
  d.prow = static_cast<const T*>(a.p) + (int64_t(b) * n + cur) * a.vocab;
  const RowStat sp = st[cur];
  d.mp = sp.m;
  d.inv_sp = 1.f / sp.s;
  if (sh_haskids) {
    const RowStat sq = st[n + depth];
    d.qrow = static_cast<const T*>(a.q) + (int64_t(b) * a.max_depth + depth) * a.vocab;
    d.mq = sq.m;
    d.inv_sq = 1.f / sq.s;
    d.c = sh_c;
  } else {
    d.qrow = d.prow;
    d.mq = 0.f;
    d.inv_sq = 0.f;
    d.c = 0.f;
  }
  d.vec_p = (reinterpret_cast<uintptr_t>(d.prow) & 15u) == 0;
  d.vec_q = (reinterpret_cast<uintptr_t>(d.qrow) & 15u) == 0;
  int y;
  float mass;
  block_draw<T>(d, a.vocab, sl2, a.u_s[b], sh, y, mass);
  if (tid < a.max_depth) a.out_path[int64_t(b) * a.max_depth + tid] = (tid < L) ? path[tid] : -1;
  if (tid == 0) {
    a.out_len[b] = L;
    a.out_tok[b] = y;
  }
}

}  // namespace

size_t tree_verify_workspace_bytes(int batch, int n_tree, int max_depth, int vocab) {
  (void)vocab;
  return ws_stats_bytes(batch, n_tree, max_depth) + align_up(size_t(batch) * n_tree * sizeof(TreeCD), 256);
}

hipError_t launch_tree_verify(const TreeVerifyArgs& a, hipStream_t stream) {
  RowStat* stats = static_cast<RowStat*>(a.ws);
  TreeCD* cd = reinterpret_cast<TreeCD*>(static_cast<char*>(a.ws) + ws_stats_bytes(a.batch, a.n_tree, a.max_depth));
  const bool bf = a.dtype == UNO_BF16;
  {
    ProfileScope ps("uno_tree_stats", stream);
    const int rows = a.batch * (a.n_tree + a.max_depth);
    if (bf)
      hipLaunchKernelGGL(tree_stats_kernel<uint16_t>, dim3(rows), dim3(kStatThreads), 0, stream, a, stats);
    else
      hipLaunchKernelGGL(tree_stats_kernel<float>, dim3(rows), dim3(kStatThreads), 0, stream, a, stats);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfileScope ps("uno_tree_residual", stream);
    const int blocks = a.batch * a.n_tree;
    if (bf)
      hipLaunchKernelGGL(tree_residual_kernel<uint16_t>, dim3(blocks), dim3(kDrawThreads), 0, stream, a, stats, cd);
    else
      hipLaunchKernelGGL(tree_residual_kernel<float>, dim3(blocks), dim3(kDrawThreads), 0, stream, a, stats, cd);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfileScope ps("uno_tree_walk_draw", stream);
    if (bf)
      hipLaunchKernelGGL(tree_walk_draw_kernel<uint16_t>, dim3(a.batch), dim3(kDrawThreads), 0, stream, a, stats, cd);
    else
      hipLaunchKernelGGL(tree_walk_draw_kernel<float>, dim3(a.batch), dim3(kDrawThreads), 0, stream, a, stats, cd);
  }
  return hipGetLastError();
}

}  // namespace uno
