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
//     c_j = c_{j-1} + D_{j-1},         D_j = F(c_j) = sum_v max(0, p_v - c_j q_v),
// and a zero F(c_j) keeps (c, D) of step j-1 from then on (the sequential
// rule keeps r).  It depends only on j, not on the rejected tokens, so the
// masses of every node are computed before the walk, chunk-parallel:
//  1. tree_setup: validate the parent array, depth and child count per node;
//  2. tree_stats: softmax partials of every AR and draft row per chunk;
//  3. tree_round j = 1..max_children: F(c_j) per (node, chunk) for nodes with
//     at least j children (c_j replayed from the earlier rounds' sums);
//  4. tree_walk: one wave per tree walks it with gathered probabilities and
//     the (c, D) sequence, and describes the final draw;
//  5. draw_seg + draw_resolve: the inverse-CDF draw of the correction (or
//     bonus) token.
#include "sampler_common.h"

namespace uno {

namespace {

constexpr int kMaxTree = 1024;

struct NodeInfo {
  int depth;     // -1: tree malformed
  int nchild;
};

struct TreeWs {
  NodeInfo* info;   // [batch][n]
  int* bad;         // [batch]
  float2* part;     // [batch * (n + D)][nchunk]
  float* fpart;     // [max_children][batch * n][nchunk]
  DrawDesc* desc;   // [batch]
  float* seg;
};

// statistics split count of the tree's rows (AR rows + draft rows)
inline __host__ __device__ int tree_stat_splits(int batch, int n, int dmax, int vocab) {
  return stats_splits(batch * (n + dmax), vocab);
}

TreeWs tree_ws(void* base, int batch, int n, int dmax, int maxc, int vocab) {
  const int nc = num_chunks(vocab);
  const int ns = tree_stat_splits(batch, n, dmax, vocab);
  char* p = static_cast<char*>(base);
  TreeWs w;
  w.info = reinterpret_cast<NodeInfo*>(p);
  p += align_up(size_t(batch) * n * sizeof(NodeInfo), 256);
  w.bad = reinterpret_cast<int*>(p);
  p += align_up(size_t(batch) * sizeof(int), 256);
  w.part = reinterpret_cast<float2*>(p);
  p += align_up(size_t(batch) * (n + dmax) * ns * sizeof(float2), 256);
  w.fpart = reinterpret_cast<float*>(p);
  p += align_up(size_t(maxc > 0 ? maxc : 1) * batch * n * nc * sizeof(float), 256);
  w.desc = reinterpret_cast<DrawDesc*>(p);
  p += align_up(size_t(batch) * sizeof(DrawDesc), 256);
  w.seg = reinterpret_cast<float*>(p);
  return w;
}

// Validates the tree (parent[0] = -1, 0 <= parent[i] < i, depth <= max_depth,
// at most max_children children, nodes with children at depth < max_depth).
__global__ __launch_bounds__(1024) void tree_setup_kernel(TreeVerifyArgs a, TreeWs w) {
  __shared__ int par[kMaxTree];
  __shared__ int sh_bad;
  const int n = a.n_tree, b = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) sh_bad = 0;
  __syncthreads();
  for (int v = tid; v < n; v += 1024) {
    const int pv = a.parent[int64_t(b) * n + v];
    par[v] = pv;
    if ((v == 0) ? (pv != -1) : (pv < 0 || pv >= v)) sh_bad = 1;
  }
  __syncthreads();
  const bool bad_shape = sh_bad != 0;
  for (int v = tid; v < n; v += 1024) {
    int depth = -1, nchild = 0;
    if (!bad_shape) {
      int d = 0, j = v;
      while (j > 0 && d <= a.max_depth) {
        j = par[j];
        ++d;
      }
      depth = (d <= a.max_depth) ? d : -1;
      for (int u = v + 1; u < n; ++u) nchild += (par[u] == v);
      if (depth < 0 || nchild > a.max_children || (nchild > 0 && depth >= a.max_depth)) sh_bad = 1;
    }
    w.info[int64_t(b) * n + v] = NodeInfo{depth, nchild};
  }
  __syncthreads();
  if (tid == 0) w.bad[b] = sh_bad;
}

template <typename T>
__device__ __forceinline__ const T* tree_row(const TreeVerifyArgs& a, int b, int j) {
  return (j < a.n_tree) ? static_cast<const T*>(a.p) + (int64_t(b) * a.n_tree + j) * a.vocab
                        : static_cast<const T*>(a.q) + (int64_t(b) * a.max_depth + (j - a.n_tree)) * a.vocab;
}

template <typename T>
__global__ __launch_bounds__(kChunkThreads) void tree_stats_kernel(TreeVerifyArgs a, TreeWs w) {
  const int row = blockIdx.x, c = blockIdx.y, ns = gridDim.y;
  const int rpb = a.n_tree + a.max_depth;
  const int b = row / rpb, j = row - b * rpb;
  const int span = split_span(a.vocab, ns);
  const int lo = c * span, hi = min(a.vocab, lo + span);
  const float2 r = range_stats<T>(tree_row<T>(a, b, j), lo, hi, a.scale_log2);
  if (threadIdx.x == 0) w.part[int64_t(row) * ns + c] = r;
}

// (c, D) after `j` rejections among the children of node `node` (replayed
// from the per-round chunk sums, each summed by the whole calling wave);
// frozen once a mass is zero.
__device__ __forceinline__ void replay_cd(const float* fpart, int bn_total, int nc, int64_t node_idx, int j,
                                          float& c, float& D, bool& frozen) {
  c = 0.f;
  D = 1.f;
  frozen = false;
  for (int t = 1; t <= j; ++t) {
    if (frozen) break;
    const float F = wave_sum_range(fpart + (int64_t(t - 1) * bn_total + node_idx) * nc, nc);
    if (F > 0.f) {
      c = c + D;
      D = F;
    } else {
      frozen = true;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kChunkThreads) void tree_round_kernel(TreeVerifyArgs a, TreeWs w, int j) {
  const int node_idx = blockIdx.x, c = blockIdx.y, nc = gridDim.y;
  const int n = a.n_tree;
  const int b = node_idx / n;
  const int bn_total = a.batch * n;
  float* dst = w.fpart + (int64_t(j - 1) * bn_total + node_idx) * nc + c;
  const NodeInfo inf = w.info[node_idx];
  if (w.bad[b] || inf.nchild < j) {
    if (threadIdx.x == 0) *dst = 0.f;
    return;
  }
  float cc, D;
  bool frozen;
  replay_cd(w.fpart, bn_total, nc, node_idx, j - 1, cc, D, frozen);
  if (frozen) {
    if (threadIdx.x == 0) *dst = 0.f;
    return;
  }
  const int i = node_idx - b * n;
  const int rpb = n + a.max_depth;
  const int ns = tree_stat_splits(a.batch, n, a.max_depth, a.vocab);
  const RowStat sp = wave_merge_chunks(w.part + (int64_t(b) * rpb + i) * ns, ns);
  const RowStat sq = wave_merge_chunks(w.part + (int64_t(b) * rpb + n + inf.depth) * ns, ns);
  DrawDesc d;
  d.prow = tree_row<T>(a, b, i);
  d.qrow = tree_row<T>(a, b, n + inf.depth);
  d.mp = sp.m;
  d.inv_sp = 1.f / sp.s;
  d.mq = sq.m;
  d.inv_sq = 1.f / sq.s;
  d.c = cc + D;
  d.active = 1;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const bool vp = row_vec_ok(static_cast<const T*>(d.prow)), vq = row_vec_ok(static_cast<const T*>(d.qrow));
  float s = 0.f;
  // wave w covers segments 4w..4w+3 of the chunk; lanes read consecutive vectors
#pragma unroll
  for (int q = 0; q < kSegPerChunk / (kChunkThreads / kWave); ++q) {
    const int e0 = c * kChunk + (wave * (kSegPerChunk / (kChunkThreads / kWave)) + q) * kSegLen + lane * 8;
    float wv[8], pw[8];
    weights8<T>(d, e0, a.vocab, a.scale_log2, vp, vq, wv, pw);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += wv[e];
  }
  s = wave_sum(s);
  __shared__ float ws[kChunkThreads / kWave];
  if ((tid & 63) == 0) ws[tid / kWave] = s;
  __syncthreads();
  if (tid == 0) {
    float tot = 0.f;
#pragma unroll
    for (int q = 0; q < kChunkThreads / kWave; ++q) tot += ws[q];
    *dst = tot;
  }
}

template <typename T>
__device__ __forceinline__ float prob_at(const T* row, int t, const RowStat& s, float sl2) {
  return fast_exp2(fmaf(load_logit<T>(row, t), sl2, -s.m)) / s.s;
}

template <typename T>
__global__ __launch_bounds__(kWave) void tree_walk_kernel(TreeVerifyArgs a, TreeWs w) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int n = a.n_tree, nc = num_chunks(a.vocab), rpb = n + a.max_depth;
  const int ns = tree_stat_splits(a.batch, n, a.max_depth, a.vocab);
  const int bn_total = a.batch * n;
  const float sl2 = a.scale_log2;
  int32_t* path_out = a.out_path + int64_t(b) * a.max_depth;
  if (w.bad[b]) {
    for (int t = lane; t < a.max_depth; t += kWave) path_out[t] = -1;
    if (lane == 0) {
      a.out_len[b] = -1;
      DrawDesc d{};
      d.active = 0;
      w.desc[b] = d;
    }
    return;
  }
  const int32_t* par = a.parent + int64_t(b) * n;
  int cur = 0, depth = 0, L = 0;
  float c = 0.f, D = 1.f;
  bool frozen = false, haskids = false;
  while (true) {
    const RowStat sp = wave_merge_chunks(w.part + (int64_t(b) * rpb + cur) * ns, ns);
    RowStat sq{};
    const bool has_q = depth < a.max_depth;
    if (has_q) sq = wave_merge_chunks(w.part + (int64_t(b) * rpb + n + depth) * ns, ns);
    const T* prow = tree_row<T>(a, b, cur);
    const T* qrow = has_q ? tree_row<T>(a, b, n + depth) : prow;
    c = 0.f;
    D = 1.f;
    frozen = false;
    haskids = false;
    bool accepted = false;
    int rank = 0;
    for (int base = cur + 1; base < n && !accepted; base += kWave) {
      const int v = base + lane;
      uint64_t mask = wave_ballot(v < n && par[v] == cur);
      while (mask && !accepted) {
        const int ch = base + int(__builtin_ctzll(mask));
        mask &= mask - 1;
        haskids = true;
        ++rank;
        const int t = a.tokens[int64_t(b) * n + ch];
        float pt = 0.f, qt = 0.f;
        if (t >= 0 && t < a.vocab) {
          pt = prob_at<T>(prow, t, sp, sl2);
          qt = prob_at<T>(qrow, t, sq, sl2);
        }
        const float rt = fmaxf(fmaf(-c, qt, pt), 0.f) / D;
        if (t >= 0 && t < a.vocab && a.u_acc[int64_t(b) * n + ch] * qt < rt) {
          if (lane == 0) path_out[L] = ch;
          ++L;
          cur = ch;
          ++depth;
          accepted = true;
        } else if (!frozen) {   // residual after this rejection
          const float F =
              wave_sum_range(w.fpart + (int64_t(rank - 1) * bn_total + int64_t(b) * n + cur) * nc, nc);
          if (F > 0.f) {
            c = c + D;
            D = F;
          } else {
            frozen = true;
          }
        }
      }
    }
    if (!accepted) {
      if (lane == 0) {
        DrawDesc d;
        d.prow = prow;
        d.qrow = qrow;
        d.mp = sp.m;
        d.inv_sp = 1.f / sp.s;
        d.mq = has_q ? sq.m : 0.f;
        d.inv_sq = has_q ? 1.f / sq.s : 0.f;
        d.c = haskids ? c : 0.f;
        d.active = 1;
        w.desc[b] = d;
        a.out_len[b] = L;
      }
      break;
    }
  }
  for (int t = L + lane; t < a.max_depth; t += kWave) path_out[t] = -1;
}

template <typename T>
hipError_t launch_tree(const TreeVerifyArgs& a, hipStream_t stream) {
  const int nc = num_chunks(a.vocab);
  TreeWs w = tree_ws(a.ws, a.batch, a.n_tree, a.max_depth, a.max_children, a.vocab);
  {
    ProfileScope ps("uno_tree_setup", stream);
    hipLaunchKernelGGL(tree_setup_kernel, dim3(a.batch), dim3(1024), 0, stream, a, w);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfileScope ps("uno_tree_stats", stream);
    hipLaunchKernelGGL(tree_stats_kernel<T>, dim3(a.batch * (a.n_tree + a.max_depth),
                       tree_stat_splits(a.batch, a.n_tree, a.max_depth, a.vocab)), dim3(kChunkThreads), 0, stream, a,
                       w);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int j = 1; j <= a.max_children; ++j) {
    ProfileScope ps("uno_tree_round", stream);
    hipLaunchKernelGGL(tree_round_kernel<T>, dim3(a.batch * a.n_tree, nc), dim3(kChunkThreads), 0, stream, a, w, j);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    ProfileScope ps("uno_tree_walk", stream);
    hipLaunchKernelGGL(tree_walk_kernel<T>, dim3(a.batch), dim3(kWave), 0, stream, a, w);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_draw<T>(w.desc, a.batch, a.vocab, a.scale_log2, w.seg, a.u_s, a.out_tok, nullptr, stream,
                        "uno_tree_draw_seg", "uno_tree_draw_resolve");
}

}  // namespace

size_t tree_verify_workspace_bytes(int batch, int n, int dmax, int maxc, int vocab) {
  const int nc = num_chunks(vocab);
  const int ns = tree_stat_splits(batch, n, dmax, vocab);
  return align_up(size_t(batch) * n * sizeof(NodeInfo), 256) + align_up(size_t(batch) * sizeof(int), 256) +
         align_up(size_t(batch) * (n + dmax) * ns * sizeof(float2), 256) +
         align_up(size_t(maxc > 0 ? maxc : 1) * batch * n * nc * sizeof(float), 256) +
         align_up(size_t(batch) * sizeof(DrawDesc), 256) + draw_seg_bytes(batch, vocab);
}

hipError_t launch_tree_verify(const TreeVerifyArgs& a, hipStream_t stream) {
  return a.dtype == UNO_BF16 ? launch_tree<uint16_t>(a, stream) : launch_tree<float>(a, stream);
}

}  // namespace uno
