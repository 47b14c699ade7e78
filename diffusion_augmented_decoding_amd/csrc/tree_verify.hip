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
// masses of every node are computed before the walk, chunk-parallel.
//
// Two launches:
//  1. tree_stats: softmax partials of every AR and draft row per split; one
//     extra block per tree validates its parent array (depth and child count
//     of every node); a few more blocks mark the values the second launch
//     publishes as not yet written and reset its work counter.
//  2. tree_flow: blocks take work items in increasing order from a counter:
//     first one gather per node with children (its children's p and q at
//     their tokens, published per child), then the residual rounds (round j,
//     node, 8192-token chunk: F(c_j) of the chunk), then one walk per tree
//     (one wave walks it with the gathered probabilities and the (c, D)
//     sequences, waiting for a node's rounds only once a child is rejected),
//     then the draw's segment masses per (tree, chunk), then one inverse-CDF
//     search per tree.  An item waits
//     only for values that items with smaller numbers publish, so the item
//     with the smallest number in progress always has its inputs and the
//     launch finishes for any number of resident blocks.  Published values
//     (a chunk's F, a tree's walk result, a segment mass) are single words,
//     written and read with device-scope atomic stores and loads, and each is
//     its own ready flag (a sentinel until written).
//
// Siblings drawn without replacement (recursive rejection sampling without
// replacement, Jeon et al. 2024): sibling j is tested against q_j, q with the
// tokens of siblings 1..j-1 removed and renormalised by Z_j = 1 - (their q
// mass), and a rejection subtracts q_j.  With C_0 = 0, D_0 = 1 the residual
// after j rejections is r_j = rho_j / D_j with
//     rho_j(v) = max(0, p_v - C_j q_v)          for v not removed,
//     rho_j(t_k) = max(0, p_{t_k} - C_k q_{t_k}) for the token of sibling k <= j
//                                                 (first occurrence),
//     C_j = C_{j-1} + D_{j-1} / Z_j,   D_j = sum_v rho_j(v)
//         = F(C_j) + sum_{k<j} [max(0, p_{t_k} - C_k q_{t_k}) - max(0, p_{t_k} - C_j q_{t_k})],
// a zero D_j freezing (C, D) as before and a Z_j without mass (below kZEps)
// leaving C unchanged.  The tokens of the siblings are inputs, so the (C, D)
// sequence is again known before the walk: the rounds compute F(C_j) chunk-
// parallel, and every replay adds the per-sibling corrections, one sibling
// per lane.  The final draw's weights are rho of the last state: the segment
// masses and the element scan put max(0, p - C_k q) in place of the common
// weight at every removed token.
#include "sampler_common.h"

namespace uno {

namespace {

constexpr int kMaxTree = 1024;
constexpr float kUnset = -1.f;                     // published masses are >= 0
constexpr uint64_t kWalkUnset = ~uint64_t(0);      // node field 2047: no tree has it
constexpr int kSpinMax = 1 << 22;                  // waits end long before; a bound, not a timeout

struct NodeInfo {
  int depth;     // -1: tree malformed
  int nchild;
};

struct TreeWs {
  NodeInfo* info;    // [batch][n]
  int* bad;          // [batch]
  float2* part;      // [batch * (n + D)][ns]
  float* fpart;      // [max_children][batch * n][nchunk]: F of round j per chunk
  uint64_t* walk;    // [batch]: the walk's result (see pack_walk)
  float* seg;        // [batch][nchunk][2 * kSegPerChunk]: segment masses of w, then p
  int* queue;        // work counter of the flow launch
  int* err;          // a wait ran past kSpinMax (never expected)
  int* cnt;          // [batch]: nodes with children (0 for a malformed tree)
  int* list;         // [batch][n]: those nodes in increasing id
  int* kids;         // without replacement: [batch][n][max_children] children in increasing id
  float* ck;         // without replacement: [batch][64] C_k of the walk's last node
  uint64_t* kidpq;   // [batch][n]: (p, q) at a node's token under its parent's AR row and its depth's draft row
};
constexpr float kZEps = 1e-6f;   // a remaining draft mass below this is taken as none (fp32 resolves no less)
constexpr int kMaxWorChildren = 64;
constexpr int kMaxListTrees = 1024;   // trees whose node lists the flow launch indexes

inline __host__ __device__ int tree_stat_splits(int batch, int n, int dmax, int vocab) {
  return stats_splits(batch * (n + dmax), vocab);
}

TreeWs tree_ws(void* base, int batch, int n, int dmax, int maxc, int vocab, int wor) {
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
  w.walk = reinterpret_cast<uint64_t*>(p);
  p += align_up(size_t(batch) * sizeof(uint64_t), 256);
  w.seg = reinterpret_cast<float*>(p);
  p += draw_seg_bytes(batch, vocab);
  w.queue = reinterpret_cast<int*>(p);
  w.err = w.queue + 1;
  p += 256;
  w.cnt = reinterpret_cast<int*>(p);
  p += align_up(size_t(batch) * sizeof(int), 256);
  w.list = reinterpret_cast<int*>(p);
  p += align_up(size_t(batch) * n * sizeof(int), 256);
  w.kidpq = reinterpret_cast<uint64_t*>(p);
  p += align_up(size_t(batch) * n * sizeof(uint64_t), 256);
  w.kids = nullptr;
  w.ck = nullptr;
  if (wor) {
    w.kids = reinterpret_cast<int*>(p);
    p += align_up(size_t(batch) * n * (maxc > 0 ? maxc : 1) * sizeof(int), 256);
    w.ck = reinterpret_cast<float*>(p);
  }
  return w;
}

__device__ __forceinline__ float load_pub(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_pub(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Validates tree b (parent[0] = -1, 0 <= parent[i] < i, depth <= max_depth,
// at most max_children children, nodes with children at depth < max_depth).
// The whole block calls it.
__device__ __forceinline__ void tree_setup_body(const TreeVerifyArgs& a, const TreeWs& w, int b) {
  __shared__ int par[kMaxTree];
  __shared__ int sh_bad;
  const int n = a.n_tree, tid = threadIdx.x, nt = blockDim.x;
  if (tid == 0) sh_bad = 0;
  __syncthreads();
  for (int v = tid; v < n; v += nt) {
    const int pv = a.parent[int64_t(b) * n + v];
    par[v] = pv;
    if ((v == 0) ? (pv != -1) : (pv < 0 || pv >= v)) sh_bad = 1;
  }
  __syncthreads();
  const bool bad_shape = sh_bad != 0;
  for (int v = tid; v < n; v += nt) {
    int depth = -1, nchild = 0;
    if (!bad_shape) {
      int d = 0, j = v;
      while (j > 0 && d <= a.max_depth) {
        j = par[j];
        ++d;
      }
      depth = (d <= a.max_depth) ? d : -1;
      if (a.wor) {   // the children in increasing id (at most max_children stored)
        int* kl = w.kids + (int64_t(b) * n + v) * a.max_children;
        for (int u = v + 1; u < n; ++u) {
          if (par[u] == v) {
            if (nchild < a.max_children) kl[nchild] = u;
            ++nchild;
          }
        }
      } else {
        for (int u = v + 1; u < n; ++u) nchild += (par[u] == v);
      }
      if (depth < 0 || nchild > a.max_children || (nchild > 0 && depth >= a.max_depth)) sh_bad = 1;
    }
    w.info[int64_t(b) * n + v] = NodeInfo{depth, nchild};
  }
  __syncthreads();
  if (tid == 0) w.bad[b] = sh_bad;
  // the nodes with children, in increasing id (wave 0; none for a malformed tree)
  if (tid < kWave) {
    int total = 0;
    if (!sh_bad) {
      for (int base = 0; base < n; base += kWave) {
        const int v = base + tid;
        const bool has = v < n && w.info[int64_t(b) * n + v].nchild > 0;
        const uint64_t m = wave_ballot(has);
        if (has) w.list[int64_t(b) * n + total + __builtin_popcountll(m & ((uint64_t(1) << tid) - 1))] = v;
        total += __builtin_popcountll(m);
      }
    }
    if (tid == 0) w.cnt[b] = total;
  }
}

template <typename T>
__device__ __forceinline__ const T* tree_row(const TreeVerifyArgs& a, int b, int j) {
  return (j < a.n_tree) ? static_cast<const T*>(a.p) + (int64_t(b) * a.n_tree + j) * a.vocab
                        : static_cast<const T*>(a.q) + (int64_t(b) * a.max_depth + (j - a.n_tree)) * a.vocab;
}

// Blocks [0, nstat): (row, split) softmax partials; [nstat, nstat + batch):
// validation of one tree each; the rest: published values set to their
// sentinels, the work counter and the error flag to 0.
template <typename T>
__global__ __launch_bounds__(kChunkThreads) void tree_stats_kernel(TreeVerifyArgs a, TreeWs w, int nstat,
                                                                   int ninit_blocks) {
  const int ns = tree_stat_splits(a.batch, a.n_tree, a.max_depth, a.vocab);
  const int blk = blockIdx.x;
  if (blk < nstat) {
    const int row = blk / ns, c = blk % ns;
    const int rpb = a.n_tree + a.max_depth;
    const int b = row / rpb, j = row - b * rpb;
    const int span = split_span(a.vocab, ns);
    const int lo = c * span, hi = min(a.vocab, lo + span);
    const float2 r = range_stats<T, false>(tree_row<T>(a, b, j), lo, hi, a.scale_log2);
    if (threadIdx.x == 0) w.part[int64_t(row) * ns + c] = r;
    return;
  }
  if (blk < nstat + a.batch) {
    tree_setup_body(a, w, blk - nstat);
    return;
  }
  const int nc = num_chunks(a.vocab);
  const int64_t nf = int64_t(a.max_children) * a.batch * a.n_tree * nc;
  const int64_t nseg = int64_t(a.batch) * nc * 2 * kSegPerChunk;
  const int64_t nck = a.wor ? int64_t(a.batch) * kMaxWorChildren : 0;
  const int64_t nkp = int64_t(a.batch) * a.n_tree;
  const int64_t stride = int64_t(ninit_blocks) * kChunkThreads;
  for (int64_t t = int64_t(blk - nstat - a.batch) * kChunkThreads + threadIdx.x;
       t < nf + nseg + a.batch + nck + nkp; t += stride) {
    if (t < nf)
      w.fpart[t] = kUnset;
    else if (t < nf + nseg)
      w.seg[t - nf] = kUnset;
    else if (t < nf + nseg + a.batch)
      w.walk[t - nf - nseg] = kWalkUnset;
    else if (t < nf + nseg + a.batch + nck)
      w.ck[t - nf - nseg - a.batch] = kUnset;
    else
      w.kidpq[t - nf - nseg - a.batch - nck] = kWalkUnset;
  }
  if (blk == nstat + a.batch && threadIdx.x == 0) {
    w.queue[0] = 0;
    w.err[0] = 0;
  }
}

// Sum of the nc (<= 128) published chunk values at v by one whole wave, once
// every one of them is written: lane l holds v[l] and v[l + 64]; the sum is
// taken in that order, then across lanes (same bits in every lane).
__device__ __forceinline__ float wave_sum_published(const float* v, int nc, int* err) {
  const int lane = threadIdx.x & (kWave - 1);
  float x0 = 0.f, x1 = 0.f;
  for (int it = 0;; ++it) {
    x0 = lane < nc ? load_pub(v + lane) : 0.f;
    x1 = lane + kWave < nc ? load_pub(v + lane + kWave) : 0.f;
    if (!wave_ballot(x0 < 0.f || x1 < 0.f)) break;
    if (it == kSpinMax) {
      if (lane == 0) atomicOr(err, 1);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  float s = 0.f;
  if (lane < nc) s += x0;
  if (lane + kWave < nc) s += x1;
  return wave_sum(s);
}

// F of rounds r0 .. r0 + cnt - 1 (cnt <= kRoundBatch) of one node, by one
// whole wave, once all of them are published: the round values sit nc apart
// starting at v (round r0).  Each F is summed exactly as wave_sum_published
// sums it; all loads of a wait iteration are in flight together.
constexpr int kRoundBatch = 8;
__device__ __forceinline__ void wave_sums_published(const float* v, int64_t round_stride, int cnt, int nc, int* err,
                                                    float (&F)[kRoundBatch]) {
  const int lane = threadIdx.x & (kWave - 1);
  float x0[kRoundBatch], x1[kRoundBatch];
  for (int it = 0;; ++it) {
    bool missing = false;
#pragma unroll
    for (int r = 0; r < kRoundBatch; ++r) {
      x0[r] = (r < cnt && lane < nc) ? load_pub(v + r * round_stride + lane) : 0.f;
      x1[r] = (r < cnt && lane + kWave < nc) ? load_pub(v + r * round_stride + lane + kWave) : 0.f;
      missing |= x0[r] < 0.f || x1[r] < 0.f;
    }
    if (!wave_ballot(missing)) break;
    if (it == kSpinMax) {
      if (lane == 0) atomicOr(err, 1);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
#pragma unroll
  for (int r = 0; r < kRoundBatch; ++r) {
    float s = 0.f;
    if (lane < nc) s += x0[r];
    if (lane + kWave < nc) s += x1[r];
    F[r] = wave_sum(s);
  }
}

template <typename T>
__device__ __forceinline__ float prob_at(const T* row, int t, const RowStat& s, float sl2) {
  return fast_exp2(fmaf(load_logit<T>(row, t), sl2, -s.m)) / s.s;
}

// ---------------------------------------------------------------- without replacement
// Child k (increasing id) of a node in lane k < m, by one whole wave: its id,
// token, uniform, p and q at the token, and whether it is the first child with
// that token (fi: the lane of the first one, for a repeated token; -1 else).
struct Sib {
  int ch, t, fi;
  float p, q, u;
  bool first;
};
template <typename T>
__device__ __forceinline__ Sib load_sib(const TreeVerifyArgs& a, const TreeWs& w, int b, int node, int m,
                                        const T* prow, const T* qrow, const RowStat& sp, const RowStat& sq) {
  const int lane = threadIdx.x & (kWave - 1);
  Sib s{-1, -1, -1, 0.f, 0.f, 1.f, false};
  const bool in = lane < m;
  if (in) {
    s.ch = w.kids[(int64_t(b) * a.n_tree + node) * a.max_children + lane];
    s.t = a.tokens[int64_t(b) * a.n_tree + s.ch];
    s.u = a.u_acc[int64_t(b) * a.n_tree + s.ch];
    if (s.t >= 0 && s.t < a.vocab) {
      s.p = prob_at<T>(prow, s.t, sp, a.scale_log2);
      s.q = prob_at<T>(qrow, s.t, sq, a.scale_log2);
    }
  }
  const bool valid = in && s.t >= 0 && s.t < a.vocab;
  for (int k = 0; k + 1 < m; ++k) {
    const int tk = __shfl(s.t, k);
    if (valid && k < lane && tk == s.t && s.fi < 0) s.fi = k;
  }
  s.first = valid && s.fi < 0;
  return s;
}

struct WorState {
  float C, D, Z;
  bool frozen;
};

// The C at which the next rejection subtracts q (C_j from state j - 1).
__device__ __forceinline__ float wor_next_c(const WorState& st) {
  return (!st.frozen && st.Z > kZEps) ? st.C + st.D / st.Z : st.C;
}

// Rejection of sibling j (1-based, lane j - 1) with F = F(C_j) summed over the
// vocabulary; ak (per lane): max(0, p - C_k q) of that lane's sibling once
// removed.  Returns C_j, the C at which the sibling's token was removed.
// Whole wave.
__device__ __forceinline__ float wor_step(WorState& st, const Sib& s, int j, float F, float& ak) {
  const int lane = threadIdx.x & (kWave - 1);
  const int l = j - 1;
  const bool fj = __shfl(s.first ? 1 : 0, l) != 0;
  const float qj = __shfl(s.q, l);
  if (!st.frozen) {
    const float Cn = wor_next_c(st);
    // tokens removed before: their rho stays at their own C_k (each term >= 0)
    const float corr = wave_sum((lane < l && s.first) ? ak - fmaxf(fmaf(-Cn, s.q, s.p), 0.f) : 0.f);
    const float Dn = F + corr;
    if (Dn > 0.f) {
      st.C = Cn;
      st.D = Dn;
    } else {
      st.frozen = true;
    }
  }
  if (lane == l && s.first) ak = fmaxf(fmaf(-st.C, s.q, s.p), 0.f);
  if (fj) st.Z -= qj;
  return st.C;
}

// Replacement weights of the removed tokens of a draw: lane k < m holds
// max(0, p - C_k q) of its sibling's token when it is that token's first
// occurrence.  Waits for the walk's C_k (published single words).
template <typename T>
__device__ __forceinline__ Sib wor_removed(const TreeVerifyArgs& a, const TreeWs& w, int b, int node, int depth,
                                           float& repl) {
  const int lane = threadIdx.x & (kWave - 1);
  const int n = a.n_tree, rpb = n + a.max_depth;
  const int ns = tree_stat_splits(a.batch, n, a.max_depth, a.vocab);
  const int m = w.info[int64_t(b) * n + node].nchild;
  Sib s{-1, -1, -1, 0.f, 0.f, 1.f, false};
  repl = 0.f;
  if (m == 0) return s;
  const RowStat sp = wave_merge_chunks(w.part + (int64_t(b) * rpb + node) * ns, ns);
  const RowStat sq = wave_merge_chunks(w.part + (int64_t(b) * rpb + n + depth) * ns, ns);
  s = load_sib<T>(a, w, b, node, m, tree_row<T>(a, b, node), tree_row<T>(a, b, n + depth), sp, sq);
  float ck = 0.f;
  for (int it = 0;; ++it) {
    ck = lane < m ? load_pub(w.ck + int64_t(b) * kMaxWorChildren + lane) : 0.f;
    if (!wave_ballot(ck < 0.f)) break;
    if (it == kSpinMax) {
      if (lane == 0) atomicOr(w.err, 1);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  repl = s.first ? fmaxf(fmaf(-ck, s.q, s.p), 0.f) : 0.f;
  return s;
}

// Puts the removed tokens' weights into the 8 weights of elements e0..e0+7.
__device__ __forceinline__ void wor_patch(float (&wv)[8], int e0, const Sib& s, float repl, int m) {
  for (int k = 0; k < m; ++k) {
    const bool fk = __shfl(s.first ? 1 : 0, k) != 0;
    const int tk = __shfl(s.t, k);
    const float rk = __shfl(repl, k);
    if (fk) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (tk == e0 + e) wv[e] = rk;
    }
  }
}

// ---------------------------------------------------------------- flow items
// Gather of node i of tree b (one whole wave): for every child v of the node,
// p and q at v's token (p from the node's AR row, q from the draft row of the
// children's depth), published as one word per child (all ones until written;
// an out-of-range token gives (0, 0)).
template <typename T>
__device__ void gather_item(const TreeVerifyArgs& a, const TreeWs& w, int node_idx) {
  const int lane = threadIdx.x & (kWave - 1);
  const int n = a.n_tree, rpb = n + a.max_depth;
  const int b = node_idx / n, i = node_idx - b * n;
  if (w.bad[b]) return;   // the walk publishes the malformed result without reading these
  const NodeInfo inf = w.info[node_idx];
  if (inf.nchild == 0) return;
  const int ns = tree_stat_splits(a.batch, n, a.max_depth, a.vocab);
  RowStat st[2];
  wave_merge_two(w.part + (int64_t(b) * rpb + i) * ns, w.part + (int64_t(b) * rpb + n + inf.depth) * ns, ns, st);
  const T* prow = tree_row<T>(a, b, i);
  const T* qrow = tree_row<T>(a, b, n + inf.depth);
  const int32_t* par = a.parent + int64_t(b) * n;
  for (int base = i + 1; base < n; base += kWave) {
    const int v = base + lane;
    if (v < n && par[v] == i) {
      const int t = a.tokens[int64_t(b) * n + v];
      float pt = 0.f, qt = 0.f;
      if (t >= 0 && t < a.vocab) {
        pt = prob_at<T>(prow, t, st[0], a.scale_log2);
        qt = prob_at<T>(qrow, t, st[1], a.scale_log2);
      }
      __hip_atomic_store(w.kidpq + int64_t(b) * n + v,
                         uint64_t(__float_as_uint(pt)) | (uint64_t(__float_as_uint(qt)) << 32), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Round j (1-based) of node node_idx, chunk c: F(c_j) of the chunk, with
// (c_j, D_j) replayed from the node's earlier rounds.  Whole block.
template <typename T>
__device__ void round_item(const TreeVerifyArgs& a, const TreeWs& w, int j, int node_idx, int c) {
  const int n = a.n_tree, nc = num_chunks(a.vocab);
  const int b = node_idx / n, i = node_idx - b * n;
  const int bn_total = a.batch * n;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  float* dst = w.fpart + (int64_t(j - 1) * bn_total + node_idx) * nc + c;
  const NodeInfo inf = w.info[node_idx];
  if (w.bad[b] || inf.nchild < j) {
    if (tid == 0) store_pub(dst, 0.f);
    return;
  }
  __shared__ float sh_cd[2];
  __shared__ int sh_frozen;
  __shared__ RowStat sh_st[2];
  if (wave == 1) {   // the merged statistics of the node's AR row and its depth's draft row
    const int rpb = n + a.max_depth;
    const int ns = tree_stat_splits(a.batch, n, a.max_depth, a.vocab);
    RowStat st[2];
    wave_merge_two(w.part + (int64_t(b) * rpb + i) * ns, w.part + (int64_t(b) * rpb + n + inf.depth) * ns, ns, st);
    if (lane == 0) {
      sh_st[0] = st[0];
      sh_st[1] = st[1];
    }
  }
  if (a.wor) {   // the replay needs the rows' statistics for the siblings' probabilities
    __syncthreads();
    if (wave == 0) {
      const Sib sb = load_sib<T>(a, w, b, i, inf.nchild, tree_row<T>(a, b, i), tree_row<T>(a, b, n + inf.depth),
                                 sh_st[0], sh_st[1]);
      WorState st{0.f, 1.f, 1.f, false};
      float ak = 0.f;
      const int64_t rs = int64_t(bn_total) * nc;
      for (int t0 = 1; t0 < j && !st.frozen; t0 += kRoundBatch) {
        const int cnt = min(kRoundBatch, j - t0);
        float F[kRoundBatch];
        wave_sums_published(w.fpart + (int64_t(t0 - 1) * bn_total + node_idx) * nc, rs, cnt, nc, w.err, F);
#pragma unroll
        for (int r = 0; r < kRoundBatch; ++r)
          if (r < cnt && !st.frozen) wor_step(st, sb, t0 + r, F[r], ak);
      }
      if (lane == 0) {
        sh_cd[0] = wor_next_c(st);
        sh_cd[1] = 0.f;
        sh_frozen = st.frozen ? 1 : 0;
      }
    }
  } else if (wave == 0) {
    float cc = 0.f, D = 1.f;
    bool frozen = false;
    const int64_t rs = int64_t(bn_total) * nc;   // between rounds of one node
    for (int t0 = 1; t0 < j && !frozen; t0 += kRoundBatch) {
      const int cnt = min(kRoundBatch, j - t0);
      float F[kRoundBatch];
      wave_sums_published(w.fpart + (int64_t(t0 - 1) * bn_total + node_idx) * nc, rs, cnt, nc, w.err, F);
#pragma unroll
      for (int r = 0; r < kRoundBatch; ++r) {
        if (r < cnt && !frozen) {
          if (F[r] > 0.f) {
            cc = cc + D;
            D = F[r];
          } else {
            frozen = true;
          }
        }
      }
    }
    if (lane == 0) {
      sh_cd[0] = cc;
      sh_cd[1] = D;
      sh_frozen = frozen ? 1 : 0;
    }
  }
  __syncthreads();
  if (sh_frozen) {
    if (tid == 0) store_pub(dst, 0.f);
    return;
  }
  const RowStat sp = sh_st[0], sq = sh_st[1];
  DrawDesc d;
  d.prow = tree_row<T>(a, b, i);
  d.qrow = tree_row<T>(a, b, n + inf.depth);
  d.mp = sp.m;
  d.inv_sp = 1.f / sp.s;
  d.mq = sq.m;
  d.inv_sq = 1.f / sq.s;
  d.c = sh_cd[0] + sh_cd[1];
  d.active = 1;
  const bool vp = row_vec_ok(static_cast<const T*>(d.prow)), vq = row_vec_ok(static_cast<const T*>(d.qrow));
  float s = 0.f;
  // wave v covers segments 4v .. 4v + 3 of the chunk; lanes read consecutive vectors
#pragma unroll
  for (int q = 0; q < kSegPerChunk / (kChunkThreads / kWave); ++q) {
    const int e0 = c * kChunk + (wave * (kSegPerChunk / (kChunkThreads / kWave)) + q) * kSegLen + lane * 8;
    float wv[8], pw[8];
    weights8<T, false>(d, e0, a.vocab, a.scale_log2, vp, vq, wv, pw);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += wv[e];
  }
  s = wave_sum(s);
  __shared__ float ws[kChunkThreads / kWave];
  if (lane == 0) ws[wave] = s;
  __syncthreads();
  if (tid == 0) {
    float tot = 0.f;
#pragma unroll
    for (int q = 0; q < kChunkThreads / kWave; ++q) tot += ws[q];
    store_pub(dst, tot);
  }
}

// The walk's result in one word: bits 0-31 the residual coefficient c (float
// bits), 32-42 the node whose AR row is drawn from, 43-53 its depth, bit 54:
// the depth has a draft row, bit 55: a draw is to be made (0: malformed tree).
__device__ __forceinline__ uint64_t pack_walk(float c, int node, int depth, bool has_q, bool active) {
  return uint64_t(__float_as_uint(c)) | (uint64_t(node) << 32) | (uint64_t(depth) << 43) |
         (uint64_t(has_q ? 1 : 0) << 54) | (uint64_t(active ? 1 : 0) << 55);
}

// The draw a walk result describes (statistics merged as the walk merged them).
template <typename T>
__device__ __forceinline__ DrawDesc walk_desc(const TreeVerifyArgs& a, const TreeWs& w, int b, uint64_t word) {
  const int n = a.n_tree, rpb = n + a.max_depth;
  const int ns = tree_stat_splits(a.batch, n, a.max_depth, a.vocab);
  const int node = int((word >> 32) & 2047), depth = int((word >> 43) & 2047);
  const bool has_q = ((word >> 54) & 1) != 0;
  DrawDesc d;
  d.active = int((word >> 55) & 1);
  d.c = __uint_as_float(uint32_t(word));
  const RowStat sp = wave_merge_chunks(w.part + (int64_t(b) * rpb + node) * ns, ns);
  d.prow = tree_row<T>(a, b, node);
  d.mp = sp.m;
  d.inv_sp = 1.f / sp.s;
  if (has_q) {
    const RowStat sq = wave_merge_chunks(w.part + (int64_t(b) * rpb + n + depth) * ns, ns);
    d.qrow = tree_row<T>(a, b, n + depth);
    d.mq = sq.m;
    d.inv_sq = 1.f / sq.s;
  } else {
    d.qrow = d.prow;
    d.mq = 0.f;
    d.inv_sq = 0.f;
  }
  return d;
}

// One whole wave walks tree b and publishes the draw it ends in.
template <typename T>
__device__ void walk_item(const TreeVerifyArgs& a, const TreeWs& w, int b) {
  const int lane = threadIdx.x & (kWave - 1);
  const int n = a.n_tree, nc = num_chunks(a.vocab), rpb = n + a.max_depth;
  const int ns = tree_stat_splits(a.batch, n, a.max_depth, a.vocab);
  const int bn_total = a.batch * n;
  const float sl2 = a.scale_log2;
  int32_t* path_out = a.out_path + int64_t(b) * a.max_depth;
  if (w.bad[b]) {
    for (int t = lane; t < a.max_depth; t += kWave) path_out[t] = -1;
    if (lane == 0) {
      a.out_len[b] = -1;
      __hip_atomic_store(w.walk + b, pack_walk(0.f, 0, 0, false, false), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  const int32_t* par = a.parent + int64_t(b) * n;
  int cur = 0, depth = 0, L = 0;
  while (true) {
    const bool has_q = depth < a.max_depth;
    float c = 0.f, D = 1.f;
    bool frozen = false, haskids = false, accepted = false;
    int rank = 0;
    // the residual masses after the first kRoundBatch rejections, waited for
    // together at the node's first rejection
    const int nkids = w.info[int64_t(b) * n + cur].nchild;
    float Fr[kRoundBatch];
    bool have_fr = false;
    for (int base = cur + 1; base < n && !accepted; base += kWave) {
      const int v = base + lane;
      const bool kid = v < n && par[v] == cur;
      uint64_t mask = wave_ballot(kid);
      // every child's token, gathered probabilities and uniform, loaded by its own lane
      int tl = -1;
      float ptl = 0.f, qtl = 0.f, ul = 1.f;
      if (kid) {
        tl = a.tokens[int64_t(b) * n + v];
        ul = a.u_acc[int64_t(b) * n + v];
      }
      uint64_t word = 0;
      for (int it = 0;; ++it) {
        word = kid ? __hip_atomic_load(w.kidpq + int64_t(b) * n + v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
        if (!wave_ballot(word == kWalkUnset)) break;
        if (it == kSpinMax) {
          if (lane == 0) atomicOr(w.err, 1);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      if (kid) {
        ptl = __uint_as_float(uint32_t(word));
        qtl = __uint_as_float(uint32_t(word >> 32));
      }
      while (mask && !accepted) {
        const int l = int(__builtin_ctzll(mask));
        const int ch = base + l;
        mask &= mask - 1;
        haskids = true;
        ++rank;
        const int t = __shfl(tl, l);
        const float pt = __shfl(ptl, l), qt = __shfl(qtl, l), u = __shfl(ul, l);
        const float rt = fmaxf(fmaf(-c, qt, pt), 0.f) / D;
        if (t >= 0 && t < a.vocab && u * qt < rt) {
          if (lane == 0) path_out[L] = ch;
          ++L;
          cur = ch;
          ++depth;
          accepted = true;
        } else if (!frozen) {   // residual after this rejection
          float F = 0.f;
          if (rank <= kRoundBatch) {
            if (!have_fr) {
              wave_sums_published(w.fpart + (int64_t(b) * n + cur) * nc, int64_t(bn_total) * nc,
                                  min(nkids, kRoundBatch), nc, w.err, Fr);
              have_fr = true;
            }
#pragma unroll
            for (int r = 0; r < kRoundBatch; ++r)
              if (r == rank - 1) F = Fr[r];
          } else {
            F = wave_sum_published(w.fpart + (int64_t(rank - 1) * bn_total + int64_t(b) * n + cur) * nc, nc, w.err);
          }
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
        a.out_len[b] = L;
        __hip_atomic_store(w.walk + b, pack_walk(haskids ? c : 0.f, cur, depth, has_q, true), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      break;
    }
  }
  for (int t = L + lane; t < a.max_depth; t += kWave) path_out[t] = -1;
}

// The walk of tree b with siblings drawn without replacement (one whole
// wave): at each node the children sit one per lane; sibling j is accepted iff
// u * q_j(t) < rho(t) / D, q_j(t) = q(t) / Z_j for a token not removed yet
// (0 for a repeated one or when no draft mass is left), rho(t) at the
// current C, or at C_k for a token first removed by sibling k.  The walk
// publishes C_k of every child of its last node, then the draw.
template <typename T>
__device__ void walk_item_wor(const TreeVerifyArgs& a, const TreeWs& w, int b) {
  const int lane = threadIdx.x & (kWave - 1);
  const int n = a.n_tree, nc = num_chunks(a.vocab), rpb = n + a.max_depth;
  const int ns = tree_stat_splits(a.batch, n, a.max_depth, a.vocab);
  const int bn_total = a.batch * n;
  int32_t* path_out = a.out_path + int64_t(b) * a.max_depth;
  if (w.bad[b]) {
    for (int t = lane; t < a.max_depth; t += kWave) path_out[t] = -1;
    if (lane == 0) {
      a.out_len[b] = -1;
      __hip_atomic_store(w.walk + b, pack_walk(0.f, 0, 0, false, false), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  int cur = 0, depth = 0, L = 0;
  while (true) {
    const bool has_q = depth < a.max_depth;
    const int m = w.info[int64_t(b) * n + cur].nchild;
    WorState st{0.f, 1.f, 1.f, false};
    float ak = 0.f, myck = 0.f;
    bool accepted = false;
    if (m > 0) {
      RowStat sts[2];
      wave_merge_two(w.part + (int64_t(b) * rpb + cur) * ns, w.part + (int64_t(b) * rpb + n + depth) * ns, ns, sts);
      const Sib sb = load_sib<T>(a, w, b, cur, m, tree_row<T>(a, b, cur), tree_row<T>(a, b, n + depth), sts[0],
                                 sts[1]);
      float Fr[kRoundBatch];
      wave_sums_published(w.fpart + (int64_t(b) * n + cur) * nc, int64_t(bn_total) * nc, min(m, kRoundBatch), nc,
                          w.err, Fr);
      for (int j = 1; j <= m && !accepted; ++j) {
        const int l = j - 1;
        const int t = __shfl(sb.t, l), ch = __shfl(sb.ch, l), fi = __shfl(sb.fi, l);
        const float pt = __shfl(sb.p, l), qt = __shfl(sb.q, l), u = __shfl(sb.u, l);
        const bool fj = __shfl(sb.first ? 1 : 0, l) != 0;
        const float ck_first = __shfl(myck, fi >= 0 ? fi : 0);
        const float qn = (fj && st.Z > kZEps) ? qt / st.Z : 0.f;
        const float rho = fmaxf(fmaf(-(fj ? st.C : ck_first), qt, pt), 0.f);
        if (t >= 0 && t < a.vocab && u * qn < rho / st.D) {
          if (lane == 0) path_out[L] = ch;
          ++L;
          cur = ch;
          ++depth;
          accepted = true;
        } else {
          float F = 0.f;
          if (!st.frozen) {
            if (j <= kRoundBatch) {
#pragma unroll
              for (int r = 0; r < kRoundBatch; ++r)
                if (r == l) F = Fr[r];
            } else {
              F = wave_sum_published(w.fpart + (int64_t(l) * bn_total + int64_t(b) * n + cur) * nc, nc, w.err);
            }
          }
          const float ck = wor_step(st, sb, j, F, ak);
          if (lane == l) myck = ck;
        }
      }
    }
    if (!accepted) {
      if (lane < m) store_pub(w.ck + int64_t(b) * kMaxWorChildren + lane, myck);
      if (lane == 0) {
        a.out_len[b] = L;
        __hip_atomic_store(w.walk + b, pack_walk(m > 0 ? st.C : 0.f, cur, depth, has_q, true), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      break;
    }
  }
  for (int t = L + lane; t < a.max_depth; t += kWave) path_out[t] = -1;
}

// Thread 0 waits for tree b's walk result; the whole block receives it.
__device__ __forceinline__ uint64_t wait_walk(const TreeWs& w, int b) {
  __shared__ uint64_t sh_word;
  if (threadIdx.x == 0) {
    uint64_t v = kWalkUnset;
    for (int it = 0;; ++it) {
      v = __hip_atomic_load(w.walk + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (v != kWalkUnset) break;
      if (it == kSpinMax) {
        atomicOr(w.err, 1);
        v = 0;   // inactive
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    sh_word = v;
  }
  __syncthreads();
  const uint64_t v = sh_word;
  __syncthreads();
  return v;
}

// Segment masses of chunk c of tree b's draw (as draw_seg_body sums them).
template <typename T>
__device__ void seg_item(const TreeVerifyArgs& a, const TreeWs& w, int b, int c) {
  const uint64_t word = wait_walk(w, b);
  if (!((word >> 55) & 1)) return;   // no draw: the search item does not read the masses
  const DrawDesc d = walk_desc<T>(a, w, b, word);
  const int nc = num_chunks(a.vocab);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const bool vp = row_vec_ok(static_cast<const T*>(d.prow)), vq = row_vec_ok(static_cast<const T*>(d.qrow));
  float* dst = w.seg + (int64_t(b) * nc + c) * (2 * kSegPerChunk);
  // without replacement: the removed tokens' weights (every wave its own copy)
  int wm = 0;
  float repl = 0.f;
  Sib sb{-1, -1, -1, 0.f, 0.f, 1.f, false};
  if (a.wor) {
    const int node = int((word >> 32) & 2047), depth = int((word >> 43) & 2047);
    wm = w.info[int64_t(b) * a.n_tree + node].nchild;
    sb = wor_removed<T>(a, w, b, node, depth, repl);
  }
#pragma unroll
  for (int q = 0; q < kSegPerWave; ++q) {
    const int k = wave * kSegPerWave + q;
    const int e0 = c * kChunk + k * kSegLen + lane * 8;
    float wv[8], pw[8];
    weights8<T, false>(d, e0, a.vocab, a.scale_log2, vp, vq, wv, pw);
    if (wm > 0) wor_patch(wv, e0, sb, repl, wm);
    float sw = 0.f, sp = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sw += wv[e];
      sp += pw[e];
    }
    const float tw = wave_sum(sw), tp = wave_sum(sp);
    if (lane == 0) {
      store_pub(dst + k, tw);
      store_pub(dst + kSegPerChunk + k, tp);
    }
  }
}

// The inverse-CDF search of tree b's draw (one whole wave): the segment
// masses in token order, the segment holding u * S, then the element within
// it (the same steps as draw_resolve_body, on published masses).
template <typename T>
__device__ void resolve_item(const TreeVerifyArgs& a, const TreeWs& w, int b, uint64_t word) {
  const int lane = threadIdx.x & (kWave - 1);
  if (!((word >> 55) & 1)) {
    if (lane == 0) a.out_tok[b] = -1;
    return;
  }
  DrawDesc d = walk_desc<T>(a, w, b, word);
  const int nc = num_chunks(a.vocab);
  const int nseg = nc * kSegPerChunk;
  int wm = 0;
  float repl = 0.f;
  Sib sb{-1, -1, -1, 0.f, 0.f, 1.f, false};
  if (a.wor) {
    const int node = int((word >> 32) & 2047), depth = int((word >> 43) & 2047);
    wm = w.info[int64_t(b) * a.n_tree + node].nchild;
    sb = wor_removed<T>(a, w, b, node, depth, repl);
  }
  const float* base = w.seg + int64_t(b) * nc * (2 * kSegPerChunk);
  auto segaddr = [&](int i, int which) {
    return base + (i / kSegPerChunk) * (2 * kSegPerChunk) + which * kSegPerChunk + (i % kSegPerChunk);
  };
  const int ngroup = (nseg + kWave - 1) / kWave;
  // wait until every mass of w and of p is published (lane l: segments l + 64 t)
  for (int it = 0;; ++it) {
    bool missing = false;
    for (int t = 0; t < ngroup; ++t) {
      const int i = t * kWave + lane;
      if (i < nseg) missing |= load_pub(segaddr(i, 0)) < 0.f || load_pub(segaddr(i, 1)) < 0.f;
    }
    if (!wave_ballot(missing)) break;
    if (it == kSpinMax) {
      if (lane == 0) atomicOr(w.err, 1);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  // S: the inclusive scan of the masses in token order, group by group
  auto total_of = [&](int which) {
    float carry = 0.f;
    for (int t = 0; t < ngroup; ++t) {
      const int i = t * kWave + lane;
      const float v = i < nseg ? load_pub(segaddr(i, which)) : 0.f;
      carry += __shfl(wave_inclusive_scan(v), kWave - 1);
    }
    return carry;
  };
  int which = 0;
  float S = total_of(0);
  if (!(S > 0.f)) {   // residual without mass: draw from p instead
    d.c = 0.f;
    which = 1;
    S = total_of(1);
  }
  const float target = a.u_s[b] * S;
  // first segment whose inclusive prefix exceeds the target, else the last
  // segment with mass (the same scan, repeated)
  int hit_seg = -1, last_pos = -1;
  float carry_before = 0.f;
  {
    float carry = 0.f;
    for (int t = 0; t < ngroup && hit_seg < 0; ++t) {
      const int c0 = t * kWave;
      const bool valid = c0 + lane < nseg;
      const float v = valid ? load_pub(segaddr(c0 + lane, which)) : 0.f;
      const float incl = wave_inclusive_scan(v) + carry;
      carry = __shfl(incl, kWave - 1);
      const uint64_t hit = wave_ballot(valid && incl > target);
      const uint64_t pos = wave_ballot(valid && v > 0.f);
      if (hit) {
        const int l = int(__builtin_ctzll(hit));
        hit_seg = c0 + l;
        carry_before = __shfl(incl - v, l);
      } else if (pos) {
        const int l = 63 - int(__builtin_clzll(pos));
        last_pos = c0 + l;
        carry_before = __shfl(incl - v, l);
      }
    }
  }
  const bool by_target = hit_seg >= 0;
  const int sidx = by_target ? hit_seg : last_pos;
  int y = 0;
  if (sidx >= 0) {
    const int e0 = (sidx / kSegPerChunk) * kChunk + (sidx % kSegPerChunk) * kSegLen + lane * 8;
    float wv[8], pw[8];
    weights8<T, false>(d, e0, a.vocab, a.scale_log2, row_vec_ok(static_cast<const T*>(d.prow)),
                row_vec_ok(static_cast<const T*>(d.qrow)), wv, pw);
    if (wm > 0 && which == 0) wor_patch(wv, e0, sb, repl, wm);
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ls += wv[j];
    const float inc = wave_inclusive_scan(ls);
    const uint64_t hit = wave_ballot(by_target && carry_before + inc > target);
    const uint64_t pos = wave_ballot(ls > 0.f);
    int sel;
    bool tgt;
    if (hit) {
      sel = int(__builtin_ctzll(hit));
      tgt = true;
    } else {
      sel = pos ? 63 - int(__builtin_clzll(pos)) : 0;
      tgt = false;
    }
    if (lane == sel) {
      float cum = carry_before + inc - ls;
      int pick = -1, lastp = -1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        cum += wv[j];
        if (wv[j] > 0.f) lastp = j;
        if (tgt && pick < 0 && cum > target) pick = j;
      }
      if (pick < 0) pick = (lastp >= 0) ? lastp : 0;
      y = e0 + pick;
    }
    y = __shfl(y, sel);
  }
  if (lane == 0) a.out_tok[b] = y;
}

// The flow launch: items in increasing order from the work counter.
template <typename T>
__global__ __launch_bounds__(kChunkThreads) void tree_flow_kernel(TreeVerifyArgs a, TreeWs w) {
  const int n = a.n_tree, nc = num_chunks(a.vocab);
  // round items: for trees whose node lists are indexed (batch <= kMaxListTrees),
  // only the nodes with children; else every node
  __shared__ int sh_pre[kMaxListTrees + 1];
  const bool listed = a.batch <= kMaxListTrees;
  int per_round;
  if (listed) {
    if (threadIdx.x < kWave) {
      int carry = 0;
      for (int base = 0; base < a.batch; base += kWave) {
        const int b = base + threadIdx.x;
        const int v = b < a.batch ? w.cnt[b] : 0;
        const float incl = wave_inclusive_scan(float(v));   // exact: counts < 2^24
        if (b < a.batch) sh_pre[b + 1] = carry + int(incl);
        carry += int(__shfl(incl, kWave - 1));
      }
      if (threadIdx.x == 0) sh_pre[0] = 0;
    }
    __syncthreads();
    per_round = sh_pre[a.batch] * nc;
  } else {
    per_round = a.batch * n * nc;
  }
  const int n_gather = per_round / nc;   // one per (listed) node
  const int n_round = n_gather + a.max_children * per_round;
  const int n_walk = n_round + a.batch;
  const int n_seg = n_walk + a.batch * nc;
  const int total = n_seg + a.batch;
  __shared__ int sh_item;
  while (true) {
    if (threadIdx.x == 0) sh_item = atomicAdd(w.queue, 1);
    __syncthreads();
    const int it = sh_item;
    __syncthreads();
    if (it >= total) break;
    if (it < n_round) {
      const bool gather = it < n_gather;
      const int r_it = it - n_gather;
      const int j = gather ? 0 : r_it / per_round + 1, rem = gather ? it * nc : r_it % per_round;
      const int slot = rem / nc;
      int node_idx = slot;
      if (listed) {   // slot -> (tree, position in its list): the last tree with sh_pre[b] <= slot
        int lo = 0, hi = a.batch - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) / 2;
          if (sh_pre[mid] <= slot) lo = mid; else hi = mid - 1;
        }
        node_idx = lo * n + w.list[int64_t(lo) * n + (slot - sh_pre[lo])];
      }
      if (gather) {
        if (threadIdx.x < kWave) gather_item<T>(a, w, node_idx);
      } else {
        round_item<T>(a, w, j, node_idx, rem % nc);
      }
    } else if (it < n_walk) {
      if (threadIdx.x < kWave) {
        if (a.wor)
          walk_item_wor<T>(a, w, it - n_round);
        else
          walk_item<T>(a, w, it - n_round);
      }
    } else if (it < n_seg) {
      const int r = it - n_walk;
      seg_item<T>(a, w, r / nc, r % nc);
    } else {
      const int b = it - n_seg;
      const uint64_t word = wait_walk(w, b);
      if (threadIdx.x < kWave) resolve_item<T>(a, w, b, word);
    }
    __syncthreads();   // the item's LDS is reused by the next one
  }
}

template <typename T>
hipError_t launch_tree(const TreeVerifyArgs& a, hipStream_t stream) {
  TreeWs w = tree_ws(a.ws, a.batch, a.n_tree, a.max_depth, a.max_children, a.vocab, a.wor);
  const int ns = tree_stat_splits(a.batch, a.n_tree, a.max_depth, a.vocab);
  const int nc = num_chunks(a.vocab);
  const int nstat = a.batch * (a.n_tree + a.max_depth) * ns;
  const int64_t init = int64_t(a.max_children) * a.batch * a.n_tree * nc + int64_t(a.batch) * nc * 2 * kSegPerChunk +
                       a.batch + (a.wor ? int64_t(a.batch) * kMaxWorChildren : 0) + int64_t(a.batch) * a.n_tree;
  const int ninit = int(std::min<int64_t>(64, (init + kChunkThreads - 1) / kChunkThreads));
  {
    ProfileScope ps("uno_tree_stats", stream);
    hipLaunchKernelGGL(tree_stats_kernel<T>, dim3(unsigned(nstat + a.batch + ninit)), dim3(kChunkThreads), 0,
                       stream, a, w, nstat, ninit);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // enough blocks for the widest step of the flow (a round's chunks), up to
  // a few per compute unit; the item order makes any count finish
  const int64_t widest = std::max<int64_t>(int64_t(a.batch) * a.n_tree * nc, int64_t(a.batch) * nc);
  const int blocks = int(std::min<int64_t>(widest, 2048));
  ProfileScope ps("uno_tree_flow", stream);
  hipLaunchKernelGGL(tree_flow_kernel<T>, dim3(unsigned(blocks)), dim3(kChunkThreads), 0, stream, a, w);
  return hipGetLastError();
}

}  // namespace

size_t tree_verify_workspace_bytes(int batch, int n, int dmax, int maxc, int vocab, int wor) {
  const int nc = num_chunks(vocab);
  const int ns = tree_stat_splits(batch, n, dmax, vocab);
  size_t bytes = align_up(size_t(batch) * n * sizeof(NodeInfo), 256) + align_up(size_t(batch) * sizeof(int), 256) +
                 align_up(size_t(batch) * (n + dmax) * ns * sizeof(float2), 256) +
                 align_up(size_t(maxc > 0 ? maxc : 1) * batch * n * nc * sizeof(float), 256) +
                 align_up(size_t(batch) * sizeof(uint64_t), 256) + draw_seg_bytes(batch, vocab) + 256 +
                 align_up(size_t(batch) * sizeof(int), 256) + align_up(size_t(batch) * n * sizeof(int), 256) +
                 align_up(size_t(batch) * n * sizeof(uint64_t), 256);
  if (wor)
    bytes += align_up(size_t(batch) * n * (maxc > 0 ? maxc : 1) * sizeof(int), 256) +
             align_up(size_t(batch) * kMaxWorChildren * sizeof(float), 256);
  return bytes;
}

hipError_t launch_tree_verify(const TreeVerifyArgs& a, hipStream_t stream) {
  return a.dtype == UNO_BF16 ? launch_tree<uint16_t>(a, stream) : launch_tree<float>(a, stream);
}

}  // namespace uno
