// Psi-Spec linear verify with early exit, for gfx950.
//
// Method: Uno summary (hyper.ai, arXiv 2609.04010), section "方法", last
// paragraph -- rejection sampling of a drafted block against the AR
// distribution, longest accepted prefix, correction from the residual
// (standard speculative sampling, Leviathan et al. 2023).  Drafts are tested
// in order and the first rejection ends the block, so the rows of positions
// after it never influence the result; this variant skips most of them.
//
// Positions 0..k are taken in rounds of 2, 2, 4, then 8 positions (short
// rounds first: most blocks end early when the draft is poor, and a round
// costs a launch gap and a tail).  Per round, two launches:
//  1. stats: one workgroup per (sequence, row of the round, split) -- rows
//     p_i for the round's positions i <= k and q_i for i < k -- computing
//     the softmax partial of the full verify (same splits, same loads), or
//     returning at once when the sequence's block has already ended;
//  2. accept: one workgroup per sequence still live merges its round's
//     partials exactly as the full verify merges every row and tests the
//     round's drafts in order; at the first rejection (or at i = k) it writes
//     the accepted length and the draw descriptor and marks the sequence
//     ended.
// Then the draw kernels of the full verify.  Accepted length, token, residual
// mass and the probabilities of the evaluated drafts are those of the full
// verify bit for bit.  A sequence reads at most 7 positions past its first
// rejection (fewer in the early rounds), and nothing in the rounds after it.
#include <algorithm>

#include "sampler_common.h"

namespace uno {

namespace {

constexpr int kMaxRound = 8;   // positions per round, at most

// Positions per round r: 2, 2, 4, then 8.
inline int round_size(int r) { return r < 2 ? 2 : (r == 2 ? 4 : kMaxRound); }

struct EeWs {
  float2* part;     // [batch (2k + 1)][nsplit], the full verify's row order
  float* xd;        // [batch (2k + 1)] draft logit
  int* live;        // [batch]: 1 while the sequence's block goes on
  DrawDesc* desc;   // [batch]
  float* seg;
};

EeWs ee_ws(void* base, int batch, int k, int vocab) {
  const int rows = batch * (2 * k + 1);
  const int nc = stats_splits(rows, vocab);
  char* p = static_cast<char*>(base);
  EeWs w;
  w.part = reinterpret_cast<float2*>(p);
  p += align_up(size_t(rows) * nc * sizeof(float2), 256);
  w.xd = reinterpret_cast<float*>(p);
  p += align_up(size_t(rows) * sizeof(float), 256);
  w.live = reinterpret_cast<int*>(p);
  p += align_up(size_t(batch) * sizeof(int), 256);
  w.desc = reinterpret_cast<DrawDesc*>(p);
  p += align_up(size_t(batch) * sizeof(DrawDesc), 256);
  w.seg = reinterpret_cast<float*>(p);
  return w;
}

// Row r of sequence b (r <= k: p row r; else q row r - k - 1) and the draft
// it scores (-1 for the bonus row p_k).
template <typename T>
__device__ __forceinline__ const T* ee_row(const VerifyLinearArgs& a, int b, int r, int* draft) {
  if (r <= a.k) {
    *draft = r < a.k ? a.drafts[int64_t(b) * a.drafts_seq + r] : -1;
    return static_cast<const T*>(a.p) + int64_t(b) * a.p_seq + int64_t(r) * a.p_row;
  }
  *draft = a.drafts[int64_t(b) * a.drafts_seq + (r - a.k - 1)];
  return static_cast<const T*>(a.q) + int64_t(b) * a.q_seq + int64_t(r - a.k - 1) * a.q_row;
}

__global__ __launch_bounds__(kChunkThreads) void ee_init_kernel(int batch, int k, EeWs w, float* out_pd,
                                                                float* out_qd) {
  const int64_t t = int64_t(blockIdx.x) * kChunkThreads + threadIdx.x;
  if (t < batch) {
    w.live[t] = 1;
    w.desc[t].prow = nullptr;
    w.desc[t].qrow = nullptr;
    w.desc[t].active = 0;
  }
  if (t < int64_t(batch) * k) {   // drafts never evaluated stay NaN
    if (out_pd) out_pd[t] = __builtin_nanf("");
    if (out_qd) out_qd[t] = __builtin_nanf("");
  }
}

// Rows of the round [i0, i1): np = i1 - i0 p rows, then nq q rows.
__device__ __forceinline__ int round_q_rows(int i0, int i1, int k) { return max(0, min(i1, k) - i0); }

template <typename T>
__global__ __launch_bounds__(kChunkThreads) void ee_stats_kernel(VerifyLinearArgs a, EeWs w, int i0, int i1) {
  const int np = i1 - i0, per = np + round_q_rows(i0, i1, a.k);
  const int b = blockIdx.x / per, j = blockIdx.x - b * per, c = blockIdx.y;
  if (!w.live[b]) return;   // the sequence's block has ended: nothing to read
  const int nc = gridDim.y;
  const int r = j < np ? i0 + j : a.k + 1 + i0 + (j - np);
  int draft;
  const T* base = ee_row<T>(a, b, r, &draft);
  const int span = split_span(a.vocab, nc);
  const int lo = c * span, hi = min(a.vocab, lo + span);
  const float2 st = range_stats<T>(base, lo, hi, a.scale_log2);
  if (threadIdx.x == 0) {
    const int64_t row = int64_t(b) * (2 * a.k + 1) + r;
    w.part[row * nc + c] = st;
    if (r != a.k) {   // rows that score a draft
      const bool in_range = draft >= 0 && draft < a.vocab;
      if (in_range && draft >= lo && draft < hi) w.xd[row] = load_logit<T>(base, draft);
      if (!in_range && c == 0) w.xd[row] = -INFINITY;   // out-of-range id: probability 0, rejected
    }
  }
}

constexpr int kEeAcceptWaves = 4;

template <typename T>
__global__ __launch_bounds__(kEeAcceptWaves * kWave) void ee_accept_kernel(VerifyLinearArgs a, EeWs w, int i0,
                                                                           int i1) {
  __shared__ float sm[2 * kMaxRound], ss[2 * kMaxRound];
  const int b = blockIdx.x, tid = threadIdx.x;
  if (!w.live[b]) return;   // uniform over the workgroup
  const int k = a.k, rps = 2 * k + 1;
  const int nc = stats_splits(a.batch * rps, a.vocab);
  const float sl2 = a.scale_log2;
  const int np = i1 - i0, nt = min(i1, k) - i0, per = np + max(0, nt);
  const int64_t r0 = int64_t(b) * rps;
  // per-draft inputs of the round, loaded before the merge
  float xp = 0.f, xq = 0.f, u = 0.f;
  if (tid < nt) {
    xp = w.xd[r0 + i0 + tid];
    xq = w.xd[r0 + k + 1 + i0 + tid];
    u = a.u_acc[int64_t(b) * k + i0 + tid];
  }
  // the full verify's merge: a group of gw lanes per row (gw from the
  // sequence's whole row count), lane sub folding splits sub, sub + gw, ...
  // then a butterfly -- so every row's (max, sum) has the same bits
  int gw = 1;
  while (gw < kWave && 2 * gw * rps <= kEeAcceptWaves * kWave) gw *= 2;
  const int rr = tid / gw, sub = tid % gw;
  float m = -INFINITY, s = 0.f;
  if (rr < per) {
    const int r = rr < np ? i0 + rr : k + 1 + i0 + (rr - np);
    const float2* part = w.part + (r0 + r) * nc;
    for (int c = sub; c < nc; c += gw) {
      const float2 v = part[c];
      lse2_merge(m, s, v.x, v.y);
    }
  }
  group_lse2(m, s, gw);
  if (rr < per && sub == 0) {
    sm[rr] = m;
    ss[rr] = s;
  }
  __syncthreads();
  if (tid >= kWave) return;
  // lane j < nt: the accept test of draft i0 + j, as in the full verify
  bool rej = false;
  float pd = 0.f, qd = 0.f;
  if (tid < nt) {
    pd = fast_exp2(fmaf(xp, sl2, -sm[tid])) / ss[tid];
    qd = fast_exp2(fmaf(xq, sl2, -sm[np + tid])) / ss[np + tid];
    rej = !(u * qd < pd);
  }
  const uint64_t mask = wave_ballot(rej);
  const int first = mask ? int(__builtin_ctzll(mask)) : nt;   // round index of the block's end
  if (tid < nt && tid <= first) {   // evaluated drafts; later ones stay NaN
    if (a.out_pd) a.out_pd[int64_t(b) * k + i0 + tid] = pd;
    if (a.out_qd) a.out_qd[int64_t(b) * k + i0 + tid] = qd;
  }
  if (tid != 0 || (!mask && i1 <= k)) return;   // the block goes on into the next round
  const int L = i0 + first;   // first rejection, or k (every draft accepted: the bonus)
  a.out_len[b] = L;
  DrawDesc d;
  d.prow = static_cast<const T*>(a.p) + int64_t(b) * a.p_seq + int64_t(L) * a.p_row;
  d.mp = sm[first];
  d.inv_sp = 1.f / ss[first];
  if (L < k) {
    d.qrow = static_cast<const T*>(a.q) + int64_t(b) * a.q_seq + int64_t(L) * a.q_row;
    d.mq = sm[np + first];
    d.inv_sq = 1.f / ss[np + first];
    d.c = 1.f;
  } else {
    d.qrow = d.prow;
    d.mq = 0.f;
    d.inv_sq = 0.f;
    d.c = 0.f;
  }
  d.active = 1;
  w.desc[b] = d;
  w.live[b] = 0;
}

template <typename T>
hipError_t launch_ee(const VerifyLinearArgs& a, hipStream_t stream) {
  const int k = a.k;
  const int nc = stats_splits(a.batch * (2 * k + 1), a.vocab);
  EeWs w = ee_ws(a.ws, a.batch, k, a.vocab);
  {
    const int64_t n = std::max<int64_t>(a.batch, int64_t(a.batch) * k);
    ProfileScope ps("uno_ee_init", stream);
    hipLaunchKernelGGL(ee_init_kernel, dim3(unsigned((n + kChunkThreads - 1) / kChunkThreads)), dim3(kChunkThreads),
                       0, stream, a.batch, k, w, a.out_pd, a.out_qd);
  }
  hipError_t e = hipGetLastError();
  for (int i0 = 0, r = 0; e == hipSuccess && i0 <= k; i0 += round_size(r++)) {
    const int i1 = std::min(i0 + round_size(r), k + 1);
    const int per = (i1 - i0) + std::max(0, std::min(i1, k) - i0);
    {
      ProfileScope ps("uno_ee_stats", stream);
      hipLaunchKernelGGL(ee_stats_kernel<T>, dim3(unsigned(a.batch * per), unsigned(nc)), dim3(kChunkThreads), 0,
                         stream, a, w, i0, i1);
    }
    e = hipGetLastError();
    if (e != hipSuccess) break;
    {
      ProfileScope ps("uno_ee_accept", stream);
      hipLaunchKernelGGL(ee_accept_kernel<T>, dim3(a.batch), dim3(kEeAcceptWaves * kWave), 0, stream, a, w, i0,
                         i1);
    }
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  return launch_draw<T>(w.desc, a.batch, a.vocab, a.scale_log2, w.seg, a.u_s, a.out_tok, a.out_mass, stream,
                        "uno_draw_seg", "uno_draw_resolve");
}

}  // namespace

size_t verify_linear_ee_workspace_bytes(int batch, int k, int vocab) {
  const int rows = batch * (2 * k + 1);
  const int nc = stats_splits(rows, vocab);
  return align_up(size_t(rows) * nc * sizeof(float2), 256) + align_up(size_t(rows) * sizeof(float), 256) +
         align_up(size_t(batch) * sizeof(int), 256) + align_up(size_t(batch) * sizeof(DrawDesc), 256) +
         draw_seg_bytes(batch, vocab);
}

hipError_t launch_verify_linear_ee(const VerifyLinearArgs& a, hipStream_t stream) {
  return a.dtype == UNO_BF16 ? launch_ee<uint16_t>(a, stream) : launch_ee<float>(a, stream);
}

}  // namespace uno
