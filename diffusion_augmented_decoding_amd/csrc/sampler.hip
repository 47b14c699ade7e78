// Psi-Spec linear verify sampler for gfx950.
//
// Method: Uno summary (hyper.ai, arXiv 2609.04010), section "方法", last
// paragraph -- rejection sampling of a drafted block against the AR
// distribution, longest accepted prefix, correction drawn from the residual
// (standard speculative sampling, Leviathan et al. 2023).
//
// Four launches on the caller's stream:
//  1. stats: one workgroup per (logit row, 8192-element chunk): softmax
//     partials (max, sum of 2^(y - max), y = logit * log2(e) / T) in a single
//     streaming pass with 16-byte non-temporal loads, plus the draft token's
//     logit from the chunk that holds it.  This pass moves ~94% of the
//     sampler's bytes and is HBM-bound.
//  2. accept: one wave per sequence merges each row's chunk partials in a
//     fixed order, evaluates the k accept tests u * q(d) < p(d), finds the
//     first rejection with a ballot, and describes the row pair the
//     correction (or bonus) is drawn from.
//  3. draw_seg: one workgroup per (sequence, chunk): masses of the residual
//     w = max(0, p_L - q_L) (or of p for a bonus) over 512-element segments.
//  4. draw_resolve: one wave per sequence: inverse CDF in token order over the
//     segment masses, then within one re-read segment.
#include "sampler_common.h"

namespace uno {

namespace {

struct LinWs {
  float2* part;     // [rows][nchunk]
  float* xd;        // [rows] draft logit (p rows 0..k-1, q rows)
  DrawDesc* desc;   // [batch]
  float* seg;       // [batch][nchunk][32]
};

LinWs lin_ws(void* base, int batch, int k, int vocab) {
  const int rows = batch * (2 * k + 1);
  const int nc = stats_splits(rows, vocab);
  char* p = static_cast<char*>(base);
  LinWs w;
  w.part = reinterpret_cast<float2*>(p);
  p += align_up(size_t(rows) * nc * sizeof(float2), 256);
  w.xd = reinterpret_cast<float*>(p);
  p += align_up(size_t(rows) * sizeof(float), 256);
  w.desc = reinterpret_cast<DrawDesc*>(p);
  p += align_up(size_t(batch) * sizeof(DrawDesc), 256);
  w.seg = reinterpret_cast<float*>(p);
  return w;
}

// row r of sequence b: j <= k -> p row j, else q row j - k - 1
template <typename T>
__device__ __forceinline__ const T* lin_row(const VerifyLinearArgs& a, int b, int j, int* draft) {
  if (j <= a.k) {
    *draft = (j < a.k) ? a.drafts[int64_t(b) * a.drafts_seq + j] : -1;
    return static_cast<const T*>(a.p) + int64_t(b) * a.p_seq + int64_t(j) * a.p_row;
  }
  const int i = j - a.k - 1;
  *draft = a.drafts[int64_t(b) * a.drafts_seq + i];
  return static_cast<const T*>(a.q) + int64_t(b) * a.q_seq + int64_t(i) * a.q_row;
}

template <typename T>
__global__ __launch_bounds__(kChunkThreads) void lin_stats_kernel(VerifyLinearArgs a, LinWs w) {
  const int row = blockIdx.x, c = blockIdx.y;
  const int nc = gridDim.y;
  const int rps = 2 * a.k + 1;
  const int b = row / rps, j = row - b * rps;
  int draft;
  const T* base = lin_row<T>(a, b, j, &draft);
  const int span = split_span(a.vocab, nc);
  const int lo = c * span, hi = min(a.vocab, lo + span);
  const float2 r = range_stats<T>(base, lo, hi, a.scale_log2);
  if (threadIdx.x == 0) {
    w.part[int64_t(row) * nc + c] = r;
    if (j != a.k) {   // rows that score a draft
      const bool in_range = draft >= 0 && draft < a.vocab;
      if (in_range && draft >= lo && draft < hi) w.xd[row] = load_logit<T>(base, draft);
      if (!in_range && c == 0) w.xd[row] = -INFINITY;   // out-of-range id: probability 0, rejected
    }
  }
}

constexpr int kAcceptWaves = 4;
constexpr int kMaxRows = 2 * 64 + 1;

template <typename T>
__global__ __launch_bounds__(kAcceptWaves * kWave) void lin_accept_kernel(VerifyLinearArgs a, LinWs w) {
  __shared__ float sm[kMaxRows], ss[kMaxRows];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int k = a.k, rps = 2 * k + 1;
  const int nc = stats_splits(a.batch * rps, a.vocab);
  const float sl2 = a.scale_log2;
  const int64_t r0 = int64_t(b) * rps;
  // per-draft inputs, loaded before the merge so their latency overlaps it
  float xp = 0.f, xq = 0.f, u = 0.f;
  if (wave == 0 && lane < k) {
    xp = w.xd[r0 + lane];
    xq = w.xd[r0 + k + 1 + lane];
    u = a.u_acc[int64_t(b) * k + lane];
  }
  // merge every row's split partials: a group of `gw` lanes per row (all rows
  // at once), each lane folding splits sub, sub + gw, ... then a butterfly
  int gw = 1;
  while (gw < kWave && 2 * gw * rps <= kAcceptWaves * kWave) gw *= 2;
  const int r = tid / gw, sub = tid % gw;
  float m = -INFINITY, s = 0.f;
  if (r < rps) {
    const float2* part = w.part + (r0 + r) * nc;
    for (int c = sub; c < nc; c += gw) {
      const float2 v = part[c];
      lse2_merge(m, s, v.x, v.y);
    }
  }
  group_lse2(m, s, gw);
  if (r < rps && sub == 0) {
    sm[r] = m;
    ss[r] = s;
  }
  __syncthreads();
  if (wave != 0) return;
  // lane i < k: accept test of draft i
  bool rej = false;
  if (lane < k) {
    const float pd = fast_exp2(fmaf(xp, sl2, -sm[lane])) / ss[lane];
    const float qd = fast_exp2(fmaf(xq, sl2, -sm[k + 1 + lane])) / ss[k + 1 + lane];
    rej = !(u * qd < pd);
    if (a.out_pd) a.out_pd[int64_t(b) * k + lane] = pd;
    if (a.out_qd) a.out_qd[int64_t(b) * k + lane] = qd;
  }
  const uint64_t mask = wave_ballot(rej);
  const int L = mask ? int(__builtin_ctzll(mask)) : k;
  if (lane == 0) {
    a.out_len[b] = L;
    DrawDesc d;
    d.prow = static_cast<const T*>(a.p) + int64_t(b) * a.p_seq + int64_t(L) * a.p_row;
    d.mp = sm[L];
    d.inv_sp = 1.f / ss[L];
    if (L < k) {
      d.qrow = static_cast<const T*>(a.q) + int64_t(b) * a.q_seq + int64_t(L) * a.q_row;
      d.mq = sm[k + 1 + L];
      d.inv_sq = 1.f / ss[k + 1 + L];
      d.c = 1.f;
    } else {
      d.qrow = d.prow;
      d.mq = 0.f;
      d.inv_sq = 0.f;
      d.c = 0.f;
    }
    d.active = 1;
    w.desc[b] = d;
  }
}

template <typename T>
hipError_t launch_lin(const VerifyLinearArgs& a, hipStream_t stream) {
  const int rows = a.batch * (2 * a.k + 1);
  const int nc = stats_splits(rows, a.vocab);
  LinWs w = lin_ws(a.ws, a.batch, a.k, a.vocab);
  {
    ProfileScope ps("uno_row_stats", stream);
    hipLaunchKernelGGL(lin_stats_kernel<T>, dim3(rows, nc), dim3(kChunkThreads), 0, stream, a, w);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfileScope ps("uno_accept", stream);
    hipLaunchKernelGGL(lin_accept_kernel<T>, dim3(a.batch), dim3(kAcceptWaves * kWave), 0, stream, a, w);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_draw<T>(w.desc, a.batch, a.vocab, a.scale_log2, w.seg, a.u_s, a.out_tok, a.out_mass, stream,
                        "uno_draw_seg", "uno_draw_resolve");
}

// ---------------------------------------------------------------- row sampler
// y[row] = inverse CDF of softmax(logits[row] / T) at u[row], in token order:
// the same statistics pass and two-launch draw as the verify sampler, with
// the draw descriptor set to w = p.
struct SrWs {
  float2* part;     // [rows][splits]
  DrawDesc* desc;   // [rows]
  float* seg;
};

SrWs sr_ws(void* base, int rows, int vocab) {
  const int ns = stats_splits(rows, vocab);
  char* p = static_cast<char*>(base);
  SrWs w;
  w.part = reinterpret_cast<float2*>(p);
  p += align_up(size_t(rows) * ns * sizeof(float2), 256);
  w.desc = reinterpret_cast<DrawDesc*>(p);
  p += align_up(size_t(rows) * sizeof(DrawDesc), 256);
  w.seg = reinterpret_cast<float*>(p);
  return w;
}

// row i of the call: sequence i / per_seq, row i % per_seq of that sequence
template <typename T>
__device__ __forceinline__ const T* sr_row(const SampleRowsArgs& a, int row) {
  const int s = row / a.per_seq, j = row - s * a.per_seq;
  return static_cast<const T*>(a.logits) + int64_t(s) * a.seq_stride + int64_t(j) * a.row_stride;
}

template <typename T>
__global__ __launch_bounds__(kChunkThreads) void sr_stats_kernel(SampleRowsArgs a, SrWs w) {
  const int row = blockIdx.x, c = blockIdx.y, ns = gridDim.y;
  const T* base = sr_row<T>(a, row);
  const int span = split_span(a.vocab, ns);
  const int lo = c * span, hi = min(a.vocab, lo + span);
  const float2 r = range_stats<T>(base, lo, hi, a.scale_log2);
  if (threadIdx.x == 0) w.part[int64_t(row) * ns + c] = r;
}

template <typename T>
__global__ __launch_bounds__(kWave) void sr_desc_kernel(SampleRowsArgs a, SrWs w) {
  const int row = blockIdx.x;
  const int ns = stats_splits(a.rows, a.vocab);
  const RowStat st = wave_merge_chunks(w.part + int64_t(row) * ns, ns);
  if (threadIdx.x == 0) {
    DrawDesc d;
    d.prow = sr_row<T>(a, row);
    d.qrow = d.prow;
    d.mp = st.m;
    d.inv_sp = 1.f / st.s;
    d.mq = 0.f;
    d.inv_sq = 0.f;
    d.c = 0.f;
    d.active = 1;
    w.desc[row] = d;
  }
}

template <typename T>
hipError_t launch_sr(const SampleRowsArgs& a, hipStream_t stream) {
  const int ns = stats_splits(a.rows, a.vocab);
  SrWs w = sr_ws(a.ws, a.rows, a.vocab);
  {
    ProfileScope ps("uno_sample_stats", stream);
    hipLaunchKernelGGL(sr_stats_kernel<T>, dim3(a.rows, ns), dim3(kChunkThreads), 0, stream, a, w);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfileScope ps("uno_sample_desc", stream);
    hipLaunchKernelGGL(sr_desc_kernel<T>, dim3(a.rows), dim3(kWave), 0, stream, a, w);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_draw<T>(w.desc, a.rows, a.vocab, a.scale_log2, w.seg, a.u, a.out_tok, nullptr, stream,
                        "uno_sample_seg", "uno_sample_resolve");
}

}  // namespace

size_t sample_rows_workspace_bytes(int rows, int vocab) {
  const int ns = stats_splits(rows, vocab);
  return align_up(size_t(rows) * ns * sizeof(float2), 256) + align_up(size_t(rows) * sizeof(DrawDesc), 256) +
         draw_seg_bytes(rows, vocab);
}

hipError_t launch_sample_rows(const SampleRowsArgs& a, hipStream_t stream) {
  return a.dtype == UNO_BF16 ? launch_sr<uint16_t>(a, stream) : launch_sr<float>(a, stream);
}

size_t verify_linear_workspace_bytes(int batch, int k, int vocab) {
  const int rows = batch * (2 * k + 1);
  const int nc = stats_splits(rows, vocab);
  return align_up(size_t(rows) * nc * sizeof(float2), 256) + align_up(size_t(rows) * sizeof(float), 256) +
         align_up(size_t(batch) * sizeof(DrawDesc), 256) + draw_seg_bytes(batch, vocab);
}

hipError_t launch_verify_linear(const VerifyLinearArgs& a, hipStream_t stream) {
  return a.dtype == UNO_BF16 ? launch_lin<uint16_t>(a, stream) : launch_lin<float>(a, stream);
}

}  // namespace uno
