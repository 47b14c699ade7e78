// Psi-Spec linear verify sampler for gfx950.
//
// Method: Uno summary (hyper.ai, arXiv 2609.04010), section "方法", last
// paragraph -- rejection sampling of a drafted block against the AR
// distribution, longest accepted prefix, correction drawn from the residual
// (standard speculative sampling, Leviathan et al. 2023).
//
// Two launches on the caller's stream:
//  1. row_stats: one workgroup per logit row (batch * (2k+1) rows).  A single
//     streaming pass computes the row's softmax statistics in the log2 domain
//     (max m, sum s of 2^(y-m), y = logit * log2(e)/T) and gathers the draft
//     token's logit.  This pass moves ~94% of the sampler's bytes and is
//     HBM-bound: 16-byte non-temporal loads, 4 loads in flight per thread,
//     one rescale per 4 vectors.
//  2. accept_residual: one workgroup per sequence.  Wave 0 evaluates the k
//     accept tests u*q(d) < p(d) and finds the first rejection with a ballot;
//     then the workgroup streams the one or two rows the correction is drawn
//     from and resolves the inverse CDF in token order (block_draw).
#include "sampler_common.h"

namespace uno {

namespace {

template <typename T>
__global__ __launch_bounds__(kStatThreads) void row_stats_kernel(VerifyLinearArgs a) {
  const int rps = 2 * a.k + 1;
  const int row = blockIdx.x;
  const int b = row / rps;
  const int j = row - b * rps;
  const T* base;
  int draft = -1;
  if (j <= a.k) {
    base = static_cast<const T*>(a.p) + int64_t(b) * a.p_seq + int64_t(j) * a.p_row;
    if (j < a.k) draft = a.drafts[int64_t(b) * a.k + j];
  } else {
    const int i = j - a.k - 1;
    base = static_cast<const T*>(a.q) + int64_t(b) * a.q_seq + int64_t(i) * a.q_row;
    draft = a.drafts[int64_t(b) * a.k + i];
  }
  row_stats_body<T>(base, a.vocab, a.scale_log2, draft, a.stats + row);
}

template <typename T>
__global__ __launch_bounds__(kDrawThreads) void accept_residual_kernel(VerifyLinearArgs a) {
  __shared__ DrawShared sh;
  __shared__ int sh_L;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int k = a.k;
  const float sl2 = a.scale_log2;
  const RowStat* st = a.stats + int64_t(b) * (2 * k + 1);

  if (wave == 0) {
    bool rej = false;
    if (lane < k) {
      const RowStat sp = st[lane];
      const RowStat sq = st[k + 1 + lane];
      const float pd = fast_exp2(fmaf(sp.yd, sl2, -sp.m)) / sp.s;
      const float qd = fast_exp2(fmaf(sq.yd, sl2, -sq.m)) / sq.s;
      const float u = a.u_acc[int64_t(b) * k + lane];
      rej = !(u * qd < pd);
      if (a.out_pd) a.out_pd[int64_t(b) * k + lane] = pd;
      if (a.out_qd) a.out_qd[int64_t(b) * k + lane] = qd;
    }
    const uint64_t mask = wave_ballot(rej);
    if (lane == 0) sh_L = mask ? int(__builtin_ctzll(mask)) : k;
  }
  __syncthreads();
  const int L = sh_L;

  DrawRows<T> d;
  d.prow = static_cast<const T*>(a.p) + int64_t(b) * a.p_seq + int64_t(L) * a.p_row;
  const RowStat sp = st[L];
  d.mp = sp.m;
  d.inv_sp = 1.f / sp.s;
  if (L < k) {
    d.qrow = static_cast<const T*>(a.q) + int64_t(b) * a.q_seq + int64_t(L) * a.q_row;
    const RowStat sq = st[k + 1 + L];
    d.mq = sq.m;
    d.inv_sq = 1.f / sq.s;
    d.c = 1.f;
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
  if (tid == 0) {
    a.out_len[b] = L;
    a.out_tok[b] = y;
    if (a.out_mass) a.out_mass[b] = mass;
  }
}

}  // namespace

size_t verify_linear_workspace_bytes(int batch, int k) {
  return align_up(size_t(batch) * size_t(2 * k + 1) * sizeof(RowStat), 256);
}

hipError_t launch_verify_linear(const VerifyLinearArgs& a, hipStream_t stream) {
  const int rows = a.batch * (2 * a.k + 1);
  {
    ProfileScope ps("uno_row_stats", stream);
    if (a.dtype == UNO_BF16)
      hipLaunchKernelGGL(row_stats_kernel<uint16_t>, dim3(rows), dim3(kStatThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(row_stats_kernel<float>, dim3(rows), dim3(kStatThreads), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfileScope ps("uno_accept_residual", stream);
    if (a.dtype == UNO_BF16)
      hipLaunchKernelGGL(accept_residual_kernel<uint16_t>, dim3(a.batch), dim3(kDrawThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(accept_residual_kernel<float>, dim3(a.batch), dim3(kDrawThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace uno
