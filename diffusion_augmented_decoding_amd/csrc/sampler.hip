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

// ---------------------------------------------------------------- sampling transforms
// The verify under a sampling transform (top-k, top-p, greedy): every p and q
// row is replaced by its transformed distribution, then the same accept,
// residual and draw rules run on those.  Four launches:
//  1. lin_cut: one 1024-thread block per row finds, exactly, the smallest
//     logit key the transform keeps (integer counts for top-k, 2^-40
//     fixed-point masses for top-p, so the result does not depend on the
//     order of the additions): top-k among the candidate keys gathered above
//     the k-th largest of the threads' own maxima, top-p by radix levels of
//     LDS histograms; the kept mass from the same exact sums; the row's
//     maximum and its first argmax (greedy) and the draft's logit;
//  2. lin_accept_cut: the accept tests on the transformed probabilities;
//  3-4. the draw kernels with the transform applied to both rows.
struct RowCut {
  float m;          // max_v y_v (y = logit log2(e) / T)
  float s;          // sum over kept v of 2^(y_v - m); 1 for greedy
  uint32_t tau;     // smallest kept logit key
  int argmax;       // greedy: the row's first argmax; -1 otherwise
};

struct CutWs {
  RowCut* cut;      // [rows]
  float* xd;        // [rows]
  DrawDesc* desc;   // [batch]
  float* seg;
};

CutWs cut_ws(void* base, int batch, int k, int vocab) {
  const int rows = batch * (2 * k + 1);
  char* p = static_cast<char*>(base);
  CutWs w;
  w.cut = reinterpret_cast<RowCut*>(p);
  p += align_up(size_t(rows) * sizeof(RowCut), 256);
  w.xd = reinterpret_cast<float*>(p);
  p += align_up(size_t(rows) * sizeof(float), 256);
  w.desc = reinterpret_cast<DrawDesc*>(p);
  p += align_up(size_t(batch) * sizeof(DrawDesc), 256);
  w.seg = reinterpret_cast<float*>(p);
  (void)vocab;
  return w;
}

struct CutParams {
  int top_k;        // 0: off
  float top_p;      // 1: off
  int greedy;
};

constexpr int kCutThreads = 1024;
constexpr int kCutWaves = kCutThreads / kWave;
constexpr double kMassScale = 1099511627776.0;   // 2^40: fixed-point masses (2^20 tokens of mass <= 1 fit)

// One pass over row elements [0, vocab) by the block: f(index, logit) for
// each, 8 consecutive elements per thread per step (16-byte loads).  Tiles
// of kCutUnroll steps wholly inside an aligned row load their vectors
// together (one memory latency per tile); each thread meets its elements in
// the same order either way.
constexpr int kCutUnroll = 4;
template <typename T, typename F>
__device__ __forceinline__ void cut_pass(const T* row, int vocab, F f) {
  constexpr int kStepE = kCutThreads * 8;
  const bool vec = row_vec_ok(row);
  int t0 = 0;
  if (vec) {
    for (; t0 + kCutUnroll * kStepE <= vocab; t0 += kCutUnroll * kStepE) {
      float x[kCutUnroll][8];
#pragma unroll
      for (int u = 0; u < kCutUnroll; ++u) load8_vec<T, false>(row, t0 + u * kStepE + threadIdx.x * 8, x[u]);
#pragma unroll
      for (int u = 0; u < kCutUnroll; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) f(t0 + u * kStepE + threadIdx.x * 8 + j, x[u][j]);
    }
  }
  for (int e0 = t0 + threadIdx.x * 8; e0 < vocab; e0 += kStepE) {
    float x[8];
    load8<T, false>(row, e0, vocab, vec, x);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (e0 + j < vocab) f(e0 + j, x[j]);
  }
}

// Radix levels over a logit key, from the top: 12 key bits, then the rest.
// bf16 keys vary in their top 16 bits only (12 + 4); fp32 keys take
// 12 + 12 + 8.  A 4096-bin first level spreads a row's elements over many
// bins (an 8-bit first level holds little more than sign and exponent, so
// most of a row lands in a few bins and the histogram atomics serialise).
constexpr int kCutBins = 4096;
constexpr int kMaxCand = 512;   // top-k candidates resolved in LDS (pairwise counts: C^2 / 1024 steps per thread)
__host__ __device__ constexpr int cut_levels(bool half) { return half ? 2 : 3; }
__device__ __forceinline__ int cut_shift(bool half, int lev) { return lev == 0 ? 20 : (half ? 16 : (lev == 1 ? 8 : 0)); }
__device__ __forceinline__ int cut_width(bool half, int lev) { return lev == 0 ? 12 : (half ? 4 : (lev == 1 ? 12 : 8)); }

__device__ __forceinline__ unsigned long long shfl_up_u64(unsigned long long v, int off) {
  const unsigned lo = __shfl_up(unsigned(v), off), hi = __shfl_up(unsigned(v >> 32), off);
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}
__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int off) {
  const unsigned lo = __shfl_xor(unsigned(v), off), hi = __shfl_xor(unsigned(v >> 32), off);
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// Block-wide maximum of a 32-bit value (red: kCutWaves words of LDS); every
// thread gets the result.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t o = __shfl_xor(v, off);
    v = o > v ? o : v;
  }
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint32_t r = red[0];
  for (int q = 1; q < kCutWaves; ++q) r = red[q] > r ? red[q] : r;
  __syncthreads();
  return r;
}

// Block-wide sum of 64-bit integers (exact; red: kCutWaves words); every
// thread gets the result.
__device__ __forceinline__ unsigned long long block_sum_u64(unsigned long long v, unsigned long long* red) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v += shfl_xor_u64(v, off);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  unsigned long long r = 0;
  for (int q = 0; q < kCutWaves; ++q) r += red[q];
  __syncthreads();
  return r;
}

// Radix step over `nb` <= 4 * kCutThreads bins: the first bin, from the top,
// at which the running total (starting from `before`) reaches `target`;
// returns the bin, and in `before` the total of the bins above it.  Thread t
// holds bins nb - 1 - 4t .. nb - 4 - 4t; the sums are exact integers (counts,
// or fixed-point masses), scanned over the block; every thread gets the
// result.  A target above the total (never reached) keeps everything: bin 0.
template <typename U>
__device__ int find_from_top(const U* hist, int nb, double target, unsigned long long& before,
                             unsigned long long* sh_w, int* sh_i) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  unsigned long long c[4], mine = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = nb - 1 - (4 * tid + q);
    c[q] = idx >= 0 ? static_cast<unsigned long long>(hist[idx]) : 0ull;
    mine += c[q];
  }
  unsigned long long incl = mine;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const unsigned long long o = shfl_up_u64(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) sh_w[wave] = incl;
  if (tid == 0) sh_i[0] = kCutThreads;
  __syncthreads();
  unsigned long long above = before;
  for (int q = 0; q < wave; ++q) above += sh_w[q];
  above += incl - mine;   // every bin above this thread's four
  const uint64_t hit = wave_ballot(double(above + mine) >= target);
  if (hit && lane == int(__builtin_ctzll(hit))) atomicMin(&sh_i[0], tid);
  __syncthreads();
  const int first = sh_i[0];
  if (tid == first) {
    unsigned long long run = above;
    int found = 3;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (found == 3 && q < 3 && double(run + c[q]) >= target) {
        found = q;
      } else if (found == 3 && q < 3) {
        run += c[q];
      }
    }
    sh_i[1] = nb - 1 - (4 * tid + found);
    sh_w[kCutWaves] = run;
  } else if (first == kCutThreads && tid == kCutThreads - 1) {
    sh_i[1] = 0;
    sh_w[kCutWaves] = above + mine;   // the block total
  }
  __syncthreads();
  const int bin = sh_i[1];
  before = sh_w[kCutWaves];
  __syncthreads();   // sh_w / sh_i free for the next step
  return bin;
}

// GREEDY: the instantiation for greedy rows (the maximum only, no histograms
// in LDS); the other serves top-k and top-p.  Held to 64 VGPRs (8 waves per
// SIMD): two workgroups per compute unit, so one streams while the other
// reduces (at 72 VGPRs only one fits and the passes run at half speed).
template <typename T, bool GREEDY>
__global__ __launch_bounds__(kCutThreads, 8) void lin_cut_kernel(VerifyLinearArgs a, CutWs w, CutParams cp) {
  __shared__ uint32_t hcnt[kCutBins];
  __shared__ unsigned long long hmass[kCutBins];
  __shared__ uint32_t red_k[kCutWaves];
  __shared__ int red_i[kCutWaves];
  __shared__ float red_f[kCutWaves];
  __shared__ unsigned long long sh_w[kCutWaves + 1];
  __shared__ int sh_i[2];
  __shared__ uint32_t sh_key;
  __shared__ int sh_idx;
  __shared__ int sh_ncand;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int rps = 2 * a.k + 1;
  const int b = row / rps, j = row - b * rps;
  int draft;
  const T* base = lin_row<T>(a, b, j, &draft);
  const int V = a.vocab;
  const float sl2 = a.scale_log2;
  constexpr bool kHalf = sizeof(T) == 2;   // bf16 rows: the low 16 key bits follow from the sign
  constexpr int kLevels = cut_levels(kHalf);
  const bool topk = !GREEDY && cp.top_k > 0 && cp.top_k < V;
  const bool topp = !GREEDY && cp.top_p < 1.f;
  if constexpr (!GREEDY) {
    for (int i = tid; i < kCutBins; i += kCutThreads) {   // only the histograms this call uses
      if (topk) hcnt[i] = 0;
      if (topk || topp) hmass[i] = 0ull;
    }
    __syncthreads();
  }
  // pass A: the largest key and its first index
  uint32_t bk = 0;
  int bi = 0x7fffffff;
  cut_pass<T>(base, V, [&](int v, float x) {
    const uint32_t kk = logit_key(x);
    if (kk > bk || (kk == bk && v < bi)) {
      bk = kk;
      bi = v;
    }
  });
  const uint32_t own_max = bk;   // this thread's largest key (0: no element)
  // block argmax: largest key, then smallest index
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t ok = __shfl_xor(bk, off);
    const int oi = __shfl_xor(bi, off);
    if (ok > bk || (ok == bk && oi < bi)) {
      bk = ok;
      bi = oi;
    }
  }
  if (lane == 0) {
    red_k[wave] = bk;
    red_i[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t k0 = red_k[0];
    int i0 = red_i[0];
    for (int q = 1; q < kCutWaves; ++q)
      if (red_k[q] > k0 || (red_k[q] == k0 && red_i[q] < i0)) {
        k0 = red_k[q];
        i0 = red_i[q];
      }
    sh_key = k0;
    sh_idx = i0;
  }
  __syncthreads();
  const uint32_t maxkey = sh_key;
  const int amax = sh_idx;
  const float m = key_logit(maxkey) * sl2;
  if (tid == 0 && j != a.k)   // rows that score a draft: its logit (-inf for an id outside [0, V))
    w.xd[row] = (draft >= 0 && draft < V) ? load_logit<T>(base, draft) : -INFINITY;
  if constexpr (GREEDY) {
    if (tid == 0) w.cut[row] = RowCut{m, 1.f, maxkey, amax};
    return;
  } else {
  // the key prefix fixed so far and its width; below it every element counts
  uint32_t prefix = 0;
  int fixed_bits = 0;
  auto in_prefix = [&](uint32_t kk) { return fixed_bits == 0 || (kk >> (32 - fixed_bits)) == (prefix >> (32 - fixed_bits)); };
  // a fixed prefix of a bf16 key: the low 16 bits follow from the sign
  auto full_key = [&](uint32_t pre) { return kHalf ? (pre | ((pre & 0x80000000u) ? 0u : 0xffffu)) : pre; };
  uint32_t tau = 0;   // keep all
  auto mass_fx = [&](float x) {   // 2^(y - m) in fixed point (2^-40), truncated
    return (unsigned long long)(double(fast_exp2(fmaf(x, sl2, -m))) * kMassScale);
  };
  // Kept mass in fixed point, taken from the last level of the transform that
  // sets tau (exact integer sums, so independent of the order of additions);
  // without top-k and top-p a pass sums it in fp32 below.
  unsigned long long kept_fx = 0;
  bool have_kept = false;
  // ---- top-k: the k-th largest key.  Fast path (k <= one key per thread):
  // the k-th largest of the threads' own maxima, t0, has at least k keys at
  // or above it (k distinct elements), so the k-th largest key is >= t0; one
  // pass gathers the keys >= t0 into LDS, and when they fit (kMaxCand) the
  // cut (and with top-p the top-p cut too) is resolved among them with exact
  // integer counts and fixed-point masses.  Otherwise (a row with many equal
  // keys at the top) the radix passes over the whole row take over.
  bool topp_done = false;
  if (topk) {
    bool fast = cp.top_k <= kCutThreads;
    if (fast) {
      unsigned long long before = 0;
      for (int lev = 0; lev < kLevels; ++lev) {   // radix select over the threads' maxima
        const int shift = cut_shift(kHalf, lev), width = cut_width(kHalf, lev);
        if (in_prefix(own_max)) atomicAdd(&hcnt[(own_max >> shift) & ((1u << width) - 1u)], 1u);
        __syncthreads();
        const int bin = find_from_top(hcnt, 1 << width, double(cp.top_k), before, sh_w, sh_i);
        prefix |= uint32_t(bin) << shift;
        fixed_bits += width;
        for (int i = tid; i < (1 << width); i += kCutThreads) hcnt[i] = 0;
        __syncthreads();
      }
      const uint32_t t0 = full_key(prefix);
      prefix = 0;
      fixed_bits = 0;
      if (tid == 0) sh_ncand = 0;
      __syncthreads();
      uint32_t* ckey = hcnt;               // candidates: keys >= t0 (first kMaxCand kept)
      unsigned long long* cmass = hmass;   // and their fixed-point masses
      cut_pass<T>(base, V, [&](int, float x) {
        const uint32_t kk = logit_key(x);
        // past kMaxCand + 1 the count no longer matters (the row falls back)
        if (kk >= t0 && *reinterpret_cast<volatile int*>(&sh_ncand) <= kMaxCand) {
          const int slot = atomicAdd(&sh_ncand, 1);
          if (slot < kMaxCand) ckey[slot] = kk;
        }
      });
      __syncthreads();
      const int C = sh_ncand;
      fast = C <= kMaxCand;
      if (fast) {
        for (int i = tid; i < C; i += kCutThreads) cmass[i] = mass_fx(key_logit(ckey[i]));
        __syncthreads();
        // tau: the largest candidate key with at least k candidates at or above it
        uint32_t best = 0;
        for (int i = tid; i < C; i += kCutThreads) {
          const uint32_t ki = ckey[i];
          int ge = 0;
          for (int q = 0; q < C; ++q) ge += ckey[q] >= ki ? 1 : 0;
          if (ge >= cp.top_k && ki > best) best = ki;
        }
        tau = block_max_u32(best, red_k);
        if (topp) {   // top-p among the kept candidates, by the same rule as the radix path
          unsigned long long tot = 0;
          for (int i = tid; i < C; i += kCutThreads)
            if (ckey[i] >= tau) tot += cmass[i];
          const double target = double(cp.top_p) * double(block_sum_u64(tot, sh_w));
          uint32_t low = 0xffffffffu;   // smallest key whose mass strictly above is below target
          for (int i = tid; i < C; i += kCutThreads) {
            const uint32_t ki = ckey[i];
            if (ki < tau) continue;
            unsigned long long above = 0;
            for (int q = 0; q < C; ++q) above += ckey[q] > ki ? cmass[q] : 0ull;
            if (double(above) < target && ki < low) low = ki;
          }
          tau = ~block_max_u32(~low, red_k);
          topp_done = true;
        }
        unsigned long long kept = 0;
        for (int i = tid; i < C; i += kCutThreads)
          if (ckey[i] >= tau) kept += cmass[i];
        kept_fx = block_sum_u64(kept, sh_w);
        have_kept = true;
      } else {   // back to the radix passes: clear the candidate storage
        for (int i = tid; i < kCutBins; i += kCutThreads) {
          hcnt[i] = 0;
          hmass[i] = 0ull;
        }
        __syncthreads();
      }
    }
    if (!fast) {
      // radix over the row; without top-p the last level also gathers the
      // masses: every key above the prefix range fixed so far is kept, and of
      // the keys inside it those from the chosen bin up
      const bool masses = !topp;
      unsigned long long before = 0;
      for (int lev = 0; lev < kLevels; ++lev) {
        const int shift = cut_shift(kHalf, lev), width = cut_width(kHalf, lev);
        const bool last = lev == kLevels - 1;
        const uint32_t mask = (1u << width) - 1u;
        const uint32_t hi = fixed_bits == 0 ? 0xffffffffu : (prefix | ((1u << (32 - fixed_bits)) - 1u));
        unsigned long long above = 0;
        cut_pass<T>(base, V, [&](int, float x) {
          const uint32_t kk = logit_key(x);
          if (in_prefix(kk)) {
            atomicAdd(&hcnt[(kk >> shift) & mask], 1u);
            if (last && masses) atomicAdd(&hmass[(kk >> shift) & mask], mass_fx(x));
          } else if (last && masses && kk > hi) {
            above += mass_fx(x);
          }
        });
        __syncthreads();
        if (last && masses) kept_fx = block_sum_u64(above, sh_w);
        const int bin = find_from_top(hcnt, 1 << width, double(cp.top_k), before, sh_w, sh_i);
        if (last && masses) {
          unsigned long long t = 0;
          for (int i = bin + tid; i < (1 << width); i += kCutThreads) t += hmass[i];
          kept_fx += block_sum_u64(t, sh_w);
          have_kept = true;
        }
        prefix |= uint32_t(bin) << shift;
        fixed_bits += width;
        for (int i = tid; i < (1 << width); i += kCutThreads) hcnt[i] = 0;
        __syncthreads();
      }
      tau = full_key(prefix);
      prefix = 0;
      fixed_bits = 0;
    }
  }
  // ---- top-p on the kept distribution: the smallest key group whose mass
  // above is below top_p of the kept mass, by fixed-point masses; the kept
  // mass is then the mass above the last level's bin plus the bin's own
  if (topp && !topp_done) {
    const uint32_t base_tau = tau;
    unsigned long long before = 0;
    double target = 0.0;
    for (int lev = 0; lev < kLevels; ++lev) {
      const int shift = cut_shift(kHalf, lev), width = cut_width(kHalf, lev);
      const uint32_t mask = (1u << width) - 1u;
      cut_pass<T>(base, V, [&](int, float x) {
        const uint32_t kk = logit_key(x);
        if (kk >= base_tau && in_prefix(kk)) atomicAdd(&hmass[(kk >> shift) & mask], mass_fx(x));
      });
      __syncthreads();
      if (lev == 0) {   // the kept mass in fixed point: the sum of the first level's bins (exact)
        if (wave == 0) {
          unsigned long long t = 0;
          for (int i = lane; i < kCutBins; i += kWave) t += hmass[i];
#pragma unroll
          for (int off = 1; off < kWave; off <<= 1) t += shfl_xor_u64(t, off);
          if (lane == 0) sh_w[kCutWaves] = t;
        }
        __syncthreads();
        target = double(cp.top_p) * double(sh_w[kCutWaves]);
        __syncthreads();
      }
      const int bin = find_from_top(hmass, 1 << width, target, before, sh_w, sh_i);
      if (lev == kLevels - 1) {
        kept_fx = before + hmass[bin];
        have_kept = true;
      }
      prefix |= uint32_t(bin) << shift;
      fixed_bits += width;
      __syncthreads();   // hmass[bin] read by every thread before the clear
      for (int i = tid; i < (1 << width); i += kCutThreads) hmass[i] = 0ull;
      __syncthreads();
    }
    tau = full_key(prefix);
    tau = tau > base_tau ? tau : base_tau;
  }
  if (have_kept) {
    if (tid == 0) w.cut[row] = RowCut{m, float(double(kept_fx) / kMassScale), tau, -1};
    return;
  }
  // kept mass (every key >= tau), each thread in index order, then waves in order
  float acc = 0.f;
  cut_pass<T>(base, V, [&](int, float x) {
    if (logit_key(x) >= tau) acc += fast_exp2(fmaf(x, sl2, -m));
  });
  acc = wave_sum(acc);
  if (lane == 0) red_f[wave] = acc;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int q = 0; q < kCutWaves; ++q) t += red_f[q];
    w.cut[row] = RowCut{m, t, tau, -1};
  }
  }
}

// One wave per sequence: the accept tests on the transformed probabilities.
template <typename T>
__global__ __launch_bounds__(kWave) void lin_accept_cut_kernel(VerifyLinearArgs a, CutWs w) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int k = a.k, rps = 2 * k + 1;
  const int64_t r0 = int64_t(b) * rps;
  const float sl2 = a.scale_log2;
  bool rej = false;
  if (lane < k) {
    const int d = a.drafts[int64_t(b) * a.drafts_seq + lane];
    const RowCut cpp = w.cut[r0 + lane], cq = w.cut[r0 + k + 1 + lane];
    const float xp = w.xd[r0 + lane], xq = w.xd[r0 + k + 1 + lane];
    const float pd = row_prob<true>(xp, d, sl2, cpp.m, 1.f / cpp.s, cpp.tau, cpp.argmax);
    const float qd = row_prob<true>(xq, d, sl2, cq.m, 1.f / cq.s, cq.tau, cq.argmax);
    rej = !(a.u_acc[int64_t(b) * k + lane] * qd < pd);
    if (a.out_pd) a.out_pd[int64_t(b) * k + lane] = pd;
    if (a.out_qd) a.out_qd[int64_t(b) * k + lane] = qd;
  }
  const uint64_t mask = wave_ballot(rej);
  const int L = mask ? int(__builtin_ctzll(mask)) : k;
  if (lane == 0) {
    a.out_len[b] = L;
    const RowCut cpp = w.cut[r0 + L];
    DrawDesc d;
    d.prow = static_cast<const T*>(a.p) + int64_t(b) * a.p_seq + int64_t(L) * a.p_row;
    d.mp = cpp.m;
    d.inv_sp = 1.f / cpp.s;
    d.tp = cpp.tau;
    d.gp = cpp.argmax;
    if (L < k) {
      const RowCut cq = w.cut[r0 + k + 1 + L];
      d.qrow = static_cast<const T*>(a.q) + int64_t(b) * a.q_seq + int64_t(L) * a.q_row;
      d.mq = cq.m;
      d.inv_sq = 1.f / cq.s;
      d.tq = cq.tau;
      d.gq = cq.argmax;
      d.c = 1.f;
    } else {
      d.qrow = d.prow;
      d.mq = 0.f;
      d.inv_sq = 0.f;
      d.tq = 0u;
      d.gq = -1;
      d.c = 0.f;
    }
    d.active = 1;
    w.desc[b] = d;
  }
}

template <typename T>
hipError_t launch_lin_cut(const VerifyLinearArgs& a, const CutParams& cp, hipStream_t stream) {
  const int rows = a.batch * (2 * a.k + 1);
  CutWs w = cut_ws(a.ws, a.batch, a.k, a.vocab);
  {
    ProfileScope ps("uno_row_cut", stream);
    if (cp.greedy)
      hipLaunchKernelGGL((lin_cut_kernel<T, true>), dim3(rows), dim3(kCutThreads), 0, stream, a, w, cp);
    else
      hipLaunchKernelGGL((lin_cut_kernel<T, false>), dim3(rows), dim3(kCutThreads), 0, stream, a, w, cp);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfileScope ps("uno_accept", stream);
    hipLaunchKernelGGL(lin_accept_cut_kernel<T>, dim3(a.batch), dim3(kWave), 0, stream, a, w);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_draw<T, true>(w.desc, a.batch, a.vocab, a.scale_log2, w.seg, a.u_s, a.out_tok, a.out_mass, stream,
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

// ---------------------------------------------------------------- tree construction
// Candidate trees drawn from the per-depth draft marginals: every node at
// depth d gets branching[d] children, breadth first; the children of a
// depth-d node draw their tokens from q row d by inverse CDF, each with its
// own uniform, with replacement (independent draws) or without (sibling j
// draws from q with the tokens of siblings 1..j-1 removed).  The q rows'
// statistics and segment masses come from the row sampler's first kernels
// (one descriptor per q row); then one wave per internal node draws its
// children in order.

// Level offsets of the breadth-first layout: off[d] = first node id at depth d.
__device__ __forceinline__ int level_of(const TreeBuildArgs& a, int v, int& off_d, int& off_next) {
  int off = 0, width = 1;
  for (int d = 0; d <= a.max_depth; ++d) {
    if (v < off + width) {
      off_d = off;
      off_next = off + width;
      return d;
    }
    off += width;
    width *= (d < a.max_depth) ? a.branching[d] : 1;
  }
  off_d = off_next = off;
  return a.max_depth;
}

// One wave per (tree, internal node): the node's children, drawn in order.
// The q row's segment masses sit in registers (lane l holds segments
// l + 64 t); a draw takes their prefix, finds the segment holding u times the
// total and then the token within it.  Without replacement every drawn token
// is zeroed in the element scan and its segment's mass is recomputed from the
// row with all drawn tokens zeroed (the same summation order as the segment
// pass), so the masses the search sees are those of the reduced row.  When no
// mass is left (every token of positive mass drawn) the draw is the smallest
// token id not drawn yet.
template <typename T>
__global__ __launch_bounds__(kWave) void build_draw_kernel(TreeBuildArgs a, SrWs w) {
  __shared__ int ex[kMaxBranch];
  const int b = blockIdx.y, v = blockIdx.x, lane = threadIdx.x;
  int off_d, off_next;
  const int d = level_of(a, v, off_d, off_next);
  const int nb = a.branching[d];
  const int first = off_next + (v - off_d) * nb;
  int32_t* par = a.out_parent + int64_t(b) * a.n;
  int32_t* tok = a.out_tokens + int64_t(b) * a.n;
  if (v == 0 && lane == 0) {
    par[0] = -1;
    tok[0] = -1;
  }
  const int row = b * a.max_depth + d;
  const DrawDesc desc = w.desc[row];
  const int vocab = a.vocab;
  const float sl2 = a.scale_log2;
  const int nchunk = num_chunks(vocab), nseg = nchunk * kSegPerChunk;
  const float* base = w.seg + int64_t(row) * nchunk * (2 * kSegPerChunk);
  const bool vp = row_vec_ok(static_cast<const T*>(desc.prow));
  constexpr int kPerLane = kMaxChunks * kSegPerChunk / kWave;
  const int ngroup = (nseg + kWave - 1) / kWave;
  float sv[kPerLane], incl[kPerLane];
#pragma unroll
  for (int t = 0; t < kPerLane; ++t) {
    const int i = t * kWave + lane;
    sv[t] = (i < nseg) ? base[(i / kSegPerChunk) * (2 * kSegPerChunk) + (i % kSegPerChunk)] : 0.f;
  }
  auto drawn = [&](int tkn, int upto) {
    for (int e = 0; e < upto; ++e)
      if (ex[e] == tkn) return true;
    return false;
  };
  for (int j = 0; j < nb; ++j) {
    const int c = first + j;
    const int ne = a.without ? j : 0;
    const float u = a.u[int64_t(b) * a.n + c];
    float carry = 0.f;
#pragma unroll
    for (int t = 0; t < kPerLane; ++t) {
      if (t < ngroup) {
        incl[t] = wave_inclusive_scan(sv[t]) + carry;
        carry = __shfl(incl[t], kWave - 1);
      }
    }
    const float S = carry;
    int y = 0;
    if (!(S > 0.f)) {
      while (drawn(y, ne)) ++y;
    } else {
      const float target = u * S;
      int hit_seg = -1, last_pos = -1;
      float carry_before = 0.f;
#pragma unroll
      for (int t = 0; t < kPerLane; ++t) {
        if (t < ngroup && hit_seg < 0) {
          const int c0 = t * kWave;
          const bool valid = c0 + lane < nseg;
          const uint64_t hit = wave_ballot(valid && incl[t] > target);
          const uint64_t pos = wave_ballot(valid && sv[t] > 0.f);
          if (hit) {
            const int l = int(__builtin_ctzll(hit));
            hit_seg = c0 + l;
            carry_before = __shfl(incl[t] - sv[t], l);
          } else if (pos) {
            const int l = 63 - int(__builtin_clzll(pos));
            last_pos = c0 + l;
            carry_before = __shfl(incl[t] - sv[t], l);
          }
        }
      }
      const bool by_target = hit_seg >= 0;
      const int sidx = by_target ? hit_seg : last_pos;
      const int e0 = (sidx / kSegPerChunk) * kChunk + (sidx % kSegPerChunk) * kSegLen + lane * 8;
      float wv[8], pw[8];
      weights8<T>(desc, e0, vocab, sl2, vp, true, wv, pw);
      float ls = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (ne > 0 && drawn(e0 + k, ne)) wv[k] = 0.f;
        ls += wv[k];
      }
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
        for (int k = 0; k < 8; ++k) {
          cum += wv[k];
          if (wv[k] > 0.f) lastp = k;
          if (tgt && pick < 0 && cum > target) pick = k;
        }
        if (pick < 0) pick = (lastp >= 0) ? lastp : 0;
        y = e0 + pick;
      }
      y = __shfl(y, sel);
    }
    if (lane == 0) {
      par[c] = v;
      tok[c] = y;
      ex[j] = y;
    }
    __syncthreads();
    if (a.without && j + 1 < nb && y < vocab) {
      // the drawn token's segment, recomputed with every drawn token zeroed
      const int sy = (y / kChunk) * kSegPerChunk + (y % kChunk) / kSegLen;
      const int s0 = (sy / kSegPerChunk) * kChunk + (sy % kSegPerChunk) * kSegLen + lane * 8;
      float wv[8], pw[8];
      weights8<T>(desc, s0, vocab, sl2, vp, true, wv, pw);
      float ls = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) ls += drawn(s0 + k, j + 1) ? 0.f : wv[k];
      const float m = wave_sum(ls);
#pragma unroll
      for (int t = 0; t < kPerLane; ++t)
        if (t * kWave + lane == sy) sv[t] = m;
    }
  }
}

template <typename T>
hipError_t launch_build(const TreeBuildArgs& a, hipStream_t stream) {
  // the q rows as a row-sampler call: statistics, descriptors, segment masses
  SampleRowsArgs s{};
  s.dtype = a.dtype;
  s.rows = a.batch * a.max_depth;
  s.vocab = a.vocab;
  s.logits = a.q;
  s.row_stride = a.q_row;
  s.per_seq = a.max_depth;
  s.seq_stride = a.q_seq;
  s.scale_log2 = a.scale_log2;
  SrWs w = sr_ws(a.ws, s.rows, a.vocab);
  const int ns = stats_splits(s.rows, a.vocab);
  {
    ProfileScope ps("uno_build_stats", stream);
    hipLaunchKernelGGL(sr_stats_kernel<T>, dim3(s.rows, ns), dim3(kChunkThreads), 0, stream, s, w);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfileScope ps("uno_build_desc", stream);
    hipLaunchKernelGGL(sr_desc_kernel<T>, dim3(s.rows), dim3(kWave), 0, stream, s, w);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfileScope ps("uno_build_seg", stream);
    hipLaunchKernelGGL((draw_seg_kernel<T, false>), dim3(s.rows, num_chunks(a.vocab)), dim3(kChunkThreads), 0, stream,
                       w.desc, a.vocab, a.scale_log2, w.seg);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  int internal = 0, width = 1;
  for (int d = 0; d < a.max_depth; ++d) {
    internal += width;
    width *= a.branching[d];
  }
  ProfileScope ps("uno_build_draw", stream);
  hipLaunchKernelGGL(build_draw_kernel<T>, dim3(unsigned(internal), unsigned(a.batch)), dim3(kWave), 0, stream, a, w);
  return hipGetLastError();
}

}  // namespace

size_t sample_rows_workspace_bytes(int rows, int vocab) {
  const int ns = stats_splits(rows, vocab);
  return align_up(size_t(rows) * ns * sizeof(float2), 256) + align_up(size_t(rows) * sizeof(DrawDesc), 256) +
         draw_seg_bytes(rows, vocab);
}

size_t tree_build_workspace_bytes(int batch, int max_depth, int vocab) {
  return sample_rows_workspace_bytes(batch * max_depth, vocab);
}

hipError_t launch_tree_build(const TreeBuildArgs& a, hipStream_t stream) {
  return a.dtype == UNO_BF16 ? launch_build<uint16_t>(a, stream) : launch_build<float>(a, stream);
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

size_t verify_linear_sampled_workspace_bytes(int batch, int k, int vocab) {
  const int rows = batch * (2 * k + 1);
  return align_up(size_t(rows) * sizeof(RowCut), 256) + align_up(size_t(rows) * sizeof(float), 256) +
         align_up(size_t(batch) * sizeof(DrawDesc), 256) + draw_seg_bytes(batch, vocab);
}

hipError_t launch_verify_linear_sampled(const VerifyLinearArgs& a, int top_k, float top_p, int greedy,
                                        hipStream_t stream) {
  const CutParams cp{top_k, top_p, greedy};
  return a.dtype == UNO_BF16 ? launch_lin_cut<uint16_t>(a, cp, stream) : launch_lin_cut<float>(a, cp, stream);
}

}  // namespace uno
