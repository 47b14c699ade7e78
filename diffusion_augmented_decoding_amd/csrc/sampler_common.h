// Device building blocks shared by the Psi-Spec verify samplers (linear and
// tree): chunked softmax statistics of logit rows, and a two-launch,
// chunk-parallel inverse-CDF draw over w_v = max(0, p_v - c q_v) (c > 0) or
// w_v = p_v (c == 0), in token-id order.
//
// Every row pass is split into 8192-element chunks so that a handful of rows
// still spreads over the whole chip; consumers merge the per-chunk partials
// in a fixed order (deterministic results).
#pragma once
#include "device_common.h"
#include "internal.h"

namespace uno {

constexpr int kChunk = 8192;                        // elements per chunk
constexpr int kChunkThreads = 256;                  // threads per chunk workgroup
constexpr int kSegPerChunk = 16;                    // 512-element segments
constexpr int kSegLen = kChunk / kSegPerChunk;
constexpr int kMaxVocab = 1 << 20;
constexpr int kMaxChunks = kMaxVocab / kChunk;      // 128

__host__ __device__ inline int num_chunks(int vocab) { return (vocab + kChunk - 1) / kChunk; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T> __device__ __forceinline__ float load_logit(const T* p, int64_t i);
template <> __device__ __forceinline__ float load_logit<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}
template <> __device__ __forceinline__ float load_logit<float>(const float* p, int64_t i) { return p[i]; }

// 16-byte row load: non-temporal (a row streamed once) or cached (a row the
// caller reads again soon, e.g. the tree verify's rounds).  Rows are device
// memory: the load goes through the global address space (a flat load would
// also count against the scalar-load counter, so waiting for a descriptor
// read would wait for every row load in flight too).
template <bool NT, typename V>
__device__ __forceinline__ V row_load(const V* p) {
  using GV = const __attribute__((address_space(1))) V;
  GV* g = (GV*)(p);
  if constexpr (NT)
    return __builtin_nontemporal_load(g);
  else
    return *g;
}

// Loads 8 consecutive logits starting at e0 (bounds- and alignment-safe;
// elements past `vocab` come back as 0 and must be masked by the caller).
template <typename T, bool NT = true>
__device__ __forceinline__ void load8(const T* row, int e0, int vocab, bool vec_ok, float (&x)[8]) {
  if (vec_ok && e0 + 8 <= vocab) {
    if constexpr (sizeof(T) == 2) {
      const u32x4 v = row_load<NT>(reinterpret_cast<const u32x4*>(row + e0));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = bf16_lo(v[j]);
        x[2 * j + 1] = bf16_hi(v[j]);
      }
    } else {
      const f32x4 v0 = row_load<NT>(reinterpret_cast<const f32x4*>(row + e0));
      const f32x4 v1 = row_load<NT>(reinterpret_cast<const f32x4*>(row + e0 + 4));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = v0[j];
        x[4 + j] = v1[j];
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = (e0 + j < vocab) ? load_logit<T>(row, e0 + j) : 0.f;
  }
}

template <typename T>
__device__ __forceinline__ bool row_vec_ok(const T* row) {
  return (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
}

// Online merge of a group of raw logits x (y = x * sl2) into (m, s).
template <int G>
__device__ __forceinline__ void online_update(float& m, float& s, const float (&x)[G], float sl2) {
  float cmax = x[0];
#pragma unroll
  for (int j = 1; j < G; ++j) cmax = fmaxf(cmax, x[j]);
  const float mn = fmaxf(m, cmax * sl2);
  float acc = s * fast_exp2(m - mn);
#pragma unroll
  for (int j = 0; j < G; ++j) acc += fast_exp2(fmaf(x[j], sl2, -mn));
  m = mn;
  s = acc;
}

// Number of pieces each row's statistics pass is split into: whole rows when
// there are enough rows to fill the chip, else enough pieces for ~2048
// workgroups (each piece a multiple of 8 elements).
__host__ __device__ inline int stats_splits(int rows, int vocab) {
  int s = (2048 + rows - 1) / rows;
  const int maxs = (vocab + 2047) / 2048;
  if (s > maxs) s = maxs;
  return s < 1 ? 1 : s;
}
__host__ __device__ inline int split_span(int vocab, int nsplit) { return ((vocab + nsplit - 1) / nsplit + 7) / 8 * 8; }

// Softmax partial (max y, sum 2^(y - max)) of elements [lo, hi) of one row by
// a kChunkThreads block, returned in thread 0.  Lanes read consecutive
// 16-byte vectors (coalesced); 4 vectors in flight per thread; one rescale
// per 4 vectors.  `lo` is a multiple of 8.
template <typename T, bool NT = true>
__device__ float2 range_stats(const T* row, int lo, int hi, float sl2) {
  constexpr int VN = 16 / sizeof(T);
  constexpr int U = 4;
  const int tid = threadIdx.x;
  float m = -INFINITY, s = 0.f;
  if (row_vec_ok(row)) {
    const int nvec = (hi - lo) / VN;
    const T* base = row + lo;
    int i = tid;
    for (; i + (U - 1) * kChunkThreads < nvec; i += U * kChunkThreads) {
      float x[U * VN];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const T* ptr = base + int64_t(i + u * kChunkThreads) * VN;
        if constexpr (sizeof(T) == 2) {
          const u32x4 v = row_load<NT>(reinterpret_cast<const u32x4*>(ptr));
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x[u * VN + 2 * j] = bf16_lo(v[j]);
            x[u * VN + 2 * j + 1] = bf16_hi(v[j]);
          }
        } else {
          const f32x4 v = row_load<NT>(reinterpret_cast<const f32x4*>(ptr));
#pragma unroll
          for (int j = 0; j < 4; ++j) x[u * VN + j] = v[j];
        }
      }
      online_update<U * VN>(m, s, x, sl2);
    }
    for (; i < nvec; i += kChunkThreads) {
      float x[VN];
      const T* ptr = base + int64_t(i) * VN;
      if constexpr (sizeof(T) == 2) {
        const u32x4 v = row_load<NT>(reinterpret_cast<const u32x4*>(ptr));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[2 * j] = bf16_lo(v[j]);
          x[2 * j + 1] = bf16_hi(v[j]);
        }
      } else {
        const f32x4 v = row_load<NT>(reinterpret_cast<const f32x4*>(ptr));
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = v[j];
      }
      online_update<VN>(m, s, x, sl2);
    }
    const int t = lo + nvec * VN + tid;
    if (t < hi) {
      float x[1] = {load_logit<T>(row, t)};
      online_update<1>(m, s, x, sl2);
    }
  } else {
    for (int t = lo + tid; t < hi; t += kChunkThreads) {
      float x[1] = {load_logit<T>(row, t)};
      online_update<1>(m, s, x, sl2);
    }
  }
  wave_lse2(m, s);
  __shared__ float sm[kChunkThreads / kWave], ss[kChunkThreads / kWave];
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  if (lane == 0) {
    sm[wave] = m;
    ss[wave] = s;
  }
  __syncthreads();
  float2 r = make_float2(-INFINITY, 0.f);
  if (tid == 0) {
    float M = sm[0], S = ss[0];
#pragma unroll
    for (int w = 1; w < kChunkThreads / kWave; ++w) lse2_merge(M, S, sm[w], ss[w]);
    r = make_float2(M, S);
  }
  return r;
}

// Merge of a row's split partials by one whole wave: lane l loads partials
// l, l+64, ... (independent loads, one memory latency), then a butterfly.
// The pairwise merge is symmetric, so every lane ends with the same bits.
__device__ __forceinline__ RowStat wave_merge_chunks(const float2* part, int nchunk) {
  const int lane = threadIdx.x & (kWave - 1);
  float m = -INFINITY, s = 0.f;
  for (int c = lane; c < nchunk; c += kWave) {
    const float2 v = part[c];
    lse2_merge(m, s, v.x, v.y);
  }
  wave_lse2(m, s);
  RowStat r;
  r.m = m;
  r.s = s;
  r.yd = 0.f;
  r.pad = 0.f;
  return r;
}

// Two rows' merges at once (all loads in flight together); each result is
// that of wave_merge_chunks on its row.
__device__ __forceinline__ void wave_merge_two(const float2* part_a, const float2* part_b, int nchunk,
                                               RowStat (&out)[2]) {
  const int lane = threadIdx.x & (kWave - 1);
  float ma = -INFINITY, sa = 0.f, mb = -INFINITY, sb = 0.f;
  for (int c = lane; c < nchunk; c += kWave) {
    const float2 va = part_a[c], vb = part_b[c];
    lse2_merge(ma, sa, va.x, va.y);
    lse2_merge(mb, sb, vb.x, vb.y);
  }
  wave_lse2(ma, sa);
  wave_lse2(mb, sb);
  out[0].m = ma;
  out[0].s = sa;
  out[0].yd = 0.f;
  out[0].pad = 0.f;
  out[1].m = mb;
  out[1].s = sb;
  out[1].yd = 0.f;
  out[1].pad = 0.f;
}

// Sum of n values by one whole wave (same bits in every lane).
__device__ __forceinline__ float wave_sum_range(const float* v, int n) {
  const int lane = threadIdx.x & (kWave - 1);
  float s = 0.f;
  for (int c = lane; c < n; c += kWave) s += v[c];
  return wave_sum(s);
}

// What a draw is taken from (filled by the accept / walk kernels).
struct DrawDesc {
  const void* prow;
  const void* qrow;
  float mp, inv_sp, mq, inv_sq;
  float c;          // 0: w = p; > 0: w = max(0, p - c q)
  int active;       // 0: no draw (token written as -1)
  // sampling transform (read by the CUT draw kernels only): tokens whose
  // logit key is below tp (tq) have probability 0 under p (q); gp (gq) >= 0:
  // the row is one-hot at that token (greedy)
  uint32_t tp, tq;
  int gp, gq;
};

// Order-preserving key of a logit: a < b as floats iff key(a) < key(b) as
// unsigned integers (finite values and -inf).  A bf16 value's key has its
// low 16 bits all 0 (positive) or all 1 (negative).
__device__ __forceinline__ uint32_t logit_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Probability of token v with logit x under a row (m, 1/s) and its
// transform (keys below `cut` out; one-hot at g >= 0).
template <bool CUT>
__device__ __forceinline__ float row_prob(float x, int v, float sl2, float m, float inv_s, uint32_t cut, int g) {
  if constexpr (CUT) {
    if (g >= 0) return v == g ? 1.f : 0.f;
    return logit_key(x) >= cut ? fast_exp2(fmaf(x, sl2, -m)) * inv_s : 0.f;
  } else {
    return fast_exp2(fmaf(x, sl2, -m)) * inv_s;
  }
}

// w of 8 elements (and p alone, for the fallback when w has no mass).
template <typename T, bool NT = true, bool CUT = false>
__device__ __forceinline__ void weights8(const DrawDesc& d, int e0, int vocab, float sl2, bool vp, bool vq,
                                         float (&w)[8], float (&pw)[8]) {
  float xp[8];
  load8<T, NT>(static_cast<const T*>(d.prow), e0, vocab, vp, xp);
  float xq[8];
  if (d.c != 0.f) load8<T, NT>(static_cast<const T*>(d.qrow), e0, vocab, vq, xq);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bool in = e0 + j < vocab;
    const float p = row_prob<CUT>(xp[j], e0 + j, sl2, d.mp, d.inv_sp, d.tp, d.gp);
    pw[j] = in ? p : 0.f;
    if (d.c != 0.f) {
      const float q = row_prob<CUT>(xq[j], e0 + j, sl2, d.mq, d.inv_sq, d.tq, d.gq);
      w[j] = in ? fmaxf(fmaf(-d.c, q, p), 0.f) : 0.f;
    } else {
      w[j] = pw[j];
    }
  }
}

// 8 logits from a 16-byte aligned row, every element in range.
template <typename T, bool NT>
__device__ __forceinline__ void load8_vec(const T* row, int e0, float (&x)[8]) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 v = row_load<NT>(reinterpret_cast<const u32x4*>(row + e0));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = bf16_lo(v[j]);
      x[2 * j + 1] = bf16_hi(v[j]);
    }
  } else {
    const f32x4 v0 = row_load<NT>(reinterpret_cast<const f32x4*>(row + e0));
    const f32x4 v1 = row_load<NT>(reinterpret_cast<const f32x4*>(row + e0 + 4));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = v0[j];
      x[4 + j] = v1[j];
    }
  }
}

constexpr int kSegPerWave = kSegPerChunk / (kChunkThreads / kWave);   // 4

// Segment sums of a chunk that lies wholly inside the row, rows 16-byte
// aligned: every load issued before the first use (one memory latency per
// thread, not one per segment).  The arithmetic is weights8's for elements
// in range, so the sums have the same bits as on the general path.
template <typename T, bool CUT, bool HASQ>
__device__ __forceinline__ void seg_sums_full(const DrawDesc& d, int ebase, float sl2, float (&sw)[kSegPerWave],
                                              float (&sp)[kSegPerWave]) {
  float xp[kSegPerWave][8], xq[kSegPerWave][8];
#pragma unroll
  for (int q = 0; q < kSegPerWave; ++q) {   // q rows first: the two variants share no leading load to hoist
    if constexpr (HASQ) load8_vec<T, true>(static_cast<const T*>(d.qrow), ebase + q * kSegLen, xq[q]);
    load8_vec<T, true>(static_cast<const T*>(d.prow), ebase + q * kSegLen, xp[q]);
  }
#pragma unroll
  for (int q = 0; q < kSegPerWave; ++q) {
    sw[q] = 0.f;
    sp[q] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int v = ebase + q * kSegLen + j;
      const float p = row_prob<CUT>(xp[q][j], v, sl2, d.mp, d.inv_sp, d.tp, d.gp);
      float w = p;
      if constexpr (HASQ) w = fmaxf(fmaf(-d.c, row_prob<CUT>(xq[q][j], v, sl2, d.mq, d.inv_sq, d.tq, d.gq), p), 0.f);
      sw[q] += w;
      sp[q] += p;
    }
  }
}

// Segment masses of chunk c of draw b: seg[(b * nchunk + c) * 2*kSegPerChunk + k]
// for the 16 segments of w, then the 16 of p.  A block of kChunkThreads threads.
template <typename T, bool CUT = false>
__device__ __forceinline__ void draw_seg_body(const DrawDesc* __restrict__ desc, int vocab, float sl2,
                                              float* __restrict__ seg, int b, int c, int nchunk) {
  const DrawDesc d = desc[b];
  if (!d.active) return;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const bool vp = row_vec_ok(static_cast<const T*>(d.prow));
  const bool vq = row_vec_ok(static_cast<const T*>(d.qrow));
  float sw[kSegPerWave], sp[kSegPerWave];
  // wave w owns segments 4w..4w+3; lane l reads elements [8l, 8l+8) of each
  const int ebase = c * kChunk + wave * kSegPerWave * kSegLen + lane * 8;
  if (vp && vq && (c + 1) * kChunk <= vocab) {   // uniform over the workgroup
    if (d.c != 0.f)
      seg_sums_full<T, CUT, true>(d, ebase, sl2, sw, sp);
    else
      seg_sums_full<T, CUT, false>(d, ebase, sl2, sw, sp);
  } else {
#pragma unroll
    for (int q = 0; q < kSegPerWave; ++q) {
      float w[8], pw[8];
      weights8<T, true, CUT>(d, ebase + q * kSegLen, vocab, sl2, vp, vq, w, pw);
      sw[q] = 0.f;
      sp[q] = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        sw[q] += w[j];
        sp[q] += pw[j];
      }
    }
  }
  float* dst = seg + (int64_t(b) * nchunk + c) * (2 * kSegPerChunk);
#pragma unroll
  for (int q = 0; q < kSegPerWave; ++q) {
    const float a = wave_sum(sw[q]), bsum = wave_sum(sp[q]);
    if (lane == 0) {
      dst[wave * kSegPerWave + q] = a;
      dst[kSegPerChunk + wave * kSegPerWave + q] = bsum;
    }
  }
}

// Grid (batch, nchunk), 256 threads.
template <typename T, bool CUT = false>
__global__ __launch_bounds__(kChunkThreads) void draw_seg_kernel(const DrawDesc* __restrict__ desc, int vocab,
                                                                 float sl2, float* __restrict__ seg) {
  draw_seg_body<T, CUT>(desc, vocab, sl2, seg, blockIdx.x, blockIdx.y, gridDim.y);
}

// Resolve the inverse CDF for one batch element (one wave): S = sum of the
// segment masses in token order, target = u * S, the segment holding it, then
// the element within the segment (re-reads 512 elements).  Falls back to p
// when w has no mass.  y = -1 when the descriptor is inactive.  Called by
// one whole wave (the first of its block).
template <typename T, bool CUT = false>
__device__ __forceinline__ void draw_resolve_body(const DrawDesc* __restrict__ desc, int vocab, float sl2,
                                                  const float* __restrict__ seg, const float* __restrict__ u_s,
                                                  int32_t* __restrict__ out_tok, float* __restrict__ out_mass,
                                                  int b) {
  const int lane = threadIdx.x & (kWave - 1);
  DrawDesc d = desc[b];
  if (!d.active) {
    if (lane == 0) {
      out_tok[b] = -1;
      if (out_mass) out_mass[b] = 0.f;
    }
    return;
  }
  const int nchunk = num_chunks(vocab);
  const int nseg = nchunk * kSegPerChunk;
  const float* base = seg + int64_t(b) * nchunk * (2 * kSegPerChunk);
  auto segval = [&](int i, int which) {   // which: 0 = w, 1 = p
    return base[(i / kSegPerChunk) * (2 * kSegPerChunk) + which * kSegPerChunk + (i % kSegPerChunk)];
  };
  // lane l owns segments l + 64 t; all loads issued before any use.  The
  // unrolled groups are guarded by a wave-uniform bound (static register
  // indices, no work past the last segment).
  constexpr int kPerLane = kMaxChunks * kSegPerChunk / kWave;
  const int ngroup = (nseg + kWave - 1) / kWave;
  const float u = u_s[b];
  float v[kPerLane], incl[kPerLane];
#pragma unroll
  for (int t = 0; t < kPerLane; ++t) v[t] = (t * kWave + lane < nseg) ? segval(t * kWave + lane, 0) : 0.f;
  // inclusive prefix of the segment masses in token order; S is its last value
  auto prefix = [&]() {
    float carry = 0.f;
#pragma unroll
    for (int t = 0; t < kPerLane; ++t) {
      if (t < ngroup) {
        incl[t] = wave_inclusive_scan(v[t]) + carry;
        carry = __shfl(incl[t], kWave - 1);
      }
    }
    return carry;
  };
  float S = prefix();
  if (!(S > 0.f)) {   // residual without mass: draw from p instead
    d.c = 0.f;
#pragma unroll
    for (int t = 0; t < kPerLane; ++t) v[t] = (t * kWave + lane < nseg) ? segval(t * kWave + lane, 1) : 0.f;
    S = prefix();
  }
  const float target = u * S;
  // first segment whose inclusive prefix exceeds the target, else the last
  // segment with mass
  int hit_seg = -1, last_pos = -1;
  float carry_before = 0.f;
#pragma unroll
  for (int t = 0; t < kPerLane; ++t) {
    if (t < ngroup && hit_seg < 0) {
      const int c0 = t * kWave;
      const bool valid = c0 + lane < nseg;
      const uint64_t hit = wave_ballot(valid && incl[t] > target);
      const uint64_t pos = wave_ballot(valid && v[t] > 0.f);
      if (hit) {
        const int l = int(__builtin_ctzll(hit));
        hit_seg = c0 + l;
        carry_before = __shfl(incl[t] - v[t], l);
      } else if (pos) {
        const int l = 63 - int(__builtin_clzll(pos));
        last_pos = c0 + l;
        carry_before = __shfl(incl[t] - v[t], l);
      }
    }
  }
  bool by_target = hit_seg >= 0;
  const int sidx = by_target ? hit_seg : last_pos;
  int y = 0;
  if (sidx >= 0) {
    const int e0 = (sidx / kSegPerChunk) * kChunk + (sidx % kSegPerChunk) * kSegLen + lane * 8;
    float w[8], pw[8];
    weights8<T, true, CUT>(d, e0, vocab, sl2, row_vec_ok(static_cast<const T*>(d.prow)),
                           row_vec_ok(static_cast<const T*>(d.qrow)), w, pw);
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ls += w[j];
    const float incl = wave_inclusive_scan(ls);
    const uint64_t hit = wave_ballot(by_target && carry_before + incl > target);
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
      float cum = carry_before + incl - ls;
      int pick = -1, lastp = -1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        cum += w[j];
        if (w[j] > 0.f) lastp = j;
        if (tgt && pick < 0 && cum > target) pick = j;
      }
      if (pick < 0) pick = (lastp >= 0) ? lastp : 0;
      y = e0 + pick;
    }
    y = __shfl(y, sel);
  }
  if (lane == 0) {
    out_tok[b] = y;
    if (out_mass) out_mass[b] = S;
  }
}

template <typename T, bool CUT = false>
__global__ __launch_bounds__(kWave) void draw_resolve_kernel(const DrawDesc* __restrict__ desc, int vocab,
                                                             float sl2, const float* __restrict__ seg,
                                                             const float* __restrict__ u_s,
                                                             int32_t* __restrict__ out_tok,
                                                             float* __restrict__ out_mass) {
  draw_resolve_body<T, CUT>(desc, vocab, sl2, seg, u_s, out_tok, out_mass, blockIdx.x);
}

// Launch the two draw kernels for `batch` descriptors (CUT: the rows carry a
// sampling transform).
template <typename T, bool CUT = false>
hipError_t launch_draw(const DrawDesc* desc, int batch, int vocab, float sl2, float* seg, const float* u_s,
                       int32_t* out_tok, float* out_mass, hipStream_t stream, const char* seg_name,
                       const char* resolve_name) {
  {
    ProfileScope ps(seg_name, stream);
    hipLaunchKernelGGL((draw_seg_kernel<T, CUT>), dim3(batch, num_chunks(vocab)), dim3(kChunkThreads), 0, stream,
                       desc, vocab, sl2, seg);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfileScope ps(resolve_name, stream);
    hipLaunchKernelGGL((draw_resolve_kernel<T, CUT>), dim3(batch), dim3(kWave), 0, stream, desc, vocab, sl2, seg,
                       u_s, out_tok, out_mass);
  }
  return hipGetLastError();
}

inline size_t draw_seg_bytes(int batch, int vocab) {
  return align_up(size_t(batch) * num_chunks(vocab) * 2 * kSegPerChunk * sizeof(float), 256);
}

}  // namespace uno
