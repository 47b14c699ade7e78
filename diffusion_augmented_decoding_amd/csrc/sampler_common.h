// Device building blocks of the Psi-Spec verify samplers (linear and tree):
// streaming softmax statistics of one logit row, and a block-wide inverse-CDF
// draw over w_v = max(0, p_v - c q_v) in token-id order.
#pragma once
#include "device_common.h"
#include "internal.h"

namespace uno {

constexpr int kStatThreads = 256;
constexpr int kStatUnroll = 4;
constexpr int kDrawThreads = 1024;
constexpr int kDrawWaves = kDrawThreads / kWave;
constexpr int kEPT = 8;                          // elements per thread per tile
constexpr int kDrawTile = kDrawThreads * kEPT;   // 8192 elements
constexpr int kSeg = kWave * kEPT;               // 512 elements per (tile, wave) segment
constexpr int kMaxVocab = 1 << 20;
constexpr int kMaxTiles = kMaxVocab / kDrawTile; // 128
constexpr int kSegSlots = kMaxTiles * kDrawWaves;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T> __device__ __forceinline__ float load_logit(const T* p, int64_t i);
template <> __device__ __forceinline__ float load_logit<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}
template <> __device__ __forceinline__ float load_logit<float>(const float* p, int64_t i) { return p[i]; }

// 16-byte vector of logits, unpacked to fp32.
template <typename T> struct Vec16;
template <> struct Vec16<uint16_t> {
  static constexpr int N = 8;
  u32x4 raw;
  __device__ __forceinline__ void load(const uint16_t* p) {
    raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  __device__ __forceinline__ float get(int j) const {
    uint32_t w = raw[j >> 1];
    return (j & 1) ? bf16_hi(w) : bf16_lo(w);
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  f32x4 raw;
  __device__ __forceinline__ void load(const float* p) {
    raw = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  }
  __device__ __forceinline__ float get(int j) const { return raw[j]; }
};

// Online update of (m, s) with a group of raw logits x (y = x * sl2).
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

// Softmax statistics of one row, by a kStatThreads-thread block:
// out = {max y, sum 2^(y - max), logit at `draft` (if >= 0)}.
template <typename T>
__device__ void row_stats_body(const T* __restrict__ row, int vocab, float sl2, int draft,
                               RowStat* __restrict__ out) {
  using V = Vec16<T>;
  constexpr int VN = V::N;
  const int tid = threadIdx.x;
  float m = -INFINITY, s = 0.f;

  const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
  int head = int(((16u - (addr & 15u)) & 15u) / sizeof(T));
  if (head > vocab) head = vocab;
  if (tid < head) {
    float x[1] = {load_logit<T>(row, tid)};
    online_update<1>(m, s, x, sl2);
  }
  const T* vrow = row + head;
  const int nvec = (vocab - head) / VN;
  int i = tid;
  for (; i + (kStatUnroll - 1) * kStatThreads < nvec; i += kStatUnroll * kStatThreads) {
    V v[kStatUnroll];
#pragma unroll
    for (int u = 0; u < kStatUnroll; ++u) v[u].load(vrow + int64_t(i + u * kStatThreads) * VN);
    float x[kStatUnroll * VN];
#pragma unroll
    for (int u = 0; u < kStatUnroll; ++u)
#pragma unroll
      for (int j = 0; j < VN; ++j) x[u * VN + j] = v[u].get(j);
    online_update<kStatUnroll * VN>(m, s, x, sl2);
  }
  for (; i < nvec; i += kStatThreads) {
    V v;
    v.load(vrow + int64_t(i) * VN);
    float x[VN];
#pragma unroll
    for (int j = 0; j < VN; ++j) x[j] = v.get(j);
    online_update<VN>(m, s, x, sl2);
  }
  const int t = head + nvec * VN + tid;
  if (t < vocab) {
    float x[1] = {load_logit<T>(row, t)};
    online_update<1>(m, s, x, sl2);
  }

  wave_lse2(m, s);
  __shared__ float sm[kStatThreads / kWave], ss[kStatThreads / kWave];
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  if (lane == 0) {
    sm[wave] = m;
    ss[wave] = s;
  }
  __syncthreads();
  if (tid == 0) {
    float M = sm[0], S = ss[0];
#pragma unroll
    for (int w = 1; w < kStatThreads / kWave; ++w) lse2_merge(M, S, sm[w], ss[w]);
    RowStat r;
    r.m = M;
    r.s = S;
    // an out-of-range draft id reads nothing and gets probability 0 (rejected)
    r.yd = (draft >= 0 && draft < vocab) ? load_logit<T>(row, draft) : -INFINITY;
    r.pad = 0.f;
    *out = r;
  }
}

// Loads 8 consecutive logits starting at e0 (bounds- and alignment-safe).
template <typename T>
__device__ __forceinline__ void load8(const T* row, int e0, int vocab, bool vec_ok, float (&x)[8]) {
  if (vec_ok && e0 + 8 <= vocab) {
    if constexpr (sizeof(T) == 2) {
      Vec16<T> v;
      v.load(row + e0);
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = v.get(j);
    } else {
      Vec16<T> v0, v1;
      v0.load(row + e0);
      v1.load(row + e0 + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = v0.get(j);
        x[4 + j] = v1.get(j);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = (e0 + j < vocab) ? load_logit<T>(row, e0 + j) : 0.f;
  }
}

// The distribution a draw is taken from: w_v = max(0, p_v - c q_v) (c > 0) or
// w_v = p_v (c == 0); p_v = 2^(x_v sl2 - mp) / sp, likewise q.
template <typename T>
struct DrawRows {
  const T* prow;
  const T* qrow;
  float mp, inv_sp, mq, inv_sq;
  float c;
  bool vec_p, vec_q;
};

template <typename T>
__device__ __forceinline__ void weights8(const DrawRows<T>& d, int e0, int vocab, float sl2, float (&w)[8]) {
  float xp[8];
  load8<T>(d.prow, e0, vocab, d.vec_p, xp);
  if (d.c != 0.f) {
    float xq[8];
    load8<T>(d.qrow, e0, vocab, d.vec_q, xq);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = fast_exp2(fmaf(xp[j], sl2, -d.mp)) * d.inv_sp;
      const float q = fast_exp2(fmaf(xq[j], sl2, -d.mq)) * d.inv_sq;
      w[j] = (e0 + j < vocab) ? fmaxf(fmaf(-d.c, q, p), 0.f) : 0.f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      w[j] = (e0 + j < vocab) ? fast_exp2(fmaf(xp[j], sl2, -d.mp)) * d.inv_sp : 0.f;
  }
}

struct DrawShared {
  float seg[kSegSlots];     // per-(tile, wave) masses, then their inclusive prefix
  int seg_hit;
  float carry, target, total;
};

// Inverse-CDF draw by a kDrawThreads-thread block: y = smallest v with
// cumsum(w)[v] > u * sum(w); if rounding leaves none, the last v with w_v > 0.
// If sum(w) == 0 for c > 0, draws from p instead.  Returns y and sum(w) in
// every thread.  Every thread of the block must call it.
template <typename T>
__device__ void block_draw(DrawRows<T> d, int vocab, float sl2, float u, DrawShared& sh, int& y_out,
                           float& mass_out) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int ntiles = (vocab + kDrawTile - 1) / kDrawTile;
  const int nseg = ntiles * kDrawWaves;
  for (int attempt = 0; attempt < 2; ++attempt) {
    for (int t = 0; t < ntiles; t += 2) {
      float w0[8], w1[8];
      const int e0 = t * kDrawTile + tid * kEPT;
      weights8<T>(d, e0, vocab, sl2, w0);
      const bool has1 = (t + 1) < ntiles;
      if (has1) weights8<T>(d, e0 + kDrawTile, vocab, sl2, w1);
      float s0 = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) s0 += w0[j];
      s0 = wave_sum(s0);
      if (lane == 0) sh.seg[t * kDrawWaves + wave] = s0;
      if (has1) {
        float s1 = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) s1 += w1[j];
        s1 = wave_sum(s1);
        if (lane == 0) sh.seg[(t + 1) * kDrawWaves + wave] = s1;
      }
    }
    __syncthreads();
    if (wave == 0) {
      float carry = 0.f;
      for (int c = 0; c < nseg; c += kWave) {
        const float v = (c + lane < nseg) ? sh.seg[c + lane] : 0.f;
        const float incl = wave_inclusive_scan(v);
        if (c + lane < nseg) sh.seg[c + lane] = carry + incl;     // inclusive prefix
        carry += __shfl(incl, kWave - 1);
      }
      const float S = carry;
      const float target = u * S;
      int seg = -1, last_pos = -1;
      for (int c = 0; c < nseg && seg < 0; c += kWave) {
        const int i = c + lane;
        const float pre = (i < nseg) ? sh.seg[i] : 0.f;
        const float prev = (i == 0) ? 0.f : ((i < nseg) ? sh.seg[i - 1] : 0.f);
        const uint64_t hit = wave_ballot(i < nseg && pre > target);
        const uint64_t pos = wave_ballot(i < nseg && pre > prev);
        if (hit) seg = c + int(__builtin_ctzll(hit));
        if (pos) last_pos = c + 63 - int(__builtin_clzll(pos));
      }
      if (seg < 0) seg = last_pos;
      if (lane == 0) {
        sh.total = S;
        sh.target = target;
        sh.seg_hit = seg;
        sh.carry = (seg > 0) ? sh.seg[seg - 1] : 0.f;
      }
    }
    __syncthreads();
    if (sh.total > 0.f || d.c == 0.f) break;
    d.c = 0.f;            // residual without mass: fall back to p
    __syncthreads();
  }

  __shared__ int sh_y;
  if (wave == 0) {
    const int seg = sh.seg_hit;
    int y = 0;
    if (seg >= 0) {
      const int t = seg / kDrawWaves, wv = seg - t * kDrawWaves;
      const int e0 = t * kDrawTile + wv * kSeg + lane * kEPT;
      float w[8];
      weights8<T>(d, e0, vocab, sl2, w);
      float ls = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ls += w[j];
      const float incl = wave_inclusive_scan(ls);
      const float carry = sh.carry, target = sh.target;
      const uint64_t hit = wave_ballot(carry + incl > target);
      const uint64_t pos = wave_ballot(ls > 0.f);
      int sel;
      bool by_target;
      if (hit) {
        sel = int(__builtin_ctzll(hit));
        by_target = true;
      } else {
        sel = pos ? 63 - int(__builtin_clzll(pos)) : 0;
        by_target = false;
      }
      if (lane == sel) {
        float cum = carry + incl - ls;
        int pick = -1, lastp = -1;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          cum += w[j];
          if (w[j] > 0.f) lastp = j;
          if (by_target && pick < 0 && cum > target) pick = j;
        }
        if (pick < 0) pick = (lastp >= 0) ? lastp : 0;
        y = e0 + pick;
      }
      y = __shfl(y, sel);
    }
    if (lane == 0) sh_y = y;
  }
  __syncthreads();
  y_out = sh_y;
  mass_out = sh.total;
}

}  // namespace uno
