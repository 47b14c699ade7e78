// Distillation losses of row pairs (student = adapter-on rows, teacher =
// adapter-off rows of the gated concatenated forward) for gfx950.
//
// Method: Uno summary (hyper.ai, arXiv 2609.04010), section "方法", the
// paragraphs on diffusion distillation: the objective alpha * L_DCD +
// beta * L_TV over one forward of the concatenated clean (teacher) and noisy
// (student) rows; the block KL between the student and the teacher
// distribution; the TV distance, which lengthens the accepted draft prefix.
// Per row pair, at temperature T (p = softmax(teacher / T), q = softmax(student / T)):
//     KL = sum_v q_v (ln q_v - ln p_v),   TV = 1/2 sum_v |q_v - p_v|,
//     dL/dz_v = grad_scale / T * q_v * (alpha (ln q_v - ln p_v - KL)
//                                       + beta / 2 (sign(q_v - p_v) - sum_u sign(q_u - p_u) q_u))
// for L = grad_scale * (alpha KL + beta TV), z the student logits.
//
// One workgroup (1024 threads) per row pair, three passes over the pair:
//   1. softmax statistics of both rows (online max / sum in the log2 domain);
//   2. KL, TV and the sign-weighted mass, each term formed from the final
//      statistics (ln q - ln p per token, so no cancellation between large
//      row-level terms);
//   3. the gradient, written in the logits' dtype.
// sign(q_v - p_v) is taken as the sign of log2 q_v - log2 p_v (the same
// order, exp2 being increasing), so pass 3 needs no teacher exponential.
// Pass 1 streams the pair from HBM; with one pair per compute unit the pair
// (2 x 297 KB at V = 151,936 in bf16) stays in the memory-side cache for the
// re-reads of passes 2 and 3.  Sums are taken in a fixed order (deterministic).
#include <type_traits>

#include "sampler_common.h"

namespace uno {

namespace {

constexpr int kDThreads = 1024;
constexpr int kDWaves = kDThreads / kWave;
constexpr int kUnroll = 4;                     // 8-element groups in flight per thread and row
constexpr float kLn2 = 0.69314718055994531f;

template <typename T>
__device__ __forceinline__ const T* pair_row(const void* base, int64_t seq_stride, int64_t row_stride, int pair,
                                             int rows) {
  const int b = pair / rows, i = pair - b * rows;
  return static_cast<const T*>(base) + int64_t(b) * seq_stride + int64_t(i) * row_stride;
}

// Block-wide sums of three values (fixed order: lanes, then waves in order).
__device__ __forceinline__ void block_sum3(float& a, float& b, float& c, float (*sh)[kDWaves]) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  a = wave_sum(a);
  b = wave_sum(b);
  c = wave_sum(c);
  if (lane == 0) {
    sh[0][wave] = a;
    sh[1][wave] = b;
    sh[2][wave] = c;
  }
  __syncthreads();
  a = b = c = 0.f;
#pragma unroll
  for (int w = 0; w < kDWaves; ++w) {
    a += sh[0][w];
    b += sh[1][w];
    c += sh[2][w];
  }
  __syncthreads();
}

__device__ __forceinline__ float mul_rn(float x, float y) {
#pragma clang fp contract(off)
  return x * y;
}

// Online (max, sum) of a group of scaled logits y (log2 domain).  Every pass
// forms y = x * (log2 e / T) as the same rounded product (never fused into a
// later subtraction), so equal rows give equal terms and a one-token row
// gives q = 1 exactly.
__device__ __forceinline__ void lse_update8(float& m, float& s, const float (&y)[8]) {
  float cmax = y[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) cmax = fmaxf(cmax, y[j]);
  const float mn = fmaxf(m, cmax);
  float acc = (m == mn) ? s : s * fast_exp2(m - mn);
#pragma unroll
  for (int j = 0; j < 8; ++j) acc += fast_exp2(y[j] - mn);
  m = mn;
  s = acc;
}

// Two floats to packed bf16 (round to nearest even) by the hardware conversion.
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T>
__device__ __forceinline__ void store8(T* row, int e0, int vocab, bool vec_ok, const float (&g)[8]) {
  if (vec_ok && e0 + 8 <= vocab) {
    if constexpr (sizeof(T) == 2) {
      u32x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = cvt_bf16x2(g[2 * j], g[2 * j + 1]);
      *reinterpret_cast<u32x4*>(row + e0) = v;
    } else {
      f32x4 v0, v1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v0[j] = g[j];
        v1[j] = g[4 + j];
      }
      *reinterpret_cast<f32x4*>(row + e0) = v0;
      *reinterpret_cast<f32x4*>(row + e0 + 4) = v1;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (e0 + j < vocab) {
        if constexpr (sizeof(T) == 2)
          row[e0 + j] = uint16_t(cvt_bf16x2(g[j], 0.f) & 0xffffu);
        else
          row[e0 + j] = g[j];
      }
    }
  }
}

constexpr int kStep = kDThreads * 8;           // elements per group across the workgroup

// The kUnroll groups of 8 of both rows at base + u * kStep.  FULL: the whole
// tile lies inside the rows and both are 16-byte aligned (a condition uniform
// over the workgroup): straight-line vector loads, all issued before the
// first use.  Otherwise the bounds-checked loads (elements past V read as 0).
template <typename T, bool NT, bool FULL>
__device__ __forceinline__ void load_pair_tile(const T* srow, const T* trow, int base, int V, bool vs, bool vt,
                                               float (&xq)[kUnroll][8], float (&xp)[kUnroll][8]) {
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    if constexpr (FULL) {
      load8_vec<T, NT>(srow, base + u * kStep, xq[u]);
      load8_vec<T, NT>(trow, base + u * kStep, xp[u]);
    } else {
      load8<T, NT>(srow, base + u * kStep, V, vs, xq[u]);
      load8<T, NT>(trow, base + u * kStep, V, vt, xp[u]);
    }
  }
}

// Runs body(std::true_type) for a tile wholly inside aligned rows, else
// body(std::false_type): the in-range path carries no per-element masks.
template <typename F>
__device__ __forceinline__ void tile_dispatch(bool full, F&& body) {
  if (full)
    body(std::true_type{});
  else
    body(std::false_type{});
}

template <typename T>
__global__ __launch_bounds__(kDThreads) void distill_kernel(DistillArgs a) {
#pragma clang fp contract(off)   // y = x * sl2 stays a rounded product in every pass
  __shared__ float sh[3][kDWaves];
  const int pair = blockIdx.x, tid = threadIdx.x;
  const int V = a.vocab;
  const float sl2 = a.scale_log2;
  const T* trow = pair_row<T>(a.teacher, a.t_seq, a.t_row, pair, a.rows);
  const T* srow = pair_row<T>(a.student, a.s_seq, a.s_row, pair, a.rows);
  const bool vt = row_vec_ok(trow), vs = row_vec_ok(srow);

  // pass 1: (max, sum) of both rows, log2 domain
  float mq = -INFINITY, sq = 0.f, mp = -INFINITY, sp = 0.f;
  for (int tile = 0; tile < V; tile += kStep * kUnroll) {
    tile_dispatch(vs && vt && tile + kStep * kUnroll <= V, [&](auto full_c) {
      constexpr bool FULL = decltype(full_c)::value;
      const int base = tile + tid * 8;
      float xq[kUnroll][8], xp[kUnroll][8];
      load_pair_tile<T, false, FULL>(srow, trow, base, V, vs, vt, xq, xp);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int e0 = base + u * kStep;
        if (FULL || e0 < V) {
          float yq[8], yp[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const bool in = FULL || e0 + j < V;
            yq[j] = in ? mul_rn(xq[u][j], sl2) : -INFINITY;
            yp[j] = in ? mul_rn(xp[u][j], sl2) : -INFINITY;
          }
          lse_update8(mq, sq, yq);
          lse_update8(mp, sp, yp);
        }
      }
    });
  }
  {
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    wave_lse2(mq, sq);
    wave_lse2(mp, sp);
    __shared__ float shm[4][kDWaves];
    if (lane == 0) {
      shm[0][wave] = mq;
      shm[1][wave] = sq;
      shm[2][wave] = mp;
      shm[3][wave] = sp;
    }
    __syncthreads();
    mq = shm[0][0];
    sq = shm[1][0];
    mp = shm[2][0];
    sp = shm[3][0];
#pragma unroll
    for (int w = 1; w < kDWaves; ++w) {
      lse2_merge(mq, sq, shm[0][w], shm[1][w]);
      lse2_merge(mp, sp, shm[2][w], shm[3][w]);
    }
    __syncthreads();
  }
  // log2 q_v = y_v - Lq (a one-token row: Lq = mq, q = 1 exactly)
  const float Lq = mq + log2f(sq), Lp = mp + log2f(sp);

  // pass 2: KL (log2 units), sum |q - p|, sum sign(q - p) q
  float kl = 0.f, tv = 0.f, ss = 0.f;
  for (int tile = 0; tile < V; tile += kStep * kUnroll) {
    tile_dispatch(vs && vt && tile + kStep * kUnroll <= V, [&](auto full_c) {
      constexpr bool FULL = decltype(full_c)::value;
      const int base = tile + tid * 8;
      float xq[kUnroll][8], xp[kUnroll][8];
      load_pair_tile<T, false, FULL>(srow, trow, base, V, vs, vt, xq, xp);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int e0 = base + u * kStep;
        const int nv = FULL ? 8 : min(8, V - e0);   // valid elements of the group (<= 0: none)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float uq = mul_rn(xq[u][j], sl2) - Lq, up = mul_rn(xp[u][j], sl2) - Lp;
          const float q = j < nv ? fast_exp2(uq) : 0.f, p = j < nv ? fast_exp2(up) : 0.f;
          const float d = uq - up;
          kl = fmaf(q, d, kl);
          tv += fabsf(q - p);
          ss += (d > 0.f) ? q : ((d < 0.f) ? -q : 0.f);
        }
      }
    });
  }
  block_sum3(kl, tv, ss, sh);
  const float KL = kLn2 * kl;
  if (tid == 0) {
    a.out_kl[pair] = KL;
    a.out_tv[pair] = 0.5f * tv;
  }
  if (!a.grad) return;

  // pass 3: the gradient in the student logits
  T* grow = static_cast<T*>(a.grad) + int64_t(pair / a.rows) * a.g_seq + int64_t(pair % a.rows) * a.g_row;
  const bool vg = row_vec_ok(static_cast<const T*>(grow));
  const float c0 = a.grad_scale * a.inv_t;
  const float akl = a.alpha * kLn2, hb = 0.5f * a.beta;
  const float off = a.alpha * KL + hb * ss;     // sum_u q_u (alpha (ln q_u - ln p_u) + beta/2 sign_u)
  for (int tile = 0; tile < V; tile += kStep * kUnroll) {
    tile_dispatch(vs && vt && tile + kStep * kUnroll <= V, [&](auto full_c) {
      constexpr bool FULL = decltype(full_c)::value;
      const int base = tile + tid * 8;
      float xq[kUnroll][8], xp[kUnroll][8];
      load_pair_tile<T, true, FULL>(srow, trow, base, V, vs, vt, xq, xp);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int e0 = base + u * kStep;
        if (FULL || e0 < V) {
          float g[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float uq = mul_rn(xq[u][j], sl2) - Lq, up = mul_rn(xp[u][j], sl2) - Lp;
            const float q = fast_exp2(uq);
            const float d = uq - up;
            const float sg = (d > 0.f) ? 1.f : ((d < 0.f) ? -1.f : 0.f);
            g[j] = c0 * q * (fmaf(akl, d, fmaf(hb, sg, -off)));
          }
          store8<T>(grow, e0, V, vg, g);
        }
      }
    });
  }
}

}  // namespace

hipError_t launch_distill(const DistillArgs& a, hipStream_t stream) {
  const unsigned pairs = unsigned(int64_t(a.batch) * a.rows);
  ProfileScope ps("uno_distill", stream);
  if (a.dtype == UNO_BF16)
    hipLaunchKernelGGL(distill_kernel<uint16_t>, dim3(pairs), dim3(kDThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(distill_kernel<float>, dim3(pairs), dim3(kDThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace uno
