// Device-side helpers shared by the gfx950 kernels of libunospec.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace uno {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 storage is the top 16 bits of an fp32.
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16 with round-to-nearest-even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// ---------------------------------------------------------------- wave reductions
// Butterfly over the 64 lanes: ds_swizzle (xor within 32 lanes) and a
// ds_bpermute-free cross-half exchange via readlane-free __shfl_xor.
template <int XOR>
__device__ __forceinline__ float swizzle_xor(float v) {
  static_assert(XOR < 32, "swizzle covers 32 lanes");
  // bit-mode pattern: and_mask = 0x1f, or_mask = 0, xor_mask = XOR
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (XOR << 10) | 0x1f));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += swizzle_xor<1>(v);
  v += swizzle_xor<2>(v);
  v += swizzle_xor<4>(v);
  v += swizzle_xor<8>(v);
  v += swizzle_xor<16>(v);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, swizzle_xor<1>(v));
  v = fmaxf(v, swizzle_xor<2>(v));
  v = fmaxf(v, swizzle_xor<4>(v));
  v = fmaxf(v, swizzle_xor<8>(v));
  v = fmaxf(v, swizzle_xor<16>(v));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// Merge of two online-softmax partials (max m, sum s of 2^(y - m)).
__device__ __forceinline__ void lse2_merge(float& m, float& s, float m2, float s2) {
  float mn = fmaxf(m, m2);
  float a = (m == mn) ? s : s * exp2f(m - mn);
  float b = (m2 == mn) ? s2 : s2 * exp2f(m2 - mn);
  m = mn;
  s = a + b;
}

template <int XOR>
__device__ __forceinline__ void lse2_step_swz(float& m, float& s) {
  float m2 = swizzle_xor<XOR>(m);
  float s2 = swizzle_xor<XOR>(s);
  lse2_merge(m, s, m2, s2);
}

__device__ __forceinline__ void wave_lse2(float& m, float& s) {
  lse2_step_swz<1>(m, s);
  lse2_step_swz<2>(m, s);
  lse2_step_swz<4>(m, s);
  lse2_step_swz<8>(m, s);
  lse2_step_swz<16>(m, s);
  float m2 = __shfl_xor(m, 32);
  float s2 = __shfl_xor(s, 32);
  lse2_merge(m, s, m2, s2);
}

// Butterfly within aligned groups of `width` lanes (a power of two <= 64,
// uniform across the wave); every lane of a group ends with the same bits.
__device__ __forceinline__ void group_lse2(float& m, float& s, int width) {
  if (width > 1) lse2_step_swz<1>(m, s);
  if (width > 2) lse2_step_swz<2>(m, s);
  if (width > 4) lse2_step_swz<4>(m, s);
  if (width > 8) lse2_step_swz<8>(m, s);
  if (width > 16) lse2_step_swz<16>(m, s);
  if (width > 32) {
    float m2 = __shfl_xor(m, 32);
    float s2 = __shfl_xor(s, 32);
    lse2_merge(m, s, m2, s2);
  }
}

// Inclusive prefix sum over the 64 lanes in lane order (Hillis-Steele; fixed order).
__device__ __forceinline__ float wave_inclusive_scan(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    float o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __ballot(p); }

}  // namespace uno
