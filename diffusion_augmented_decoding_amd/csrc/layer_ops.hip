// Per-row and elementwise operations of a decoder layer, gfx950: RMSNorm with
// an optional fused residual add, rotary position embedding, SwiGLU product.
//
// Method context: Uno summary (hyper.ai, arXiv 2609.04010), section "实验":
// the adapters are attached to an open-weight Qwen3-8B model, so one decode
// step runs that model's layers (pre-norm RMSNorm, rotary embeddings on q and
// k, SwiGLU MLP, residual stream) over the concatenated clean + noisy rows.
// All three are HBM-bound streams: one pass over their inputs, bf16 in and
// out, fp32 arithmetic, 16-byte vector accesses.
#include "device_common.h"
#include "internal.h"

namespace uno {

namespace {

constexpr int kNormThreads = 256;
constexpr int kNormMaxVec = 8;            // 8-element vectors per thread: dim <= 256 * 8 * 8

__device__ __forceinline__ void unpack8(const u32x4 v, float (&x)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = bf16_lo(v[j]);
    x[2 * j + 1] = bf16_hi(v[j]);
  }
}

__device__ __forceinline__ u32x4 pack8(const float (&x)[8]) {
  return u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
}

// One workgroup per row, VPT 8-element vectors per thread (dim <= 256 * 8 *
// VPT).  RES: s = x + res is rounded to bf16 and stored to sum_out (which may
// alias x), and the rounded s is what gets normalised.  out may be null
// (residual add only).  The weight vectors are loaded with the row, so the
// only dependent step after the loads is the reduction.
template <bool RES, int VPT>
__global__ __launch_bounds__(kNormThreads) void rms_norm_kernel(RmsNormArgs a) {
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nvec = a.dim / 8;
  const uint16_t* xr = static_cast<const uint16_t*>(a.x) + row * a.ldx;
  const uint16_t* wr = static_cast<const uint16_t*>(a.weight);
  const bool norm = a.out != nullptr;
  u32x4 xv[VPT], rv[VPT], wv[VPT];
#pragma unroll
  for (int c = 0; c < VPT; ++c) {
    const int i = tid + c * kNormThreads;
    if (i < nvec) {
      xv[c] = *reinterpret_cast<const u32x4*>(xr + 8 * i);
      if constexpr (RES) rv[c] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.res) + row * a.ldr + 8 * i);
      if (norm) wv[c] = *reinterpret_cast<const u32x4*>(wr + 8 * i);
    }
  }
  float v[VPT][8];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < VPT; ++c) {
    const int i = tid + c * kNormThreads;
    if (i < nvec) {
      unpack8(xv[c], v[c]);
      if constexpr (RES) {
        float y[8];
        unpack8(rv[c], y);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[c][e] = bf16_to_f32(f32_to_bf16(v[c][e] + y[e]));
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.sum_out) + row * a.lds + 8 * i) = pack8(v[c]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(v[c][e], v[c][e], ss);
    }
  }
  if (!norm) return;
  ss = wave_sum(ss);
  __shared__ float red[kNormThreads / kWave];
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kNormThreads / kWave; ++w) tot += red[w];
  const float rs = 1.f / sqrtf(tot / float(a.dim) + a.eps);
  uint16_t* orow = static_cast<uint16_t*>(a.out) + row * a.ldo;
#pragma unroll
  for (int c = 0; c < VPT; ++c) {
    const int i = tid + c * kNormThreads;
    if (i < nvec) {
      float w[8];
      unpack8(wv[c], w);
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = v[c][e] * rs * w[e];
      *reinterpret_cast<u32x4*>(orow + 8 * i) = pack8(o);
    }
  }
}

// Cache slot of a clean row for the optional KV append: rows come in
// sequences of 2*block (clean then noisy); clean row j of sequence b goes to
// slot cache_len[b] + j of that sequence's cache when the slot is inside the
// capacity.  Returns false for noisy rows, rows past the capacity and calls
// without an append; else sets the row's key and value destinations.
__device__ __forceinline__ bool append_slot(const RopeArgs& a, int64_t row, uint16_t*& kd, uint16_t*& vd) {
  if (!a.cache_len) return false;
  const int64_t b = row / (2 * a.block);
  const int j = int(row % (2 * a.block));
  if (j >= a.block) return false;
  const int64_t slot = int64_t(a.cache_len[b]) + j;
  if (slot < 0 || slot >= a.cap) return false;
  const int64_t off = (b * a.cap + slot) * int64_t(a.n_heads2) * 128;
  kd = static_cast<uint16_t*>(a.k_cache) + off;
  vd = static_cast<uint16_t*>(a.v_cache) + off;
  return true;
}

// In-place rotary embedding, one workgroup per row.  Thread t owns pair
// index i = t % 64 and forms the angle pos * theta^(-i/64) once, in double
// precision (positions far into a long context keep their phase), then
// rotates the pair (x_i, x_{i+64}) of every 4th head from t / 64 on, in x
// and then in the optional second tensor at the same positions (q and k).
// With a norm weight a head is first scaled by 1 / sqrt(mean(head^2) + eps)
// and the weight (one wave holds the whole head: a wave-wide sum), in fp32,
// rounded to bf16 once, after the rotation.
__global__ __launch_bounds__(256) void rope_kernel(RopeArgs a) {
  const int64_t row = blockIdx.x;
  const int i = threadIdx.x & 63, h0 = threadIdx.x >> 6;
  const double inv_freq = exp(-double(i) / 64.0 * log(double(a.theta)));
  double s, c;
  sincos(double(a.positions[row]) * inv_freq, &s, &c);
  const float cs = float(c), sn = float(s);
  auto rotate = [&](uint16_t* p, const uint16_t* nw) {
    float x1 = bf16_to_f32(p[i]), x2 = bf16_to_f32(p[i + 64]);
    if (nw) {
      const float rs = 1.f / sqrtf(wave_sum(fmaf(x2, x2, x1 * x1)) / 128.f + a.norm_eps);
      x1 = x1 * rs * bf16_to_f32(nw[i]);
      x2 = x2 * rs * bf16_to_f32(nw[i + 64]);
    }
    p[i] = f32_to_bf16(x1 * cs - x2 * sn);
    p[i + 64] = f32_to_bf16(x2 * cs + x1 * sn);
  };
  const uint16_t* nw1 = static_cast<const uint16_t*>(a.norm_w);
  const uint16_t* nw2 = static_cast<const uint16_t*>(a.norm_w2);
  uint16_t* xr = static_cast<uint16_t*>(a.x) + row * a.ldx;
  for (int h = h0; h < a.n_heads; h += 4) rotate(xr + h * 128, nw1);
  if (a.x2) {
    uint16_t* xr2 = static_cast<uint16_t*>(a.x2) + row * a.ldx2;
    for (int h = h0; h < a.n_heads2; h += 4) rotate(xr2 + h * 128, nw2);
    uint16_t *kd, *vd;
    if (append_slot(a, row, kd, vd)) {
      __syncthreads();   // the rotated row, written by this workgroup, is complete
      const uint16_t* vr = static_cast<const uint16_t*>(a.v) + row * a.ldv;
      for (int e = threadIdx.x; e < a.n_heads2 * 128; e += 256) {
        kd[e] = xr2[e];
        vd[e] = vr[e];
      }
    }
  }
}

// Vectorised rotary embedding (x, x2 8-byte aligned, leading dimensions
// multiples of 4), one workgroup per row: the 64 angles of the row are formed
// once, in double precision, by the first 64 threads and shared through LDS;
// then thread t rotates pairs 4 (t % 16) .. + 3 of heads t / 16, t / 16 + 16,
// ... with 8-byte loads and stores of x_i and x_{i+64}.  The optional
// per-head norm sums the head's squares over the 16 lanes that hold it.
__global__ __launch_bounds__(256) void rope_vec_kernel(RopeArgs a) {
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ float cs_s[64], sn_s[64];
  if (tid < 64) {
    const double inv_freq = exp(-double(tid) / 64.0 * log(double(a.theta)));
    double s, c;
    sincos(double(a.positions[row]) * inv_freq, &s, &c);
    cs_s[tid] = float(c);
    sn_s[tid] = float(s);
  }
  __syncthreads();
  const int i0 = 4 * (tid & 15), h0 = tid >> 4;
  float cs[4], sn[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    cs[j] = cs_s[i0 + j];
    sn[j] = sn_s[i0 + j];
  }
  // rotates the head at p in place (normed first with weight nw when given);
  // dup (optional) receives a copy of the result
  auto rotate = [&](uint16_t* p, uint16_t* dup, const uint16_t* nw) {
    const uint2 lo = *reinterpret_cast<const uint2*>(p + i0), hi = *reinterpret_cast<const uint2*>(p + 64 + i0);
    float x1[4] = {bf16_lo(lo.x), bf16_hi(lo.x), bf16_lo(lo.y), bf16_hi(lo.y)};
    float x2[4] = {bf16_lo(hi.x), bf16_hi(hi.x), bf16_lo(hi.y), bf16_hi(hi.y)};
    if (nw) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) ss = fmaf(x2[j], x2[j], fmaf(x1[j], x1[j], ss));
      // the 16 lanes of one head: xor distances 1..8 stay inside the group
      ss += swizzle_xor<1>(ss);
      ss += swizzle_xor<2>(ss);
      ss += swizzle_xor<4>(ss);
      ss += swizzle_xor<8>(ss);
      const float rs = 1.f / sqrtf(ss / 128.f + a.norm_eps);
      const uint2 wl = *reinterpret_cast<const uint2*>(nw + i0), wh = *reinterpret_cast<const uint2*>(nw + 64 + i0);
      const float w1[4] = {bf16_lo(wl.x), bf16_hi(wl.x), bf16_lo(wl.y), bf16_hi(wl.y)};
      const float w2[4] = {bf16_lo(wh.x), bf16_hi(wh.x), bf16_lo(wh.y), bf16_hi(wh.y)};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x1[j] = x1[j] * rs * w1[j];
        x2[j] = x2[j] * rs * w2[j];
      }
    }
    float o1[4], o2[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o1[j] = x1[j] * cs[j] - x2[j] * sn[j];
      o2[j] = x2[j] * cs[j] + x1[j] * sn[j];
    }
    const uint2 r1 = make_uint2(pack_bf16x2(o1[0], o1[1]), pack_bf16x2(o1[2], o1[3]));
    const uint2 r2 = make_uint2(pack_bf16x2(o2[0], o2[1]), pack_bf16x2(o2[2], o2[3]));
    *reinterpret_cast<uint2*>(p + i0) = r1;
    *reinterpret_cast<uint2*>(p + 64 + i0) = r2;
    if (dup) {
      *reinterpret_cast<uint2*>(dup + i0) = r1;
      *reinterpret_cast<uint2*>(dup + 64 + i0) = r2;
    }
  };
  const uint16_t* nw1 = static_cast<const uint16_t*>(a.norm_w);
  const uint16_t* nw2 = static_cast<const uint16_t*>(a.norm_w2);
  uint16_t* xr = static_cast<uint16_t*>(a.x) + row * a.ldx;
  for (int h = h0; h < a.n_heads; h += 16) rotate(xr + h * 128, nullptr, nw1);
  if (a.x2) {
    uint16_t* xr2 = static_cast<uint16_t*>(a.x2) + row * a.ldx2;
    uint16_t *kd = nullptr, *vd = nullptr;
    const bool app = append_slot(a, row, kd, vd);
    for (int h = h0; h < a.n_heads2; h += 16) rotate(xr2 + h * 128, app ? kd + h * 128 : nullptr, nw2);
    if (app) {
      // the value row goes to the cache unchanged, in 8-byte pieces
      const uint2* vr = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.v) + row * a.ldv);
      for (int e = threadIdx.x; e < a.n_heads2 * 32; e += 256) reinterpret_cast<uint2*>(vd)[e] = vr[e];
    }
  }
}

// out = silu(g) * u = g / (1 + e^-g) * u, 8 elements per thread.
__global__ __launch_bounds__(256) void silu_mul_kernel(SiluMulArgs a) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per_row = a.dim / 8;
  if (t >= a.rows * per_row) return;
  const int64_t row = t / per_row;
  const int c = int(t - row * per_row);
  float g[8], u[8], o[8];
  unpack8(*reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.g) + row * a.ldg + 8 * c), g);
  unpack8(*reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.u) + row * a.ldu + 8 * c), u);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = g[e] / (1.f + expf(-g[e])) * u[e];
  *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + row * a.ldo + 8 * c) = pack8(o);
}

}  // namespace

int rms_norm_max_dim() { return kNormThreads * 8 * kNormMaxVec; }

template <bool RES>
static hipError_t launch_norm_vpt(const RmsNormArgs& a, hipStream_t stream) {
  const int vpt = (a.dim / 8 + kNormThreads - 1) / kNormThreads;
  const dim3 grid(unsigned(a.rows)), block(kNormThreads);
  if (vpt <= 1)
    hipLaunchKernelGGL((rms_norm_kernel<RES, 1>), grid, block, 0, stream, a);
  else if (vpt <= 2)
    hipLaunchKernelGGL((rms_norm_kernel<RES, 2>), grid, block, 0, stream, a);
  else if (vpt <= 4)
    hipLaunchKernelGGL((rms_norm_kernel<RES, 4>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((rms_norm_kernel<RES, kNormMaxVec>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_rms_norm(const RmsNormArgs& a, hipStream_t stream) {
  ProfileScope ps(a.res ? "uno_add_rms_norm" : "uno_rms_norm", stream);
  return a.res ? launch_norm_vpt<true>(a, stream) : launch_norm_vpt<false>(a, stream);
}

hipError_t launch_rope(const RopeArgs& a, hipStream_t stream) {
  ProfileScope ps("uno_rope", stream);
  auto vec_ok = [](const void* p, int64_t ld) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0 && ld % 4 == 0; };
  const bool vec = vec_ok(a.x, a.ldx) && (!a.x2 || vec_ok(a.x2, a.ldx2)) &&
                   (!a.cache_len || (vec_ok(a.v, a.ldv) && vec_ok(a.k_cache, 0) && vec_ok(a.v_cache, 0))) &&
                   (!a.norm_w || vec_ok(a.norm_w, 0)) && (!a.norm_w2 || vec_ok(a.norm_w2, 0));
  if (vec)
    hipLaunchKernelGGL(rope_vec_kernel, dim3(unsigned(a.rows)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(rope_kernel, dim3(unsigned(a.rows)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const SiluMulArgs& a, hipStream_t stream) {
  const int64_t n = a.rows * (a.dim / 8);
  ProfileScope ps("uno_silu_mul", stream);
  hipLaunchKernelGGL(silu_mul_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace uno

namespace uno {

namespace {

// One workgroup per row: the embedding row copied in 16-byte vectors, the
// row's gate and position written by thread 0.  Clean row j sits at
// ctx + j and noisy row j at ctx + block + j (the noisy rows stand for the
// next block); ctx is the sequence's valid cache rows, clamped to the
// capacity as the attention kernel clamps it.
__global__ __launch_bounds__(256) void step_setup_kernel(StepSetupArgs a) {
  const int64_t row = blockIdx.x;
  const int j = int(row % (2 * a.block));
  const int tok = a.tokens[row];
  const bool ok = tok >= 0 && tok < a.vocab;
  const int nvec = a.hidden / 8;
  const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.embed) + int64_t(ok ? tok : 0) * a.hidden);
  u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.h) + row * a.hidden);
  for (int i = threadIdx.x; i < nvec; i += 256) dst[i] = ok ? src[i] : u32x4{0u, 0u, 0u, 0u};
  if (threadIdx.x == 0) {
    int ctx = a.ctx;
    if (a.cache_len) ctx = min(max(a.cache_len[row / (2 * a.block)], 0), a.cap);
    a.gate[row] = j >= a.block ? 1 : 0;
    a.positions[row] = ctx + j;
  }
}

// The commit of one sequence (cache_len may be null: no cache to commit to).
// Returns false when the sequence is flagged.
__device__ __forceinline__ bool commit_one(int b, int cap, int32_t* accept_len, int32_t* cache_len) {
  const int L = accept_len[b];
  if (!cache_len) return L >= 0;
  const int len = min(max(cache_len[b], 0), cap);
  if (L < 0 || int64_t(len) + L + 1 > cap) {
    accept_len[b] = -1;
    return false;
  }
  cache_len[b] = len + L + 1;
  return true;
}

}  // namespace

// One thread per sequence: the kept rows (the block's AR token and the L
// accepted drafts, already written by the forward pass) join the valid
// prefix when they all fit; otherwise the sequence is flagged.
__global__ __launch_bounds__(256) void kv_commit_kernel(int batch, int cap, int32_t* accept_len, int32_t* cache_len) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= batch) return;
  commit_one(b, cap, accept_len, cache_len);
}

// One workgroup of 2*block threads per sequence: thread 0 commits (and on a
// flag writes token -1 too); thread j then writes id j of the next step:
// the token y (j = 0), draft j - 1 (j < block), or the noisy id (read and
// written by the same thread, so next may alias tokens).
__global__ __launch_bounds__(256) void step_finish_kernel(StepFinishArgs a) {
  const int b = blockIdx.x, j = threadIdx.x;
  __shared__ int32_t y;
  if (j == 0) {
    const bool ok = commit_one(b, a.cap, a.accept_len, a.cache_len);
    if (!ok) a.token[b] = -1;
    y = ok ? a.token[b] : -1;
  }
  __syncthreads();
  if (!a.next || j >= 2 * a.block) return;
  const int64_t at = int64_t(b) * 2 * a.block + j;
  int32_t id;
  if (j == 0)
    id = y;
  else if (j < a.block)
    id = a.drafts[int64_t(b) * (a.block - 1) + (j - 1)];
  else
    id = a.tokens[at];
  a.next[at] = id;
}

hipError_t launch_kv_commit(int batch, int cap, int32_t* accept_len, int32_t* cache_len, hipStream_t stream) {
  ProfileScope ps("uno_kv_commit", stream);
  hipLaunchKernelGGL(kv_commit_kernel, dim3(unsigned((batch + 255) / 256)), dim3(256), 0, stream, batch, cap,
                     accept_len, cache_len);
  return hipGetLastError();
}

hipError_t launch_step_finish(const StepFinishArgs& a, hipStream_t stream) {
  ProfileScope ps("uno_step_finish", stream);
  const unsigned threads = unsigned((2 * a.block + 63) / 64 * 64);
  hipLaunchKernelGGL(step_finish_kernel, dim3(unsigned(a.batch)), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_step_setup(const StepSetupArgs& a, hipStream_t stream) {
  ProfileScope ps("uno_step_setup", stream);
  hipLaunchKernelGGL(step_setup_kernel, dim3(unsigned(a.rows)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace uno
