// Gated-LoRA backward for gfx950: the gradients of
//     y = x W^T + s diag(g) (x A^T) B^T
// in x, A and B (W is the frozen AR weight), the training side of the gated
// concatenated forward.
//
// Method: Uno summary (hyper.ai, arXiv 2609.04010), section "方法": the
// diffusion weights are low-rank adapters on every AR weight matrix, trained
// by distillation with the AR weights frozen; one forward runs over the
// concatenated clean and noisy rows with the adapter masked off on clean rows.
// With dY = dL/dy, U = diag(g) (x A^T):
//     dB = s dY^T U,   dT = s diag(g) dY B,   dA = dT^T x,   dx = dY W + dT A.
//
// Every product is one launch of a bf16 MFMA GEMM (v_mfma_f32_32x32x16_bf16,
// 128 x 128 output tiles, 32-deep K tiles, four waves of 64 x 64) that takes
// each operand in whichever layout it is stored in:
//   "xk": the reduction index contiguous (row-major x, dY, A as the B side of
//         x A^T): 16-byte LDS fragment reads;
//   "kx": the output index contiguous (W, A and B as right-hand sides, dY and
//         the row-gradients read along rows): the tile is staged row-major
//         and the MFMA fragment (8 consecutive k at one output index per lane)
//         comes from two ds_read_b64_tr_b16, which transpose 4 x 16 patches
//         of 16-bit values across each 16-lane group -- no transposition pass.
// dx = [dY | dT] [W ; A] is one GEMM with two K segments.  U and dT are kept
// in bf16 (the forward's adapter input is bf16 too); dA and dB are fp32.
// Products with few output tiles (U and dT have M/128 x r/128 of them) split
// their reduction over blockIdx.z into fp32 partials, which a second launch
// sums in split order (deterministic) and scales / converts.
//
// Given W^T (the frozen weight transposed once, e.g. by uno_transpose_bf16),
// the bf16 products instead run on the forward's kernels, whose operands all
// have the reduction index contiguous: U = g (x A^T) and dT = s g (dY (B^T)^T)
// on the LoRA-down, dx = dY (W^T)^T + dT (A^T)^T on the main GEMM with its
// adapter columns; A^T and B^T (r x K and r x N) are transposed per call.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace uno {

namespace {

constexpr int kBT = 128;                      // output tile (rows and columns)
constexpr int kBK = 32;                       // reduction tile
constexpr int kThr = 256;                     // 4 waves, 2 x 2, 64 x 64 each
constexpr int kXkPitch = kBK + 8;             // elements per LDS row of an "xk" tile (80 bytes)
constexpr int kKxPitch = kBT + 16;            // elements per LDS row of a "kx" tile (288 bytes)
constexpr int kXkBytes = kBT * kXkPitch * 2;
constexpr int kKxBytes = kBK * kKxPitch * 2;
constexpr int kOpBytes = kXkBytes > kKxBytes ? kXkBytes : kKxBytes;
constexpr int kStageBytes = 2 * kOpBytes;     // A and B tiles

typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));

struct BwdGemm {
  int M, N, K, k1;                  // C[M][N] = alpha * g[m] * sum_k A(m, k) B(k, n); k >= k1: second segment
  const uint16_t* a; int64_t lda;
  const uint16_t* a2; int64_t lda2;
  const uint16_t* b; int64_t ldb;
  const uint16_t* b2; int64_t ldb2;
  void* c; int64_t ldc;
  float alpha;
  const uint8_t* gate;              // optional: rows with gate 0 are written as 0
  int kt_per_split;                 // K tiles per split
  int nsplit;                       // > 1: raw fp32 partials to part, summed by split_reduce_kernel
  float* part;                      // [nsplit][M][N]
};

// One operand's K tile, global -> registers (two 16-byte vectors per thread).
// KX: element (i, k) at p[k * ld + i], else at p[i * ld + k]; i < lim, k < klim
// (tile-relative k from 0), zero outside.
template <bool KX>
__device__ __forceinline__ void gload(u32x4 (&v)[2], const uint16_t* p, int64_t ld, int i0, int lim, int k0,
                                      int klim) {
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int q = threadIdx.x + kThr * r;
    int i, k;
    if constexpr (KX) {
      k = q >> 4;
      i = (q & 15) * 8;
    } else {
      i = q >> 2;
      k = (q & 3) * 8;
    }
    const bool ok = i0 + i < lim && k0 + k < klim;
    v[r] = ok ? *reinterpret_cast<const u32x4*>(KX ? p + int64_t(k0 + k) * ld + (i0 + i)
                                                     : p + int64_t(i0 + i) * ld + (k0 + k))
              : u32x4{0u, 0u, 0u, 0u};
  }
}

template <bool KX>
__device__ __forceinline__ void sstore(unsigned char* tile, const u32x4 (&v)[2]) {
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int q = threadIdx.x + kThr * r;
    const int off = KX ? ((q >> 4) * kKxPitch + (q & 15) * 8) : ((q >> 2) * kXkPitch + (q & 3) * 8);
    *reinterpret_cast<u32x4*>(tile + off * 2) = v[r];
  }
}

// The four transposing reads of two "kx" fragments, waited for in the same
// block (their outputs are written when the wait completes).
__device__ __forceinline__ void tr_read4(s16x4 (&t)[4], const uint32_t (&addr)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\t"
      "ds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3])
      : "memory");
}

// The two MFMA fragments (output indices base + 32 f + lane % 32, k = 16 kk +
// 8 (lane / 32) + 0..7) of one operand from its LDS tile.
template <bool KX>
__device__ __forceinline__ void frags(bf16x8 (&f)[2], const unsigned char* tile, uint32_t tile_lds, int base,
                                      int kk) {
  const int lane = threadIdx.x & (kWave - 1);
  const int h = lane >> 5;
  if constexpr (!KX) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int i = base + 32 * g + (lane & 31);
      f[g] = *reinterpret_cast<const bf16x8*>(tile + (i * kXkPitch + 16 * kk + 8 * h) * 2);
    }
  } else {
    // lane j of each 16-lane group addresses row (j / 4) of a 4-row patch at
    // columns 4 (j % 4) .. + 3 and receives column j of the patch, rows 0..3
    const int j = lane & 15;
    uint32_t addr[4];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int col = base + 32 * g + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int row = 16 * kk + 8 * h + 4 * hh + (j >> 2);
        addr[2 * g + hh] = tile_lds + uint32_t((row * kKxPitch + col) * 2);
      }
    }
    s16x4 t[4];
    tr_read4(t, addr);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const s16x4 lo = t[2 * g], hi = t[2 * g + 1];
      const short __attribute__((ext_vector_type(8))) v8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      f[g] = __builtin_bit_cast(bf16x8, v8);
    }
  }
}

// Two products in one launch (same operand layouts): blockIdx.z < z0 runs
// split blockIdx.z of p0, the rest split blockIdx.z - z0 of p1; blockIdx.x
// numbers the output tiles of either (row-major over the tile grid).
template <bool AKX, bool BKX, bool OUTF32>
__global__ __launch_bounds__(kThr) void bwd_gemm_kernel(BwdGemm p0, BwdGemm p1, int z0) {
  __shared__ __align__(16) unsigned char smem[2 * kStageBytes];
  uint32_t lds_base = uint32_t(reinterpret_cast<uintptr_t>(smem));
  asm volatile("" : "+s"(lds_base));
  const bool first = int(blockIdx.z) < z0;
  const BwdGemm& p = first ? p0 : p1;
  const int zi = first ? int(blockIdx.z) : int(blockIdx.z) - z0;
  const int tiles_n = (p.N + kBT - 1) / kBT;
  if (int(blockIdx.x) >= tiles_n * ((p.M + kBT - 1) / kBT)) return;
  const int n0 = (int(blockIdx.x) % tiles_n) * kBT, m0 = (int(blockIdx.x) / tiles_n) * kBT;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int wm = wave >> 1, wn = wave & 1;
  const int kt0 = zi * p.kt_per_split;
  const int nkt = min((p.K + kBK - 1) / kBK - kt0, p.kt_per_split);

  auto load_tile = [&](int kt, u32x4 (&va)[2], u32x4 (&vb)[2]) {
    const int k = kt * kBK;
    if (k < p.k1) {
      gload<AKX>(va, p.a, p.lda, m0, p.M, k, p.k1);
      gload<BKX>(vb, p.b, p.ldb, n0, p.N, k, p.k1);
    } else {
      gload<AKX>(va, p.a2, p.lda2, m0, p.M, k - p.k1, p.K - p.k1);
      gload<BKX>(vb, p.b2, p.ldb2, n0, p.N, k - p.k1, p.K - p.k1);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  u32x4 va[2], vb[2];
  if (nkt > 0) {
    load_tile(kt0, va, vb);
    sstore<AKX>(smem, va);
    sstore<BKX>(smem + kOpBytes, vb);
  }
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nkt;
    if (more) load_tile(kt0 + kt + 1, va, vb);
    const unsigned char* As = smem + cur * kStageBytes;
    const unsigned char* Bs = As + kOpBytes;
    const uint32_t As_l = lds_base + uint32_t(cur * kStageBytes), Bs_l = As_l + kOpBytes;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8 fa[2], fb[2];
      frags<AKX>(fa, As, As_l, wm * 64, kk);
      frags<BKX>(fb, Bs, Bs_l, wn * 64, kk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[i], fa[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      unsigned char* nxt = smem + (cur ^ 1) * kStageBytes;
      sstore<AKX>(nxt, va);
      sstore<BKX>(nxt + kOpBytes, vb);
    }
    __syncthreads();
  }

  // lane l holds C[m = .. + 32 j + l % 32][n = .. + 32 i + 8 g + 4 (l / 32) + e] in acc[i][j][4 g + e]
  const int lh = lane >> 5;
  if (p.nsplit > 1) {   // raw partial sums of this split
    float* part = p.part + int64_t(zi) * p.M * p.N;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int m = m0 + wm * 64 + 32 * j + (lane & 31);
      if (m >= p.M) continue;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * 64 + 32 * i + 8 * g + 4 * lh;
          if (n < p.N)
            *reinterpret_cast<f32x4*>(part + int64_t(m) * p.N + n) =
                f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = m0 + wm * 64 + 32 * j + (lane & 31);
    if (m >= p.M) continue;
    const float sc = (p.gate && p.gate[m] == 0) ? 0.f : p.alpha;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * 64 + 32 * i + 8 * g + 4 * lh;
        if (n >= p.N) continue;
        const float v0 = sc * acc[i][j][4 * g], v1 = sc * acc[i][j][4 * g + 1];
        const float v2 = sc * acc[i][j][4 * g + 2], v3 = sc * acc[i][j][4 * g + 3];
        if constexpr (OUTF32) {
          float* dst = static_cast<float*>(p.c) + int64_t(m) * p.ldc + n;
          *reinterpret_cast<f32x4*>(dst) = f32x4{v0, v1, v2, v3};
        } else {
          uint16_t* dst = static_cast<uint16_t*>(p.c) + int64_t(m) * p.ldc + n;
          *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
        }
      }
    }
  }
}

// out[m][n] = alpha * g(m) * sum_s part[s][m][n] (splits summed in order); 4
// columns per thread; quads [0, nq0) belong to p0, the rest to p1.
template <bool OUTF32>
__global__ __launch_bounds__(256) void split_reduce_kernel(BwdGemm p0, BwdGemm p1, int64_t nq0, int64_t nq) {
  int64_t q = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (q >= nq) return;
  const bool first = q < nq0;
  const BwdGemm& p = first ? p0 : p1;
  if (!first) q -= nq0;
  const int m = int(q / (p.N / 4)), n = int(q % (p.N / 4)) * 4;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < p.nsplit; ++z) s += *reinterpret_cast<const f32x4*>(p.part + (int64_t(z) * p.M + m) * p.N + n);
  const float sc = (p.gate && p.gate[m] == 0) ? 0.f : p.alpha;
  s *= sc;
  if constexpr (OUTF32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(p.c) + int64_t(m) * p.ldc + n) = s;
  } else {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.c) + int64_t(m) * p.ldc + n) =
        make_uint2(pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]));
  }
}

// Reduction splits: enough workgroups for two per compute unit, each split
// at least 4 K tiles long.
int choose_splits(int M, int N, int K) {
  const int64_t tiles = int64_t((M + kBT - 1) / kBT) * ((N + kBT - 1) / kBT);
  const int nkt = (K + kBK - 1) / kBK;
  int s = int((512 + tiles - 1) / tiles);
  s = std::min(s, std::max(1, nkt / 4));
  return std::max(1, std::min(s, 64));
}

size_t split_bytes(int M, int N, int K) {
  const int s = choose_splits(M, N, K);
  return s > 1 ? align_up(size_t(s) * M * N * sizeof(float), 256) : 0;
}

// Fixes a product's splits (its partials at part).
void plan_splits(BwdGemm& p, float* part) {
  const int nkt = (p.K + kBK - 1) / kBK;
  const int splits = choose_splits(p.M, p.N, p.K);
  p.kt_per_split = std::max(1, (nkt + splits - 1) / splits);
  p.nsplit = std::max(1, (nkt + p.kt_per_split - 1) / p.kt_per_split);   // no empty split
  p.part = part;
}

// One product, or two with the same operand layouts in one launch (p1 with
// its partials after p0's), each followed by the split sums where split.
template <bool AKX, bool BKX, bool OUTF32>
hipError_t run2(BwdGemm p0, const BwdGemm* p1in, float* part, hipStream_t stream, const char* name) {
  plan_splits(p0, part);
  BwdGemm p1 = p0;
  int z1 = 0;
  if (p1in) {
    p1 = *p1in;
    plan_splits(p1, part + (p0.nsplit > 1 ? size_t(p0.nsplit) * p0.M * p0.N : 0));
    z1 = p1.nsplit;
  }
  auto tiles = [](const BwdGemm& p) { return ((p.N + kBT - 1) / kBT) * ((p.M + kBT - 1) / kBT); };
  const int gx = std::max(tiles(p0), p1in ? tiles(p1) : 0);
  ProfileScope ps(name, stream);
  hipLaunchKernelGGL((bwd_gemm_kernel<AKX, BKX, OUTF32>), dim3(gx, 1, p0.nsplit + z1), dim3(kThr), 0, stream, p0, p1,
                     p0.nsplit);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nq0 = p0.nsplit > 1 ? int64_t(p0.M) * (p0.N / 4) : 0;
  const int64_t nq1 = (p1in && p1.nsplit > 1) ? int64_t(p1.M) * (p1.N / 4) : 0;
  if (nq0 + nq1 == 0) return hipSuccess;
  if (nq0 == 0) {   // only p1 is split
    hipLaunchKernelGGL(split_reduce_kernel<OUTF32>, dim3(unsigned((nq1 + 255) / 256)), dim3(256), 0, stream, p1, p1,
                       nq1, nq1);
  } else {
    hipLaunchKernelGGL(split_reduce_kernel<OUTF32>, dim3(unsigned((nq0 + nq1 + 255) / 256)), dim3(256), 0, stream,
                       p0, p1, nq0, nq0 + nq1);
  }
  return hipGetLastError();
}

template <bool AKX, bool BKX, bool OUTF32>
hipError_t run(BwdGemm p, float* part, hipStream_t stream, const char* name) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  return run2<AKX, BKX, OUTF32>(p, nullptr, part, stream, name);
}

BwdGemm gemm(int M, int N, int K, const void* a, int64_t lda, const void* b, int64_t ldb, void* c, int64_t ldc,
             float alpha, const uint8_t* gate) {
  BwdGemm p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.k1 = K;
  p.a = p.a2 = static_cast<const uint16_t*>(a);
  p.lda = p.lda2 = lda;
  p.b = p.b2 = static_cast<const uint16_t*>(b);
  p.ldb = p.ldb2 = ldb;
  p.c = c;
  p.ldc = ldc;
  p.alpha = alpha;
  p.gate = gate;
  return p;
}

// dst[c][r] = src[r][c] for rows x cols bf16 matrices, one or two per launch
// (blockIdx.z): 64 x 64 tiles through LDS; 16-byte loads along src rows and
// 16-byte stores along dst rows where aligned and whole, single elements
// otherwise.
struct TransposeJob {
  const uint16_t* src;
  int64_t lds;
  uint16_t* dst;
  int64_t ldd;
  int rows, cols;
};

constexpr int kTPitch = 64 + 8;   // LDS row pitch (elements)

__global__ __launch_bounds__(256) void transpose_kernel(TransposeJob j0, TransposeJob j1) {
  __shared__ __align__(16) uint16_t tile[64 * kTPitch];
  const TransposeJob& j = blockIdx.z == 0 ? j0 : j1;
  const int tc = (j.cols + 63) / 64;
  if (int(blockIdx.x) >= tc * ((j.rows + 63) / 64)) return;
  const int r0 = (int(blockIdx.x) / tc) * 64, c0 = (int(blockIdx.x) % tc) * 64;
  const bool vsrc = (j.lds % 8 == 0) && ((reinterpret_cast<uintptr_t>(j.src) & 15u) == 0);
  const bool vdst = (j.ldd % 8 == 0) && ((reinterpret_cast<uintptr_t>(j.dst) & 15u) == 0);
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int q = threadIdx.x + 256 * rr;
    const int row = q >> 3, cc = (q & 7) * 8;
    const int r = r0 + row, c = c0 + cc;
    uint16_t v[8];
    if (r < j.rows && vsrc && c + 8 <= j.cols) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(j.src + int64_t(r) * j.lds + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = uint16_t(x[e] & 0xffffu);
        v[2 * e + 1] = uint16_t(x[e] >> 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (r < j.rows && c + e < j.cols) ? j.src[int64_t(r) * j.lds + c + e] : 0;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[row * kTPitch + cc + e] = v[e];
  }
  __syncthreads();
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int q = threadIdx.x + 256 * rr;
    const int orow = q >> 3, rc = (q & 7) * 8;   // dst row = src column c0 + orow
    const int c = c0 + orow, r = r0 + rc;
    if (c >= j.cols) continue;
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[(rc + e) * kTPitch + orow];
    uint16_t* d = j.dst + int64_t(c) * j.ldd + r;
    if (vdst && r + 8 <= j.rows) {
      u32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = uint32_t(v[2 * e]) | (uint32_t(v[2 * e + 1]) << 16);
      *reinterpret_cast<u32x4*>(d) = x;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (r + e < j.rows) d[e] = v[e];
    }
  }
}

hipError_t launch_transpose2(const TransposeJob& j0, const TransposeJob* j1, hipStream_t stream) {
  const TransposeJob& k1 = j1 ? *j1 : j0;
  auto tiles = [](const TransposeJob& j) { return int64_t((j.cols + 63) / 64) * ((j.rows + 63) / 64); };
  const int64_t gx = std::max(tiles(j0), tiles(k1));
  ProfileScope ps("uno_transpose", stream);
  hipLaunchKernelGGL(transpose_kernel, dim3(unsigned(gx), 1, j1 ? 2 : 1), dim3(256), 0, stream, j0, k1);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_transpose_bf16(const void* src, int64_t lds, void* dst, int64_t ldd, int64_t rows, int64_t cols,
                                 hipStream_t stream) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const TransposeJob j{static_cast<const uint16_t*>(src), lds, static_cast<uint16_t*>(dst), ldd, int(rows),
                       int(cols)};
  return launch_transpose2(j, nullptr, stream);
}

namespace {

// The products on the forward's kernels (see the file header); the adapter
// gradients stay on the generic kernel (fp32 outputs).
hipError_t launch_with_wt(const LoraBackwardArgs& a, uint16_t* u, uint16_t* dt, hipStream_t stream) {
  const int64_t M = a.M, N = a.N, K = a.K, r = a.r;
  char* ws = static_cast<char*>(a.ws) + 2 * align_up(size_t(M) * r * 2, 256);
  uint16_t* at = reinterpret_cast<uint16_t*>(ws);                        // A^T [K][r]
  ws += align_up(size_t(K) * r * 2, 256);
  uint16_t* bt = reinterpret_cast<uint16_t*>(ws);                        // B^T [r][N]
  ws += align_up(size_t(N) * r * 2, 256);
  float* part = reinterpret_cast<float*>(ws);
  const TransposeJob ja{static_cast<const uint16_t*>(a.a), a.lda, at, r, int(r), int(K)};
  const TransposeJob jb{static_cast<const uint16_t*>(a.b), a.ldb, bt, N, int(N), int(r)};
  hipError_t e = launch_transpose2(ja, &jb, stream);
  if (e != hipSuccess) return e;
  LoraDownArgs ld{};
  ld.M = M;
  ld.K = K;
  ld.n = r;
  ld.x = a.x;
  ld.ldx = a.ldx;
  ld.a = a.a;
  ld.lda = a.lda;
  ld.gate = a.gate;
  ld.lora_scale = 1.f;
  ld.t = u;
  ld.part = part;
  e = launch_lora_down(ld, stream);                                      // U = g (x A^T)
  if (e != hipSuccess) return e;
  ld.K = N;
  ld.x = a.dy;
  ld.ldx = a.lddy;
  ld.a = bt;
  ld.lda = N;
  ld.lora_scale = a.lora_scale;
  ld.t = dt;
  e = launch_lora_down(ld, stream);                                      // dT = s g (dY B)
  if (e != hipSuccess) return e;
  {   // dB and dA in one launch (same layouts)
    const BwdGemm gda = gemm(int(r), int(K), int(M), dt, r, a.x, a.ldx, a.da, a.ldda, 1.f, nullptr);
    e = run2<true, true, true>(gemm(int(N), int(r), int(M), a.dy, a.lddy, u, r, a.db, a.lddb, a.lora_scale, nullptr),
                               &gda, part, stream, "uno_lora_bwd_dadb");
  }
  if (e != hipSuccess || !a.dx) return e;
  GatedLoraArgs g{};                                                     // dx = dY W + dT A
  g.dtype = UNO_BF16;
  g.M = M;
  g.N = K;
  g.K = N;
  g.r = r;
  g.x = a.dy;
  g.ldx = a.lddy;
  g.w = a.w_t;
  g.ldw = a.ldwt;
  g.b = at;
  g.ldb = r;
  g.gate = a.gate;          // any non-NULL gate: the adapter columns are on (T is given)
  g.lora_scale = 1.f;
  g.y = a.dx;
  g.ldy = a.lddx;
  g.ws = part;
  g.t_pre = dt;
  g.ldt_pre = r;
  return launch_gated_lora(g, stream);
}

}  // namespace

size_t lora_backward_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r, int with_wt) {
  const int m = int(M), n = int(N), k = int(K), rr = int(r);
  size_t part = std::max({split_bytes(m, rr, k), split_bytes(m, rr, n), split_bytes(n, rr, m) + split_bytes(rr, k, m),
                          split_bytes(m, k, n + rr)});
  size_t extra = 0;
  if (with_wt) {   // A^T, B^T, the LoRA-down's and the main GEMM's partials
    extra = align_up(size_t(K) * r * 2, 256) + align_up(size_t(N) * r * 2, 256);
    part = std::max({part, lora_down_part_bytes(M, r, K), lora_down_part_bytes(M, r, N),
                     gated_lora_workspace_bytes(UNO_BF16, M, K, N, 0)});
  }
  return 2 * align_up(size_t(M) * r * 2, 256) + extra + part;
}

hipError_t launch_lora_backward(const LoraBackwardArgs& a, hipStream_t stream) {
  const int M = int(a.M), N = int(a.N), K = int(a.K), r = int(a.r);
  uint16_t* u = static_cast<uint16_t*>(a.ws);                                          // [M][r] bf16
  uint16_t* dt = reinterpret_cast<uint16_t*>(static_cast<char*>(a.ws) + align_up(size_t(M) * r * 2, 256));
  float* part = reinterpret_cast<float*>(static_cast<char*>(a.ws) + 2 * align_up(size_t(M) * r * 2, 256));
  // no gate: every row is a clean row, U = dT = 0 (written as 0 * the products)
  const uint8_t* gate = a.gate;
  const float on = gate ? 1.f : 0.f;
  hipError_t e;
  if (a.w_t && gate) return launch_with_wt(a, u, dt, stream);
  // U = g (x A^T): x "xk", A as the right-hand side B(k, j) = A[j][k] ("xk")
  e = run<false, false, false>(gemm(M, r, K, a.x, a.ldx, a.a, a.lda, u, r, on, gate), part, stream, "uno_lora_bwd_u");
  if (e != hipSuccess) return e;
  // dT = s g (dY B): dY "xk", B(k = n, j) = B[n][j] ("kx")
  e = run<false, true, false>(gemm(M, r, N, a.dy, a.lddy, a.b, a.ldb, dt, r, on * a.lora_scale, gate), part,
                              stream, "uno_lora_bwd_dt");
  if (e != hipSuccess) return e;
  // dB = s dY^T U: A(n, m) = dY[m][n] ("kx"), B(m, j) = U[m][j] ("kx")
  // dA = dT^T x: A(j, m) = dT[m][j] ("kx"), B(m, k) = x[m][k] ("kx"); one launch with dB
  {
    const BwdGemm gda = gemm(r, K, M, dt, r, a.x, a.ldx, a.da, a.ldda, 1.f, nullptr);
    e = run2<true, true, true>(gemm(N, r, M, a.dy, a.lddy, u, r, a.db, a.lddb, a.lora_scale, nullptr), &gda, part,
                               stream, "uno_lora_bwd_dadb");
  }
  if (e != hipSuccess) return e;
  if (!a.dx) return hipSuccess;
  // dx = [dY | dT] [W ; A]: A side "xk" in both segments, W(n, k) and A(j, k) "kx"
  BwdGemm p = gemm(M, K, N + r, a.dy, a.lddy, a.w, a.ldw, a.dx, a.lddx, 1.f, nullptr);
  p.k1 = N;
  p.a2 = dt;
  p.lda2 = r;
  p.b2 = static_cast<const uint16_t*>(a.a);
  p.ldb2 = a.lda;
  return run<false, true, false>(p, part, stream, "uno_lora_bwd_dx");
}

}  // namespace uno
