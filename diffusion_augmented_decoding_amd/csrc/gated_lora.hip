// Gated-LoRA linear layer for gfx950.
//
// Method: Uno summary (hyper.ai, arXiv 2609.04010), section "方法": LoRA
// adapters on every AR weight matrix; one forward over concatenated clean +
// noisy rows where a per-row mask switches the adapter off (clean/verify,
// AR weights only) or on (noisy/draft, AR + adapter weights).
//
//   y = x W^T + s * diag(g) (x A^T) B^T  =  [x | t] [W | B]^T,
//   t = s * diag(g) (x A^T)   (M x r, held as bf16)
//
// bf16 path, three launches on the caller's stream:
//  1. lora_down: split-K MFMA GEMM x A^T -> fp32 partials [splits][M][r];
//  2. lora_gate: t = bf16(s * g[m] * sum of partials); rows with g = 0 are
//     written as exact zeros, so they add exact zeros in step 3 (bit-identical
//     to the call without adapter);
//  3. gemm: one MFMA K-loop over the concatenated K + r columns, bf16 out.
// The gate is therefore folded into the producer of t; y is written once.
//
// GEMM kernel: BM x BN x 64 tiles, WM x WN waves, v_mfma_f32_32x32x16_bf16.
// The MFMA "A" operand is the weight tile (N side) and "B" the activation
// tile (M side), so each lane ends up owning 4 consecutive output columns per
// register group (8-byte bf16 / 16-byte fp32 stores).  Global -> register ->
// LDS double buffering with one barrier per K-tile; LDS rows are 128 B with
// the 16-byte chunk index XOR-swizzled by (row & 7), which makes the
// fragment reads (32 rows, same chunk) bank-conflict free.  Tiles are mapped
// to block ids so that the blocks one XCD runs (ids congruent mod 8) cover a
// contiguous band of N-tiles across all M-tiles: each weight tile is then
// fetched into one XCD's L2 and reused by every M-tile there.
#include "device_common.h"
#include "internal.h"

namespace uno {

namespace {

constexpr int kBK = 64;                  // K elements per tile (128 bytes per LDS row)
constexpr int kChunksPerRow = kBK / 8;   // 16-byte chunks per row

struct GemmParams {
  int M, N, K1, K2;                    // K1 columns from (x, w), then K2 from (t, b)
  const uint16_t* x; int64_t ldx;
  const uint16_t* w; int64_t ldw;
  const uint16_t* t; int64_t ldt;
  const uint16_t* b; int64_t ldb;
  int ktiles_per_split;                // K-tiles per split (blockIdx.y)
  int tiles_m, tiles_n;
  // output: bf16 y (mode 0) or fp32 partials [split][M][N] (mode 1)
  uint16_t* y; int64_t ldy;
  float* part;
};

__device__ __forceinline__ u32x4 load_chunk(const uint16_t* base, int64_t ld, int row, int nrows,
                                            int kc, const uint16_t* base2, int64_t ld2, int K1,
                                            int Ktot) {
  u32x4 z = {0u, 0u, 0u, 0u};
  if (row >= nrows || kc >= Ktot) return z;
  const uint16_t* p = (kc < K1) ? base + int64_t(row) * ld + kc : base2 + int64_t(row) * ld2 + (kc - K1);
  return *reinterpret_cast<const u32x4*>(p);
}

template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(WM * WN * kWave) void gemm_bf16_kernel(GemmParams p) {
  constexpr int NT = WM * WN * kWave;
  constexpr int TM = BM / WM, TN = BN / WN;        // wave tile
  constexpr int FM = TM / 32, FN = TN / 32;        // 32x32 fragments per wave
  constexpr int CH_A = BN * kChunksPerRow;         // weight-tile chunks
  constexpr int CH_B = BM * kChunksPerRow;         // activation-tile chunks
  constexpr int LA = (CH_A + NT - 1) / NT;
  constexpr int LB = (CH_B + NT - 1) / NT;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");

  extern __shared__ __align__(16) unsigned char smem[];
  // stage s: [BN rows of weights][BM rows of activations], 128 B per row
  constexpr int STAGE = (BN + BM) * kBK * 2;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid / kWave;
  const int wm = wave % WM, wn = wave / WM;

  // XCD-aware tile order: block id b runs on XCD b % 8; give each XCD a
  // contiguous range of (n-major, m-minor) tiles.
  const int ntiles = p.tiles_m * p.tiles_n;
  const int bid = blockIdx.x;
  int tile;
  if ((ntiles & 7) == 0) {
    tile = (bid & 7) * (ntiles >> 3) + (bid >> 3);
  } else {
    tile = bid;
  }
  const int tm = tile % p.tiles_m, tn = tile / p.tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;

  const int Ktot = p.K1 + p.K2;
  const int kt_total = (Ktot + kBK - 1) / kBK;
  const int kt_begin = blockIdx.y * p.ktiles_per_split;
  int kt_end = kt_begin + p.ktiles_per_split;
  if (kt_end > kt_total) kt_end = kt_total;

  f32x16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 ra[LA], rb[LB];

  auto gload = [&](int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int cid = tid + i * NT;
      const int row = cid / kChunksPerRow, c = cid % kChunksPerRow;
      ra[i] = (cid < CH_A) ? load_chunk(p.w, p.ldw, n0 + row, p.N, k0 + 8 * c, p.b, p.ldb, p.K1, Ktot)
                           : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int cid = tid + i * NT;
      const int row = cid / kChunksPerRow, c = cid % kChunksPerRow;
      rb[i] = (cid < CH_B) ? load_chunk(p.x, p.ldx, m0 + row, p.M, k0 + 8 * c, p.t, p.ldt, p.K1, Ktot)
                           : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&](int stage) {
    unsigned char* base = smem + stage * STAGE;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int cid = tid + i * NT;
      if (cid < CH_A) {
        const int row = cid / kChunksPerRow, c = cid % kChunksPerRow;
        *reinterpret_cast<u32x4*>(base + row * (kBK * 2) + ((c ^ (row & 7)) * 16)) = ra[i];
      }
    }
    unsigned char* bb = base + BN * kBK * 2;
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int cid = tid + i * NT;
      if (cid < CH_B) {
        const int row = cid / kChunksPerRow, c = cid % kChunksPerRow;
        *reinterpret_cast<u32x4*>(bb + row * (kBK * 2) + ((c ^ (row & 7)) * 16)) = rb[i];
      }
    }
  };

  const int lrow = lane & 31, lhalf = lane >> 5;
  if (kt_begin < kt_end) {
    gload(kt_begin);
    sstore(0);
    __syncthreads();
    for (int kt = kt_begin; kt < kt_end; ++kt) {
      const int cur = (kt - kt_begin) & 1;
      const bool more = kt + 1 < kt_end;
      if (more) gload(kt + 1);
      const unsigned char* As = smem + cur * STAGE;
      const unsigned char* Bs = As + BN * kBK * 2;
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        const int c = 2 * kk + lhalf;
        bf16x8 fa[FN], fb[FM];
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          const int row = wn * TN + i * 32 + lrow;
          fa[i] = *reinterpret_cast<const bf16x8*>(As + row * (kBK * 2) + ((c ^ (row & 7)) * 16));
        }
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          const int row = wm * TM + j * 32 + lrow;
          fb[j] = *reinterpret_cast<const bf16x8*>(Bs + row * (kBK * 2) + ((c ^ (row & 7)) * 16));
        }
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
          for (int j = 0; j < FM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
      if (more) sstore(cur ^ 1);
      __syncthreads();
    }
  }

  // epilogue: lane owns column m = lrow of each fragment, rows n = 8g + 4*lhalf + e
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int m = m0 + wm * TM + j * 32 + lrow;
    if (m >= p.M) continue;
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * TN + i * 32 + 8 * g + 4 * lhalf;
        const float v0 = acc[i][j][4 * g + 0], v1 = acc[i][j][4 * g + 1];
        const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
        if constexpr (MODE == 0) {
          uint16_t* dst = p.y + int64_t(m) * p.ldy + n;
          if (n + 3 < p.N) {
            uint32_t lo = pack_bf16x2(v0, v1), hi = pack_bf16x2(v2, v3);
            *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
          } else {
            const float vv[4] = {v0, v1, v2, v3};
            for (int e = 0; e < 4; ++e)
              if (n + e < p.N) dst[e] = f32_to_bf16(vv[e]);
          }
        } else {
          float* dst = p.part + (int64_t(blockIdx.y) * p.M + m) * p.N + n;
          if (n + 3 < p.N && (p.N & 3) == 0) {
            *reinterpret_cast<f32x4*>(dst) = f32x4{v0, v1, v2, v3};
          } else {
            const float vv[4] = {v0, v1, v2, v3};
            for (int e = 0; e < 4; ++e)
              if (n + e < p.N) dst[e] = vv[e];
          }
        }
      }
    }
  }
}

// t[m, j] = bf16(scale * g[m] * sum_s part[s][m][j]); exact 0 for g = 0.
__global__ __launch_bounds__(256) void lora_gate_kernel(const float* __restrict__ part, int splits, int M,
                                                        int r, const uint8_t* __restrict__ gate,
                                                        float scale, uint16_t* __restrict__ t) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= int64_t(M) * r) return;
  const int m = int(i / r);
  if (gate[m] == 0) {
    t[i] = 0;
    return;
  }
  float s = 0.f;
  for (int sp = 0; sp < splits; ++sp) s += part[int64_t(sp) * M * r + i];
  t[i] = f32_to_bf16(scale * s);
}

// ------------------------------------------------------------------ fp32 path
__global__ __launch_bounds__(256) void lora_down_f32_kernel(const float* __restrict__ x, int64_t ldx,
                                                            const float* __restrict__ a, int64_t lda,
                                                            const uint8_t* __restrict__ gate, float scale,
                                                            int M, int K, int r, float* __restrict__ t) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= int64_t(M) * r) return;
  const int m = int(i / r), j = int(i % r);
  if (gate[m] == 0) {
    t[i] = 0.f;
    return;
  }
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  int kk = 0;
  for (; kk + 3 < K; kk += 4)
    for (int e = 0; e < 4; ++e) s[e] = fmaf(x[int64_t(m) * ldx + kk + e], a[int64_t(j) * lda + kk + e], s[e]);
  for (; kk < K; ++kk) s[0] = fmaf(x[int64_t(m) * ldx + kk], a[int64_t(j) * lda + kk], s[0]);
  t[i] = scale * ((s[0] + s[1]) + (s[2] + s[3]));
}

__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ x, int64_t ldx,
                                                       const float* __restrict__ w, int64_t ldw,
                                                       const float* __restrict__ t,
                                                       const float* __restrict__ b, int64_t ldb,
                                                       int M, int N, int K, int r,
                                                       float* __restrict__ y, int64_t ldy) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= int64_t(M) * N) return;
  const int m = int(i / N), n = int(i % N);
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  int kk = 0;
  for (; kk + 3 < K; kk += 4)
    for (int e = 0; e < 4; ++e) s[e] = fmaf(x[int64_t(m) * ldx + kk + e], w[int64_t(n) * ldw + kk + e], s[e]);
  for (; kk < K; ++kk) s[0] = fmaf(x[int64_t(m) * ldx + kk], w[int64_t(n) * ldw + kk], s[0]);
  float acc = (s[0] + s[1]) + (s[2] + s[3]);
  if (t != nullptr) {
    float l = 0.f;
    for (int j = 0; j < r; ++j) l = fmaf(t[int64_t(m) * r + j], b[int64_t(n) * ldb + j], l);
    acc += l;    // g = 0 rows: t = 0 -> l = 0 exactly
  }
  y[int64_t(m) * ldy + n] = acc;
}

template <int BM, int BN, int WM, int WN, int MODE>
hipError_t run_gemm(GemmParams p, int splits, hipStream_t stream, const char* name) {
  auto kern = gemm_bf16_kernel<BM, BN, WM, WN, MODE>;
  const size_t lds = 2 * size_t(BN + BM) * kBK * 2;
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    configured = true;
  }
  p.tiles_m = (p.M + BM - 1) / BM;
  p.tiles_n = (p.N + BN - 1) / BN;
  const int kt_total = (p.K1 + p.K2 + kBK - 1) / kBK;
  p.ktiles_per_split = (kt_total + splits - 1) / splits;
  dim3 grid(p.tiles_m * p.tiles_n, splits);
  ProfileScope ps(name, stream);
  hipLaunchKernelGGL(kern, grid, dim3(WM * WN * kWave), lds, stream, p);
  return hipGetLastError();
}

int lora_down_splits(int64_t M, int64_t r, int64_t K) {
  const int64_t tiles = ((M + 63) / 64) * ((r + 63) / 64);
  int64_t s = (256 + tiles - 1) / tiles;
  const int64_t kt = (K + kBK - 1) / kBK;
  if (s > kt / 2) s = kt / 2;
  if (s < 1) s = 1;
  if (s > 16) s = 16;
  return int(s);
}

}  // namespace

size_t gated_lora_workspace_bytes(uno_dtype dtype, int64_t M, int64_t N, int64_t K, int64_t r) {
  (void)N;
  if (r == 0) return 0;
  if (dtype == UNO_F32) return align_up(size_t(M) * size_t(r) * 4, 256);
  const int s = lora_down_splits(M, r, K);
  return align_up(size_t(M) * size_t(r) * 2, 256) + align_up(size_t(s) * size_t(M) * size_t(r) * 4, 256);
}

hipError_t launch_gated_lora(const GatedLoraArgs& a, hipStream_t stream) {
  const bool lora = a.r > 0 && a.gate != nullptr;
  if (a.dtype == UNO_F32) {
    float* t = nullptr;
    if (lora) {
      t = static_cast<float*>(a.ws);
      const int64_t n = a.M * a.r;
      ProfileScope ps("uno_lora_down_f32", stream);
      hipLaunchKernelGGL(lora_down_f32_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream,
                         static_cast<const float*>(a.x), a.ldx, static_cast<const float*>(a.a), a.lda,
                         a.gate, a.lora_scale, int(a.M), int(a.K), int(a.r), t);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    const int64_t n = a.M * a.N;
    ProfileScope ps("uno_gemm_f32", stream);
    hipLaunchKernelGGL(gemm_f32_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const float*>(a.x), a.ldx, static_cast<const float*>(a.w), a.ldw, t,
                       static_cast<const float*>(a.b), a.ldb, int(a.M), int(a.N), int(a.K),
                       lora ? int(a.r) : 0, static_cast<float*>(a.y), a.ldy);
    return hipGetLastError();
  }

  uint16_t* t = nullptr;
  if (lora) {
    const int splits = lora_down_splits(a.M, a.r, a.K);
    t = static_cast<uint16_t*>(a.ws);
    float* part = reinterpret_cast<float*>(static_cast<char*>(a.ws) + align_up(size_t(a.M) * a.r * 2, 256));
    GemmParams d{};
    d.M = int(a.M);
    d.N = int(a.r);
    d.K1 = int(a.K);
    d.K2 = 0;
    d.x = static_cast<const uint16_t*>(a.x);
    d.ldx = a.ldx;
    d.w = static_cast<const uint16_t*>(a.a);
    d.ldw = a.lda;
    d.part = part;
    hipError_t e = run_gemm<64, 64, 2, 2, 1>(d, splits, stream, "uno_lora_down_bf16");
    if (e != hipSuccess) return e;
    const int64_t n = a.M * a.r;
    {
      ProfileScope ps("uno_lora_gate", stream);
      hipLaunchKernelGGL(lora_gate_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, part,
                         splits, int(a.M), int(a.r), a.gate, a.lora_scale, t);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  GemmParams g{};
  g.M = int(a.M);
  g.N = int(a.N);
  g.K1 = int(a.K);
  g.K2 = lora ? int(a.r) : 0;
  g.x = static_cast<const uint16_t*>(a.x);
  g.ldx = a.ldx;
  g.w = static_cast<const uint16_t*>(a.w);
  g.ldw = a.ldw;
  g.t = t;
  g.ldt = a.r;
  g.b = static_cast<const uint16_t*>(a.b);
  g.ldb = a.ldb;
  g.y = static_cast<uint16_t*>(a.y);
  g.ldy = a.ldy;
  return run_gemm<128, 128, 2, 2, 0>(g, 1, stream, "uno_gemm_bf16");
}

}  // namespace uno
