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
// bf16 path, launches on the caller's stream:
//  1. lora_down: split-K MFMA GEMM x A^T -> fp32 partials [splits][M][r];
//  2. lora_gate: t = bf16(s * g[m] * sum of partials); rows with g = 0 are
//     written as exact zeros, so they add exact zeros in step 3 (bit-identical
//     to the call without adapter);
//  3. gemm: one MFMA K-loop over the concatenated K + r columns; bf16 out, or
//     fp32 split-K partials followed by 4. gemm_reduce (fixed summation order).
// The gate is therefore folded into the producer of t; y is written once.
//
// GEMM kernel: BM x BN x 64 tiles, WM x WN waves, v_mfma_f32_32x32x16_bf16.
// The MFMA "A" operand is the weight tile (N side) and "B" the activation
// tile (M side), so each lane ends up owning 4 consecutive output columns per
// register group (8-byte bf16 / 16-byte fp32 stores).  Global -> register ->
// LDS double buffering with one barrier per K-tile; the LDS stores of the
// next tile are spread over the four 16-deep k-steps of the current one so
// they overlap the MFMAs.  Global loads are branch-free (always from a valid
// address, then masked), so all of a thread's loads issue back to back.  LDS
// rows are 128 B with the 16-byte chunk index XOR-swizzled by (row & 7),
// which makes the fragment reads (32 rows, same chunk) bank-conflict free.
// Tiles are mapped to block ids so that the blocks one XCD runs (ids
// congruent mod 8) form a contiguous band, and the band is ordered in groups
// of 8 M-tiles by all N-tiles: the workgroups an XCD runs at once then share
// both their weight and their activation tiles in that XCD's L2.  A second
// kernel, gemm_dl_kernel, loads K-tiles straight into LDS (global_load_lds)
// through a deeper stage ring; the dispatcher picks per shape whichever
// measured faster (the LoRA-down at 4096 rows runs on it).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace uno {

namespace {

constexpr int kBK = 64;                  // K elements per tile (128 bytes per LDS row)
constexpr int kChunksPerRow = kBK / 8;   // 16-byte chunks per row

struct GemmParams {
  int M, N, K1, K2;                    // K1 columns from (x, w), then K2 from (t, b)
  const uint16_t* x; int64_t ldx;      // activation rows (M side)
  const uint16_t* w; int64_t ldw;      // weight rows (N side)
  const uint16_t* t; int64_t ldt;
  const uint16_t* b; int64_t ldb;
  int ktiles_per_split;                // K-tiles per split (blockIdx.y)
  int tiles_m, tiles_n;
  int xcd_remap;                       // map block ids so one XCD runs a contiguous tile band
  uint16_t* y; int64_t ldy;            // MODE 0 output
  int y_vec;                           // 8-byte stores allowed (ldy % 4 == 0, y 8-byte aligned)
  float* part;                         // MODE 1 output: fp32 [split][M][N]
  const uint16_t* w2;                  // MODE 2: up-projection weights (gate in w), ld ldw
  const uint16_t* b2;                  // MODE 2: up-projection adapter B (gate in b), ld ldb
  int kr;                              // MODE 2: K-tiles per adapter (r / 64); t = [t_gate | t_up]
  // MODE 0, two segments: output columns from seg_n on come from (w2, b2, t +
  // t2_off) and go to y2 (same ldy), column n - seg_n; 0 = one segment
  int seg_n;
  int64_t t2_off;
  uint16_t* y2;
  // Gate-merged weights (MODE 0 and 2, FAST, no adapter columns): logical
  // rows m >= merge_m (the gated rows) read wm / wm2, the copies of w / w2 with
  // the adapter merged in (W + s B A); rows below merge_m read w / w2.  With
  // row_blk > 0 the logical rows are gathered: row m < merge_m is physical
  // row (m / row_blk) * 2 row_blk + m % row_blk (the first row_blk rows of
  // every 2 row_blk, the clean rows), row merge_m + i is physical row
  // (i / row_blk) * 2 row_blk + row_blk + i % row_blk (the noisy rows), for
  // the activations and the output alike.  0: off.
  int merge_m;
  int row_blk;
  const uint16_t* wm;
  const uint16_t* wm2;
  // LoRA-down (gemm_dl_kernel) only: > 0 gathers the x rows, logical row i
  // reading physical row (i / g) * 2g + g + i % g (the noisy rows of
  // sequences of g clean + g noisy rows); the partials stay in logical rows
  int gather_blk;
};

// Physical row of logical row m under the gate-merged row order.
__device__ __forceinline__ int phys_row(const GemmParams& p, int m) {
  if (p.row_blk <= 0) return m;
  const bool gated = m >= p.merge_m;
  const int i = gated ? m - p.merge_m : m;
  return (i / p.row_blk) * 2 * p.row_blk + (gated ? p.row_blk : 0) + i % p.row_blk;
}

// Output tile of linear index `tile`.  Mode 1: column-major (M-tiles
// fastest), so the contiguous band of tiles one XCD runs spans few N-tiles
// and every M-tile.  Mode 2: groups of 8 M-tiles, N-tiles across the group,
// so an XCD's band (and the workgroups it runs at once) is a 2D block of
// M- and N-tiles that share both operands in that XCD's L2.
__device__ __forceinline__ void tile_coords(const GemmParams& p, int tile, int& tm, int& tn) {
  if (p.xcd_remap == 2 && p.tiles_m >= 8) {
    const int gsz = 8 * p.tiles_n;
    const int g = tile / gsz, rem = tile - g * gsz;
    const int gm = min(8, p.tiles_m - 8 * g);   // rows in this (possibly partial) group
    tm = 8 * g + rem % gm;
    tn = rem / gm;
  } else {
    tm = tile % p.tiles_m;
    tn = tile / p.tiles_m;
  }
}

// 16-byte chunk (8 bf16 along K) at K index kc of a row: from (base, ld) for
// kc < K1, from (base2, ld2) at kc - K1 below Ktot.  Out-of-range chunks read
// `base` instead (always valid) and are zeroed later, when written to LDS:
// masking here would consume the value and force a wait on the load.
__device__ __forceinline__ u32x4 load_chunk_raw(const uint16_t* base, int64_t ld, const uint16_t* base2,
                                                int64_t ld2, int row, bool ok, int kc, int K1) {
  const bool first = kc < K1;
  const uint16_t* p = first ? base + int64_t(row) * ld + kc : base2 + int64_t(row) * ld2 + (kc - K1);
  p = ok ? p : base;
  return *reinterpret_cast<const u32x4*>(p);
}

// K-tiles [kt_begin, kt_end) of split blockIdx.y: the splits divide the
// tiles of the first K1 columns; the last split also takes the adapter
// columns.  A row whose adapter input is zero therefore sums exactly the same
// partial products, split by split, as the call without adapter.
__device__ __forceinline__ void split_range(const GemmParams& p, int bk, int kt_total, int& kt_begin, int& kt_end) {
  const int kt1 = (p.K1 + bk - 1) / bk;
  const int y = blockIdx.y;
  kt_begin = min(y * p.ktiles_per_split, kt1);
  kt_end = (y + 1 == int(gridDim.y)) ? kt_total : min((y + 1) * p.ktiles_per_split, kt1);
}

// BM x BN block tile, WM x WN waves, P K-tiles of register prefetch, DBF:
// 1 = double-buffer the MFMA fragments across k-steps, 2 = defer each
// K-tile's last k-step across the barrier (below), MODE: 0 = bf16 out,
// 1 = fp32 split-K partials, 2 = SwiGLU of a gate and an up projection
// (below).
// MODE 2 (FAST only, BN = 256 on 8 waves): a block tile covers BN / 2
// features of both projections.  Its weight rows come in four bands of 64:
// gate rows of features n0 .. n0 + 63, up rows of the same features, then the
// same for n0 + 64 .. n0 + 127, so each wave's 128 rows hold 64 gate and the
// 64 matching up rows, and fragment i + FN / 2 of a lane sits at the same
// feature as fragment i.  The adapter columns run over t = [t_gate | t_up]
// (2r of them): gate rows read B_gate against t_gate and zeros (buffer reads
// past the end) against t_up, up rows the reverse.  The epilogue writes
// bf16(silu(g) * u) from the fp32 accumulators.
// FAST: every K-tile is whole (K1 and K2 multiples of 64) and every operand
// spans < 2 GB, so tiles are read with buffer loads: a per-lane row offset
// fixed for the whole K loop plus a scalar offset (chunk group, K-tile), with
// rows past M / N and K-tiles past the split falling outside the buffer and
// reading zeros.  No per-load address arithmetic or masking is left in the
// loop, and the LDS slot of each chunk is a fixed offset.
template <int BM, int BN, int WM, int WN, int P, int DBF, int MODE, int FAST>
__global__ __launch_bounds__(WM * WN * kWave) void gemm_bf16_kernel(GemmParams p_in) {
  GemmParams p = p_in;
  constexpr int NT = WM * WN * kWave;
  constexpr int TM = BM / WM, TN = BN / WN;        // wave tile
  constexpr int FM = TM / 32, FN = TN / 32;        // 32x32 fragments per wave
  constexpr int CH_A = BN * kChunksPerRow;         // weight-tile chunks
  constexpr int CH_B = BM * kChunksPerRow;         // activation-tile chunks
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(CH_A % NT == 0 && CH_B % NT == 0, "tile chunks must divide among threads");
  constexpr int LA = CH_A / NT, LB = CH_B / NT, LT = LA + LB;
  constexpr int STAGE = (BN + BM) * kBK * 2;

  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid / kWave;
  const int wm = wave % WM, wn = wave / WM;

  const int ntiles = p.tiles_m * p.tiles_n;
  const int bid = blockIdx.x;
  const int tile = (p.xcd_remap && (ntiles & 7) == 0) ? (bid & 7) * (ntiles >> 3) + (bid >> 3) : bid;
  int tm, tn;
  tile_coords(p, tile, tm, tn);
  static_assert(MODE != 2 || (FAST && BN == 256 && WM * WN == 8), "SwiGLU tiles: 256 weight rows, 8 waves");
  static_assert(MODE >= 0 && MODE <= 2, "modes of the main kernel: bf16 out, partials, SwiGLU");
  const int m0 = tm * BM;
  int n0 = tn * (MODE == 2 ? BN / 2 : BN);   // MODE 2: first feature of the tile
  if constexpr (FAST && MODE != 1) {
    // gated rows (tiles never straddle merge_m): the merged weights
    if (p.merge_m > 0 && m0 >= p.merge_m) {
      p.w = p.wm;
      p.w2 = p.wm2;
    }
  }
  if constexpr (MODE == 0 && FAST) {
    // two segments (tiles never straddle seg_n): rebase onto the second
    if (p.seg_n > 0) {
      if (n0 >= p.seg_n) {
        p.w = p.w2;
        p.b = p.b2;
        p.t = p.t + p.t2_off;
        p.y = p.y2;
        n0 -= p.seg_n;
        p.N -= p.seg_n;
      } else {
        p.N = p.seg_n;
      }
    }
  }

  const int Ktot = p.K1 + p.K2;
  const int kt_total = (Ktot + kBK - 1) / kBK;
  int kt_begin, kt_end;
  split_range(p, kBK, kt_total, kt_begin, kt_end);

  f32x16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Chunk i of this thread (A chunks first, then B): tile row and 16-byte
  // column.  reg[s] is one of P register sets holding a K-tile in flight:
  // K-tile j is loaded P iterations before it is stored to LDS, so each
  // global load has P compute phases to land.
  u32x4 reg[P][LT];
  auto chunk_row = [&](int i) { return ((i < LA ? i : i - LA) * NT + tid) / kChunksPerRow; };
  auto chunk_col = [&](int i) { return ((i < LA ? i : i - LA) * NT + tid) % kChunksPerRow; };

  // K-tiles outside [kt_begin, kt_end) are never stored; their loads read the
  // (cached) matrix base so every iteration issues the same loads, which lets
  // the compiler count outstanding loads exactly instead of draining them.
  auto chunk_ok = [&](int i, int kt) {
    const int row = chunk_row(i), kc = kt * kBK + 8 * chunk_col(i);
    return (i < LA ? (n0 + row < p.N) : (m0 + row < p.M)) && kc < Ktot && kt < kt_end;
  };
  auto gload1 = [&](u32x4 (&dst)[LT], int i, int kt) {
    const int row = chunk_row(i), c = chunk_col(i);
    const bool ok = chunk_ok(i, kt);
    if (i < LA)
      dst[i] = load_chunk_raw(p.w, p.ldw, p.b, p.ldb, n0 + row, ok, kt * kBK + 8 * c, p.K1);
    else
      dst[i] = load_chunk_raw(p.x, p.ldx, p.t, p.ldt, m0 + row, ok, kt * kBK + 8 * c, p.K1);
  };
  // LDS byte offset of 16-byte chunk c of tile row `row`: the chunk index is
  // XOR-swizzled by row so that the 8 (or 16) rows one ds_read_b128 phase
  // touches land in distinct banks under a 32- or a 64-bank LDS
  auto lds_off = [](int row, int c) { return row * (kBK * 2) + ((c ^ (row & 7) ^ ((row >> 3) & 1)) * 16); };
  // write chunk i of a register set holding K-tile kt, zeroing invalid chunks
  auto sstore_slow = [&](const u32x4 (&src)[LT], int stage, int i, int kt) {
    const int row = chunk_row(i), c = chunk_col(i);
    unsigned char* base = smem + stage * STAGE + (i < LA ? 0 : BN * kBK * 2);
    const u32x4 v = chunk_ok(i, kt) ? src[i] : u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(base + lds_off(row, c)) = v;
  };

  // ---- FAST addressing (see above): chunk i covers tile rows
  // (i mod side) * NT/8 + tid/8, 16-byte column tid % 8 of the K-tile
  constexpr int RPG = NT / kChunksPerRow;          // tile rows per chunk group
  static_assert(!FAST || (RPG % 16 == 0), "the LDS swizzle must not depend on the chunk group");
  // (buffer descriptors are built unconditionally: the non-FAST path ignores them)
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.w), 0, int(int64_t(p.N) * p.ldw * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.b), 0, int(int64_t(p.N) * p.ldb * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.x), 0, int(int64_t(p.M) * p.ldx * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rt =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.t), 0, int(int64_t(p.M) * p.ldt * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw2 =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.w2), 0, int(int64_t(p.N) * p.ldw * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb2 =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.b2), 0, int(int64_t(p.N) * p.ldb * 2), 0x00020000);
  uint32_t va1 = 0, va2 = 0, vb1 = 0, vb2 = 0, slot = 0;
  int kt1 = 0;
  if constexpr (FAST) {
    const uint32_t col = uint32_t(tid % kChunksPerRow) * 16;
    const int trow = tid / kChunksPerRow;
    va1 = uint32_t((n0 + trow) * p.ldw * 2) + col;
    va2 = uint32_t((n0 + trow) * p.ldb * 2) + col;
    vb1 = uint32_t(phys_row(p, m0 + trow) * p.ldx * 2) + col;
    vb2 = uint32_t((m0 + trow) * p.ldt * 2) + col;
    slot = uint32_t(lds_off(trow, tid % kChunksPerRow));
    kt1 = p.K1 / kBK;
  }
  auto gload_fast = [&](u32x4 (&dst)[LT], int i, int kt) {
    // every choice below is wave-uniform; the descriptors are never selected
    // at run time (a selected descriptor would need a readfirstlane loop)
    const bool live = kt < kt_end;
    const bool first = kt < kt1;
    const int q = i < LA ? i : i - LA;
    const int ktl = first ? kt : kt - kt1;
    if (i < LA && MODE == 2) {
      // chunk group i: band i / 2 (features n0 + 64 (i / 2) ..), gate rows for
      // even i, up rows for odd i; an adapter K-tile belongs to the gate
      // (ktl < kr) or to the up projection, the other rows read zeros
      const bool up = (i & 1) != 0;
      const bool half = ktl >= p.kr;
      const bool valid = first || (half == up);
      const int step = first ? RPG * int(p.ldw) * 2 : RPG * int(p.ldb) * 2;
      const int kcol = (first || !half) ? ktl : ktl - p.kr;
      uint32_t off = (first ? va1 : va2) + uint32_t((i >> 1) * step + kcol * kBK * 2);
      off = (live && valid) ? off : 0x80000000u;
      if (up)
        dst[i] = __builtin_bit_cast(u32x4, first ? __builtin_amdgcn_raw_buffer_load_b128(rw2, off, 0, 0)
                                                 : __builtin_amdgcn_raw_buffer_load_b128(rb2, off, 0, 0));
      else
        dst[i] = __builtin_bit_cast(u32x4, first ? __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0)
                                                 : __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0));
    } else if (i < LA) {
      const int step = first ? RPG * int(p.ldw) * 2 : RPG * int(p.ldb) * 2;
      uint32_t off = (first ? va1 : va2) + uint32_t(q * step + ktl * kBK * 2);
      off = live ? off : 0x80000000u;   // past the split: out of range, reads 0
      dst[i] = __builtin_bit_cast(u32x4, first ? __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0)
                                               : __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0));
    } else {
      // gathered rows: RPG is a multiple of row_blk, so RPG logical rows
      // further on are 2 RPG physical rows further on
      const int step = first ? RPG * int(p.ldx) * (p.row_blk > 0 ? 4 : 2) : RPG * int(p.ldt) * 2;
      uint32_t off = (first ? vb1 : vb2) + uint32_t(q * step + ktl * kBK * 2);
      off = live ? off : 0x80000000u;
      dst[i] = __builtin_bit_cast(u32x4, first ? __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0)
                                               : __builtin_amdgcn_raw_buffer_load_b128(rt, off, 0, 0));
    }
  };
  auto sstore_fast = [&](const u32x4 (&src)[LT], int stage, int i) {
    const int q = i < LA ? i : i - LA;
    unsigned char* base = smem + stage * STAGE + (i < LA ? 0 : BN * kBK * 2) + q * RPG * kBK * 2;
    *reinterpret_cast<u32x4*>(base + slot) = src[i];
  };
  auto sstore = [&](const u32x4 (&src)[LT], int stage, int i, int kt) {
    if constexpr (FAST)
      sstore_fast(src, stage, i);
    else
      sstore_slow(src, stage, i, kt);
  };
  auto gload = [&](u32x4 (&dst)[LT], int i, int kt) {
    if constexpr (FAST)
      gload_fast(dst, i, kt);
    else
      gload1(dst, i, kt);
  };

  const int lrow = lane & 31, lhalf = lane >> 5;
  auto read_frags = [&](const unsigned char* As, const unsigned char* Bs, int kk, bf16x8 (&fa)[FN],
                        bf16x8 (&fb)[FM]) {
    const int c = 2 * kk + lhalf;
#pragma unroll
    for (int i = 0; i < FN; ++i)
      fa[i] = *reinterpret_cast<const bf16x8*>(As + lds_off(wn * TN + i * 32 + lrow, c));
#pragma unroll
    for (int j = 0; j < FM; ++j)
      fb[j] = *reinterpret_cast<const bf16x8*>(Bs + lds_off(wm * TM + j * 32 + lrow, c));
  };
  // Compute one K-tile from LDS stage `cur`.  Interleaved with its MFMAs:
  // the fragments of the next k-step (double-buffered), and chunk by chunk
  // the LDS store of register set `set` (K-tile kt_next, into the other
  // stage) followed, when RELOAD, by the load of K-tile kt_reload into the
  // chunk just freed.  Stores past the last K-tile write zeros into the
  // stage nobody reads again, which keeps each k-step one basic block.
  auto compute = [&](auto reload_tag, int cur, u32x4 (&set)[LT], int kt_next, int kt_reload) {
    constexpr bool RELOAD = decltype(reload_tag)::value;
    const unsigned char* As = smem + cur * STAGE;
    const unsigned char* Bs = As + BN * kBK * 2;
    constexpr int NB = DBF ? 2 : 1;
    bf16x8 fa[NB][FN], fb[NB][FM];
    if constexpr (DBF) read_frags(As, Bs, 0, fa[0], fb[0]);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int fb_cur = DBF ? (kk & 1) : 0;
      if constexpr (DBF) {
        if (kk + 1 < kBK / 16) read_frags(As, Bs, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
      } else {
        read_frags(As, Bs, kk, fa[0], fb[0]);
      }
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[fb_cur][i], fb[fb_cur][j], acc[i][j], 0, 0, 0);
#pragma unroll
      for (int i = kk * LT / 4; i < (kk + 1) * LT / 4; ++i) {
        sstore(set, cur ^ 1, i, kt_next);
        if constexpr (RELOAD) gload(set, i, kt_reload);
      }
      // one MFMA, then one of each pending memory op, repeated
      const int nr = DBF ? ((kk + 1 < kBK / 16) ? FN + FM : 0) : 0;
      const int nw = (kk + 1) * LT / 4 - kk * LT / 4;
#pragma unroll
      for (int q = 0; q < FN * FM; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (q < nr) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (q < nw) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        if (RELOAD && q < nw) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
  };

  // DBF == 2: the last k-step of a K-tile is deferred across the barrier.
  // Its fragments are read into (da, db) with the third k-step's, under that
  // k-step's MFMAs (so the stage may be overwritten once the barrier is
  // passed), and its MFMAs are issued after the barrier, under the reads of
  // the next K-tile's first k-step: the matrix pipe stays busy while those
  // reads are in flight, where the other form waits for them after every
  // barrier.  The LDS stores of the next K-tile are spread over the first
  // three k-steps.  The k-steps of every accumulator keep their order, so the
  // results are the other form's bit for bit.
  bf16x8 da[FN], db[FM];
  auto mfma_frags = [&](const bf16x8 (&fa)[FN], const bf16x8 (&fb)[FM]) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };
  auto compute_def = [&](auto def_tag, int cur, u32x4 (&set)[LT], int kt_next, int kt_reload) {
    constexpr bool DEF = decltype(def_tag)::value;
    constexpr int KS = kBK / 16;
    const unsigned char* As = smem + cur * STAGE;
    const unsigned char* Bs = As + BN * kBK * 2;
    bf16x8 fa[FN], fb[FM];
#pragma unroll
    for (int kk = 0; kk + 1 < KS; ++kk) {
      read_frags(As, Bs, kk, fa, fb);
      // the deferred k-step's reads go out with the last undeferred
      // k-step's, under its MFMAs
      if (kk + 2 == KS) read_frags(As, Bs, KS - 1, da, db);
      if (DEF && kk == 0) mfma_frags(da, db);
      mfma_frags(fa, fb);
#pragma unroll
      for (int i = kk * LT / (KS - 1); i < (kk + 1) * LT / (KS - 1); ++i) {
        sstore(set, cur ^ 1, i, kt_next);
        gload(set, i, kt_reload);
      }
      const int nw = (kk + 1) * LT / (KS - 1) - kk * LT / (KS - 1);
      if (DEF && kk == 0) {
        // the reads first, then the deferred MFMAs, then this k-step's
        __builtin_amdgcn_sched_group_barrier(0x100, FN + FM, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, FN * FM, 0);
      }
      if (kk + 2 == KS) __builtin_amdgcn_sched_group_barrier(0x100, 2 * (FN + FM), 0);
#pragma unroll
      for (int q = 0; q < FN * FM; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (q < nw) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        if (q < nw) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
  };
  static_assert(DBF != 2 || P == 1, "the deferred k-step form keeps one K-tile of register prefetch");

  if constexpr (DBF == 2) {
    if (kt_begin < kt_end) {
#pragma unroll
      for (int i = 0; i < LT; ++i) gload(reg[0], i, kt_begin);
#pragma unroll
      for (int i = 0; i < LT; ++i) {
        sstore(reg[0], 0, i, kt_begin);
        gload(reg[0], i, kt_begin + 1);
      }
      __syncthreads();
      compute_def(std::false_type{}, 0, reg[0], kt_begin + 1, kt_begin + 2);
      __syncthreads();
      for (int kt = kt_begin + 1; kt < kt_end; ++kt) {
        compute_def(std::true_type{}, (kt - kt_begin) & 1, reg[0], kt + 1, kt + 2);
        __syncthreads();
      }
      mfma_frags(da, db);
    }
  } else if (kt_begin < kt_end) {
    // prologue: K-tiles kt_begin .. kt_begin+P-1 into sets 0..P-1; tile 0 to LDS
#pragma unroll
    for (int s = 0; s < P; ++s)
#pragma unroll
      for (int i = 0; i < LT; ++i) gload(reg[s], i, kt_begin + s);
#pragma unroll
    for (int i = 0; i < LT; ++i) {
      sstore(reg[0], 0, i, kt_begin);
      gload(reg[0], i, kt_begin + P);
    }
    __syncthreads();
    // invariant at iteration t (K-tile kt = kt_begin + t): LDS stage t & 1 holds
    // tile kt; set (t + 1 + j) % P holds tile kt + 1 + j, j = 0..P-1
    int kt0 = kt_begin;
    for (; kt0 + P <= kt_end; kt0 += P) {
#pragma unroll
      for (int u = 0; u < P; ++u) {
        const int kt = kt0 + u;
        compute(std::true_type{}, (kt - kt_begin) & 1, reg[(u + 1) % P], kt + 1, kt + 1 + P);
        __syncthreads();
      }
    }
    // tail: fewer than P K-tiles left, all already in registers
#pragma unroll
    for (int u = 0; u + 1 < P; ++u) {
      const int kt = kt0 + u;
      if (kt < kt_end) {
        compute(std::false_type{}, (kt - kt_begin) & 1, reg[(u + 1) % P], kt + 1, 0);
        __syncthreads();
      }
    }
  }

  if constexpr (MODE == 2) {
    // fragment i (gate) and i + FN / 2 (up) of a lane hold the same features
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int m = m0 + wm * TM + j * 32 + lrow;
      if (m >= p.M) continue;
#pragma unroll
      for (int i = 0; i < FN / 2; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * (TN / 2) + i * 32 + 8 * g + 4 * lhalf;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float gv = acc[i][j][4 * g + e], uv = acc[i + FN / 2][j][4 * g + e];
            o[e] = gv / (1.f + expf(-gv)) * uv;
          }
          uint16_t* dst = p.y + int64_t(phys_row(p, m)) * p.ldy + n;
          if (p.y_vec && n + 3 < p.N) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
          } else {
            for (int e = 0; e < 4; ++e)
              if (n + e < p.N) dst[e] = f32_to_bf16(o[e]);
          }
        }
      }
    }
    return;
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
          uint16_t* dst = p.y + int64_t(phys_row(p, m)) * p.ldy + n;
          if (p.y_vec && n + 3 < p.N) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
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

// ------------------------------------------------------------------
// Direct-to-LDS variant: K-tiles of 32 (64-byte LDS rows) move from global
// memory straight into LDS with global_load_lds_dwordx4 (no register staging,
// no LDS store instructions), S stages deep, so S - 1 K-tiles are in flight
// while one is computed.  One wave instruction fills 1 KB of LDS (lane l at
// byte 16 l), i.e. 16 rows x 4 chunks; each lane therefore loads the global
// chunk whose swizzled LDS slot it fills.  Chunks past K (or of K-tiles past
// the split) read a zero block; rows past M / N read the last valid row (their
// outputs are never stored).  The 64-byte-row swizzle, chunk c of row r at
// c ^ ((r >> 1) & 3) ^ ((r >> 3) & 1), keeps the fragment reads conflict-free
// for both 8- and 16-lane LDS phases.
constexpr int kBKd = 32;                  // K elements per direct-load K-tile

__device__ __align__(16) const uint32_t kZeroChunk[4] = {0u, 0u, 0u, 0u};

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int BM, int BN, int WM, int WN, int S, int MODE>
__global__ __launch_bounds__(WM * WN * kWave) void gemm_dl_kernel(GemmParams p) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int ROWS = BN + BM;                         // LDS rows per stage (weights first)
  constexpr int BLKS = (ROWS + 15) / 16;                // 1 KB wave-instruction blocks of real rows
  constexpr int LPW = (BLKS + NW - 1) / NW;             // load instructions per wave per stage
  constexpr int STAGE = LPW * NW * 1024;                // bytes (blocks past BLKS are padding)
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(BN % 16 == 0 && BM % 16 == 0, "tile rows come in 16-row blocks");
  static_assert(S >= 3, "the pipeline keeps two stages ahead of the one computed");
  static_assert(MODE >= 0 && MODE <= 2, "modes: bf16 out, partials, SwiGLU");

  extern __shared__ __align__(16) unsigned char smem_raw[];
  // the LDS base as an opaque value: the optimizer cannot tell which LDS bytes
  // the direct loads write, so it keeps every LDS read
  uint32_t lds_base = uint32_t(reinterpret_cast<uintptr_t>(smem_raw));
  asm volatile("" : "+s"(lds_base));

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave % WM, wn = wave / WM;

  const int ntiles = p.tiles_m * p.tiles_n;
  const int bid = blockIdx.x;
  const int tile = (p.xcd_remap && (ntiles & 7) == 0) ? (bid & 7) * (ntiles >> 3) + (bid >> 3) : bid;
  int tm, tn;
  tile_coords(p, tile, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int Ktot = p.K1 + p.K2;
  const int kt_total = (Ktot + kBKd - 1) / kBKd;
  int kt_begin, kt_end;
  split_range(p, kBKd, kt_total, kt_begin, kt_end);

  // this lane's slot in each of its LPW blocks: stage row, logical chunk,
  // first- and second-part row pointers (clamped to a valid row)
  const uint16_t* src1[LPW];
  const uint16_t* src2[LPW];
  int lcol[LPW];
  bool real[LPW];
#pragma unroll
  for (int q = 0; q < LPW; ++q) {
    const int blk = q * NW + wave;
    const int row = blk * 16 + lane / 4;
    const int rr = row < BN ? row : row - BN;                // row within its region
    lcol[q] = 8 * ((lane & 3) ^ ((rr >> 1) & 3) ^ ((rr >> 3) & 1));
    real[q] = (LPW * NW == BLKS) || row < ROWS;   // padding blocks only when the rows do not fill them
    if (row < BN) {
      const int n = min(n0 + rr, p.N - 1);
      src1[q] = p.w + int64_t(n) * p.ldw;
      src2[q] = p.b + int64_t(n) * p.ldb;
    } else {
      const int m = min(m0 + rr, p.M - 1);
      const int g = p.gather_blk;
      const int pm = g > 0 ? (m / g) * 2 * g + g + m % g : m;
      src1[q] = p.x + int64_t(pm) * p.ldx;
      src2[q] = p.t + int64_t(pm) * p.ldt;
    }
  }
  const uint16_t* zero = reinterpret_cast<const uint16_t*>(kZeroChunk);
  auto issue = [&](int stage, int kt) {
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
      const int kc = kt * kBKd + lcol[q];
      // branch-free (bitwise, no short-circuit): one basic block per stage
      const bool ok = real[q] & (kt < kt_end) & (kc < Ktot);
      const uint16_t* g = kc < p.K1 ? src1[q] + kc : src2[q] + (kc - p.K1);
      g = ok ? g : zero;
      const uint32_t dst = lds_base + uint32_t(stage * STAGE + (q * NW + wave) * 1024);
      __builtin_amdgcn_global_load_lds(g, reinterpret_cast<__attribute__((address_space(3))) void*>(uintptr_t(dst)),
                                       16, 0, 0);
    }
  };

  f32x16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int lrow = lane & 31, lhalf = lane >> 5;
  auto frag = [&](int stage, int row, int c) {
    const uint32_t off = uint32_t(stage * STAGE + row * 64 + ((c ^ ((row >> 1) & 3) ^ ((row >> 3) & 1)) * 16));
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(uintptr_t(lds_base + off));
  };

  // Software pipeline over stages: the fragments of a stage's first k-step
  // are read right after the barrier that publishes the stage, while the
  // previous stage's second k-step still runs on the matrix cores; the wait
  // and barrier for the next stage sit between the two k-steps' MFMAs, whose
  // execution covers them.
  auto read = [&](int stage, int kk, bf16x8 (&fa)[FN], bf16x8 (&fb)[FM]) {
#pragma unroll
    for (int a = 0; a < FN; ++a) fa[a] = frag(stage, wn * TN + a * 32 + lrow, 2 * kk + lhalf);
#pragma unroll
    for (int b = 0; b < FM; ++b) fb[b] = frag(stage, BN + wm * TM + b * 32 + lrow, 2 * kk + lhalf);
  };
  auto mma = [&](const bf16x8 (&fa)[FN], const bf16x8 (&fb)[FM]) {
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
      for (int b = 0; b < FM; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
  };
  auto sync_stage = [&]() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  const int nk = kt_end - kt_begin;
  if (nk > 0) {
    bf16x8 f0a[FN], f0b[FM], f1a[FN], f1b[FM];
#pragma unroll
    for (int s = 0; s + 1 < S; ++s) issue(s, kt_begin + s);
    wait_vm<(S - 2) * LPW>();   // stage 0 landed
    sync_stage();
    read(0, 0, f0a, f0b);
    for (int i = 0; i < nk; ++i) {
      read(i % S, 1, f1a, f1b);
      mma(f0a, f0b);
      __builtin_amdgcn_sched_group_barrier(0x100, FN + FM, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, FN * FM, 0);
      wait_vm<(S - 3) * LPW>();   // stage i + 1 landed (past the end: zero loads)
      sync_stage();
      issue((i + S - 1) % S, kt_begin + i + S - 1);
      read((i + 1) % S, 0, f0a, f0b);
      mma(f1a, f1b);
      __builtin_amdgcn_sched_group_barrier(0x020, LPW, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, FN + FM, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, FN * FM, 0);
    }
  }
  // drain the trailing (unused) prefetches before the workgroup exits
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));

  if constexpr (MODE == 2) {
    // fragment i (gate) and i + FN / 2 (up) of a lane hold the same features
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int m = m0 + wm * TM + j * 32 + lrow;
      if (m >= p.M) continue;
#pragma unroll
      for (int i = 0; i < FN / 2; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * (TN / 2) + i * 32 + 8 * g + 4 * lhalf;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float gv = acc[i][j][4 * g + e], uv = acc[i + FN / 2][j][4 * g + e];
            o[e] = gv / (1.f + expf(-gv)) * uv;
          }
          uint16_t* dst = p.y + int64_t(m) * p.ldy + n;
          if (p.y_vec && n + 3 < p.N) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
          } else {
            for (int e = 0; e < 4; ++e)
              if (n + e < p.N) dst[e] = f32_to_bf16(o[e]);
          }
        }
      }
    }
    return;
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
          if (p.y_vec && n + 3 < p.N) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
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

// y = bf16(sum_s part[s]) in split order; 4 consecutive outputs per thread.
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float* __restrict__ part, int splits, int M, int N,
                                                          uint16_t* __restrict__ y, int64_t ldy, int y_vec) {
  const int64_t q = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per_row = (N + 3) / 4;
  if (q >= int64_t(M) * per_row) return;
  const int m = int(q / per_row);
  const int n = int(q - int64_t(m) * per_row) * 4;
  const int64_t plane = int64_t(M) * N;
  const float* src = part + int64_t(m) * N + n;
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  if (n + 3 < N && (N & 3) == 0) {
    for (int sp = 0; sp < splits; ++sp) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(src + sp * plane);
      s[0] += v[0];
      s[1] += v[1];
      s[2] += v[2];
      s[3] += v[3];
    }
  } else {
    for (int sp = 0; sp < splits; ++sp)
      for (int e = 0; e < 4; ++e)
        if (n + e < N) s[e] += src[sp * plane + e];
  }
  uint16_t* dst = y + int64_t(m) * ldy + n;
  if (y_vec && n + 3 < N) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]));
  } else {
    for (int e = 0; e < 4; ++e)
      if (n + e < N) dst[e] = f32_to_bf16(s[e]);
  }
}

// t[m, j] = bf16(scale * g[m] * sum_s part[s][m][j]); exact 0 for g = 0.
__global__ __launch_bounds__(256) void lora_gate_kernel(const float* __restrict__ part, int splits, int M, int r,
                                                        const uint8_t* __restrict__ gate, float scale,
                                                        uint16_t* __restrict__ t) {
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

// The same, four consecutive elements per thread (r % 4 == 0): 16-byte
// partial loads and an 8-byte store; the splits are summed in the same order.
// gblk > 0: the structured gate (rows j < gblk of every 2 * gblk are 0, the
// rest 1) with partials over the gated rows only ([splits][M / 2][r], row
// (m / 2gblk) * gblk + j - gblk); `gate` is then not read.
__global__ __launch_bounds__(256) void lora_gate4_kernel(const float* __restrict__ part, int splits, int M, int r,
                                                         const uint8_t* __restrict__ gate, float scale,
                                                         uint16_t* __restrict__ t, int gblk) {
  const int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= int64_t(M) * r) return;
  const int m = int(i / r);
  int pm = m, prow = M;
  if (gblk > 0) {
    const int j = m % (2 * gblk);
    pm = j < gblk ? -1 : (m / (2 * gblk)) * gblk + (j - gblk);
    prow = M / 2;
  } else if (gate[m] == 0) {
    pm = -1;
  }
  if (pm < 0) {
    *reinterpret_cast<uint2*>(t + i) = make_uint2(0u, 0u);
    return;
  }
  const int64_t plane = int64_t(prow) * r;
  const float* src = part + int64_t(pm) * r + (i - int64_t(m) * r);
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  // unrolled so the loads of 8 splits are in flight together; the adds keep split order
#pragma unroll 8
  for (int sp = 0; sp < splits; ++sp) s += *reinterpret_cast<const f32x4*>(src + sp * plane);
  *reinterpret_cast<uint2*>(t + i) =
      make_uint2(pack_bf16x2(scale * s[0], scale * s[1]), pack_bf16x2(scale * s[2], scale * s[3]));
}

// ------------------------------------------------------------------ merge
// out[n][k] = bf16(w[n][k] + scale * sum_j b[n][j] a[j][k]): the sum over
// j = 0 .. r-1 in order with fp32 fused multiply-adds, one rounding at the end.
// One thread per 8 consecutive k of a row n (grid.y = n); vec: 16-byte loads
// and stores (every leading dimension a multiple of 8, 16-byte aligned bases).
__global__ __launch_bounds__(256) void lora_merge_kernel(const uint16_t* __restrict__ w, int64_t ldw,
                                                         const uint16_t* __restrict__ a, int64_t lda,
                                                         const uint16_t* __restrict__ b, int64_t ldb, float scale,
                                                         int K, int r, uint16_t* __restrict__ out, int64_t ldo,
                                                         int vec) {
  const int n = blockIdx.y;
  const int k0 = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (k0 >= K) return;
  const int cnt = min(8, K - k0);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const uint16_t* brow = b + int64_t(n) * ldb;
  for (int j = 0; j < r; ++j) {
    const float bj = bf16_to_f32(brow[j]);
    const uint16_t* arow = a + int64_t(j) * lda + k0;
    if (vec && cnt == 8) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(arow);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(bj, bf16_lo(v[e]), acc[2 * e]);
        acc[2 * e + 1] = fmaf(bj, bf16_hi(v[e]), acc[2 * e + 1]);
      }
    } else {
      for (int e = 0; e < cnt; ++e) acc[e] = fmaf(bj, bf16_to_f32(arow[e]), acc[e]);
    }
  }
  const uint16_t* wrow = w + int64_t(n) * ldw + k0;
  uint16_t* orow = out + int64_t(n) * ldo + k0;
  if (vec && cnt == 8) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(wrow);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = pack_bf16x2(bf16_lo(v[e]) + scale * acc[2 * e], bf16_hi(v[e]) + scale * acc[2 * e + 1]);
    *reinterpret_cast<u32x4*>(orow) = o;
  } else {
    for (int e = 0; e < cnt; ++e) orow[e] = f32_to_bf16(bf16_to_f32(wrow[e]) + scale * acc[e]);
  }
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
                                                       const float* __restrict__ t, const float* __restrict__ b,
                                                       int64_t ldb, int M, int N, int K, int r,
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

// ------------------------------------------------------------------ dispatch
// Kernel configurations: block tile, wave grid, register prefetch depth
// (K-tiles in flight, sized so loads have about 1 us to land) and fragment
// double-buffering (off where it would push the tile past 512 registers).
struct TileShape {
  const char* name;
  int bm, bn, waves;
};
constexpr TileShape kShapes[] = {
    {"64x64w4", 64, 64, 4},          {"128x128w4", 128, 128, 4},      {"256x192w4", 256, 192, 4},
    {"256x192w8", 256, 192, 8},      {"256x192w8p1", 256, 192, 8},    {"256x192w8p2d0", 256, 192, 8},
    {"256x128w8", 256, 128, 8},      {"256x128w8p2d0", 256, 128, 8},  {"256x256w4", 256, 256, 4},
    {"256x256w8p1", 256, 256, 8},    {"dl256x256s4", 256, 256, 8},    {"dl256x256s5", 256, 256, 8},
    {"dl256x192s4", 256, 192, 8},    {"dl256x192s5", 256, 192, 8},    {"dl256x128s6", 256, 128, 8},
    {"dl128x128s6", 128, 128, 4},    {"dl256x256w4s4", 256, 256, 4},  {"dl256x256w4s5", 256, 256, 4},
    {"dl128x384s4", 128, 384, 8},    {"dl128x256s6", 128, 256, 8},    {"dl128x384s5", 128, 384, 8},
    {"dl128x256s4", 128, 256, 8},    {"dl64x384s4", 64, 384, 4},      {"dl64x256s4", 64, 256, 4},
    {"dl64x128s6", 64, 128, 2},
};
constexpr int kNumShapes = int(sizeof(kShapes) / sizeof(kShapes[0]));

struct TileCfg {
  int shape;   // index into kShapes
  int splits;
};

// The buffer-load path needs whole K-tiles and operands whose byte offsets
// (including rows up to one tile past the end) stay below 2^31.
bool fast_ok(const GemmParams& p, int bm, int bn) {
  const int64_t lim = int64_t(1) << 31;
  return p.K1 % kBK == 0 && p.K2 % kBK == 0 && int64_t(p.N + bn) * p.ldw * 2 < lim &&
         int64_t(p.N + bn) * p.ldb * 2 < lim && int64_t(p.M + bm) * p.ldx * 2 < lim &&
         int64_t(p.M + bm) * p.ldt * 2 < lim;
}

template <int BM, int BN, int WM, int WN, int P, int DBF, int MODE, int FAST>
hipError_t launch_tile_k(GemmParams p, int splits, hipStream_t stream, const char* name) {
  auto kern = gemm_bf16_kernel<BM, BN, WM, WN, P, DBF, MODE, FAST>;
  const size_t lds = 2 * size_t(BN + BM) * kBK * 2;
  static std::atomic<uint64_t> configured{0};
  {
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), int(lds), configured);
    if (e != hipSuccess) return e;
  }
  constexpr int TILE_N = MODE == 2 ? BN / 2 : BN;   // MODE 2: features per tile
  p.tiles_m = (p.M + BM - 1) / BM;
  p.tiles_n = (p.N + TILE_N - 1) / TILE_N;
  {
    const char* env = tuning_env("UNO_GEMM_XCD");   // tuning override: 0 no remap, 1 column bands, 2 (default) 2D groups
    p.xcd_remap = env ? atoi(env) : 2;
  }
  p.ktiles_per_split = ((p.K1 + kBK - 1) / kBK + splits - 1) / splits;
  dim3 grid(p.tiles_m * p.tiles_n, splits);
  ProfileScope ps(name, stream);
  hipLaunchKernelGGL(kern, grid, dim3(WM * WN * kWave), lds, stream, p);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int P, int DBF, int MODE>
hipError_t launch_tile(GemmParams p, int splits, hipStream_t stream, const char* name) {
  // the gate-merged row order exists on the buffer-load path only
  if (p.merge_m > 0)
    return fast_ok(p, BM, BN) ? launch_tile_k<BM, BN, WM, WN, P, DBF, MODE, 1>(p, splits, stream, name)
                              : hipErrorNotSupported;
  const char* env = tuning_env("UNO_GEMM_FAST");   // tuning override: 0 keeps the masked loads
  if (fast_ok(p, BM, BN) && !(env && atoi(env) == 0))
    return launch_tile_k<BM, BN, WM, WN, P, DBF, MODE, 1>(p, splits, stream, name);
  return launch_tile_k<BM, BN, WM, WN, P, DBF, MODE, 0>(p, splits, stream, name);
}

template <int BM, int BN, int WM, int WN, int S, int MODE>
hipError_t launch_tile_dl(GemmParams p, int splits, hipStream_t stream, const char* name) {
  auto kern = gemm_dl_kernel<BM, BN, WM, WN, S, MODE>;
  constexpr int NW = WM * WN;
  constexpr int LPW = ((BN + BM + 15) / 16 + NW - 1) / NW;
  const size_t lds = size_t(S) * LPW * NW * 1024;
  static std::atomic<uint64_t> configured{0};
  {
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), int(lds), configured);
    if (e != hipSuccess) return e;
  }
  p.tiles_m = (p.M + BM - 1) / BM;
  p.tiles_n = (p.N + BN - 1) / BN;
  {
    const char* env = tuning_env("UNO_GEMM_XCD");
    p.xcd_remap = env ? atoi(env) : 2;
  }
  p.ktiles_per_split = ((p.K1 + kBKd - 1) / kBKd + splits - 1) / splits;
  dim3 grid(p.tiles_m * p.tiles_n, splits);
  ProfileScope ps(name, stream);
  hipLaunchKernelGGL(kern, grid, dim3(NW * kWave), lds, stream, p);
  return hipGetLastError();
}

// The shapes the dispatcher chooses are always built; the others only in a
// tuning build (they are reachable through the tile overrides alone).
// The LoRA-down shapes (direct-to-LDS kernel, MODE 1: partials for the gate kernel).
template <int MODE>
hipError_t launch_cfg_dl(const TileCfg& c, const GemmParams& p, hipStream_t stream, const char* name) {
  switch (c.shape) {
    case 15: return launch_tile_dl<128, 128, 2, 2, 6, MODE>(p, c.splits, stream, name);
    case 18: return launch_tile_dl<128, 384, 2, 4, 4, MODE>(p, c.splits, stream, name);
    case 21: return launch_tile_dl<128, 256, 2, 4, 4, MODE>(p, c.splits, stream, name);
#ifdef UNO_TUNING
    case 22: return launch_tile_dl<64, 384, 1, 4, 4, MODE>(p, c.splits, stream, name);
    case 23: return launch_tile_dl<64, 256, 1, 4, 4, MODE>(p, c.splits, stream, name);
    case 24: return launch_tile_dl<64, 128, 1, 2, 6, MODE>(p, c.splits, stream, name);
    case 19: return launch_tile_dl<128, 256, 2, 4, 6, MODE>(p, c.splits, stream, name);
    case 20: return launch_tile_dl<128, 384, 2, 4, 5, MODE>(p, c.splits, stream, name);
#endif
    default: break;
  }
  return hipErrorInvalidValue;
}

template <int MODE>
hipError_t launch_cfg(const TileCfg& c, const GemmParams& p, hipStream_t stream, const char* name) {
  switch (c.shape) {
    case 0: return launch_tile<64, 64, 2, 2, 4, 1, MODE>(p, c.splits, stream, name);
    case 1: return launch_tile<128, 128, 2, 2, 4, 1, MODE>(p, c.splits, stream, name);
    case 5: return launch_tile<256, 192, 4, 2, 2, 0, MODE>(p, c.splits, stream, name);
    case 9:
#ifdef UNO_TUNING
      if (const char* env = tuning_env("UNO_GEMM_DEFER"))   // tuning override: 0 = no deferred k-step
        if (atoi(env) == 0) return launch_tile<256, 256, 4, 2, 1, 0, MODE>(p, c.splits, stream, name);
#endif
      return launch_tile<256, 256, 4, 2, 1, 2, MODE>(p, c.splits, stream, name);
#ifdef UNO_TUNING
    case 2: return launch_tile<256, 192, 2, 2, 2, 0, MODE>(p, c.splits, stream, name);
    case 3: return launch_tile<256, 192, 4, 2, 2, 1, MODE>(p, c.splits, stream, name);
    case 4: return launch_tile<256, 192, 4, 2, 1, 1, MODE>(p, c.splits, stream, name);
    case 6: return launch_tile<256, 128, 4, 2, 3, 1, MODE>(p, c.splits, stream, name);
    case 7: return launch_tile<256, 128, 4, 2, 2, 0, MODE>(p, c.splits, stream, name);
    case 8: return launch_tile<256, 256, 2, 2, 1, 0, MODE>(p, c.splits, stream, name);
    case 10: return launch_tile_dl<256, 256, 4, 2, 4, MODE>(p, c.splits, stream, name);
    case 11: return launch_tile_dl<256, 256, 4, 2, 5, MODE>(p, c.splits, stream, name);
    case 12: return launch_tile_dl<256, 192, 4, 2, 4, MODE>(p, c.splits, stream, name);
    case 13: return launch_tile_dl<256, 192, 4, 2, 5, MODE>(p, c.splits, stream, name);
    case 14: return launch_tile_dl<256, 128, 4, 2, 6, MODE>(p, c.splits, stream, name);
    case 16: return launch_tile_dl<256, 256, 2, 2, 4, MODE>(p, c.splits, stream, name);
    case 17: return launch_tile_dl<256, 256, 2, 2, 5, MODE>(p, c.splits, stream, name);
#endif
    default: break;
  }
  if constexpr (MODE == 1) return launch_cfg_dl<MODE>(c, p, stream, name);
  return hipErrorInvalidValue;
}

int shape_index(const char* name) {
  for (int i = 0; i < kNumShapes; ++i)
    if (strcmp(kShapes[i].name, name) == 0) return i;
  return -1;
}

// Main-GEMM configuration.  UNO_GEMM_TILE="<shape name>[/splits]" overrides
// the choice (tuning sweeps).
// The choice depends on the base K only, so a call with and without adapter
// columns runs the same kernel and split (bit-identical gate-0 rows).
TileCfg choose_main_tile(int64_t M, int64_t N, int64_t Ktot) {
  const char* env = tuning_env("UNO_GEMM_TILE");
  if (env) {
    char nm[32] = {0};
    int s = 1;
    const char* slash = strchr(env, '/');
    const size_t len = slash ? size_t(slash - env) : strlen(env);
    if (len < sizeof(nm)) {
      memcpy(nm, env, len);
      if (slash) s = atoi(slash + 1);
      const int id = shape_index(nm);
      if (id >= 0 && s >= 1 && s <= 16) return {id, s};
    }
  }
  // Measured on MI355X at M = 1024 (event-timed sweeps, buffer-load path), where M < 2048:
  //   4096 -> 12288: 256x192 (8 waves, 2-deep prefetch; 256 tiles, one per CU), 1.02 PFLOP/s;
  //   12288 -> 4096: 256x256 (8 waves) with 4 K-splits;
  //   4096 -> 4096: 128x128 (4 waves), no split (256 tiles);
  //   4096 -> 1024: 128x128 (4 waves) with 4 K-splits.
  auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  const int64_t kt = (Ktot + kBK - 1) / kBK;
  auto splits_for = [&](int64_t t, int smax, int min_kt) {
    int s = 1;
    while (t * s < 192 && s < smax && kt / (2 * s) >= min_kt) s *= 2;
    return s;
  };
  // Measured at M = 4096 (the decode step's rows): the register-prefetch
  // 256x256 kernel (8 waves) leads for every projection with N >= 2048 and
  // for the LM head (1.0-1.15 PFLOP/s against 0.6-1.0 for the others).
  if (M >= 2048 && N >= 2048) return {9, 1};
  if (M >= 512 && N % 192 == 0 && tiles(256, 192) >= 192) return {5, 1};
  if (M >= 512 && N % 256 == 0 && tiles(256, 256) >= 64 && kt >= 128) return {9, splits_for(tiles(256, 256), 4, 8)};
  if (M >= 512 && N % 128 == 0) return {1, splits_for(tiles(128, 128), 4, 8)};
  return {1, splits_for(tiles(128, 128), 4, 16)};
}

// LoRA-down tile and split count.  Measured at M = 4096 (event-timed): the
// direct-load 128x128 tile with 8 K-splits takes 18 us at K = 4096 and 30 us
// at K = 12288, against 25 and 67 us for 64x64 tiles with 2 splits; below
// 2048 rows the 64x64 tile spreads over enough workgroups.
TileCfg lora_down_cfg(int64_t M, int64_t r, int64_t K) {
  const int64_t kt = (K + kBK - 1) / kBK;
  int shape = 0;
  int64_t s;
  if (M >= 2048 && r % 128 == 0) {
    // 128 rows x all of a group's adapter rows where they fit one tile (x is
    // then read once per split, not once per 128 adapter rows), 8 K-splits:
    // at 4096 x 4096 the q|k|v group (r = 384) takes 28 us against 41 with
    // 128 x 128 tiles, gate|up (256) 22.5 against 30.6
    shape = r % 384 == 0 ? 18 : (r % 256 == 0 ? 21 : 15);
    // at least 8 K-splits, more when the row tiles alone leave CUs idle:
    // 2048 rows take 16 tiles x 12 splits.  More splits shorten this kernel
    // but lengthen the split sum (every split is re-read): inside the decode
    // step (noisy rows gathered) the two together take 4.57 ms per step at 8
    // splits, 4.38 at 12 and 4.48 at 16
    const int64_t tiles_m = (M + 127) / 128;
    s = std::max<int64_t>(8, (192 + tiles_m - 1) / tiles_m);
  } else {
    const int64_t tiles = ((M + 63) / 64) * ((r + 63) / 64);
    s = (256 + tiles - 1) / tiles;
  }
  {
    const char* env = tuning_env("UNO_LORA_SPLITS");   // tuning override (sweeps): partials for this many splits
    if (env && atoi(env) >= 1 && atoi(env) <= 16) s = atoi(env);
  }
  if (s > kt / 2) s = kt / 2;
  if (s < 1) s = 1;
  if (s > 16) s = 16;
  return TileCfg{shape, int(s)};
}

int lora_down_splits(int64_t M, int64_t r, int64_t K) { return lora_down_cfg(M, r, K).splits; }

}  // namespace

size_t gated_lora_workspace_bytes(uno_dtype dtype, int64_t M, int64_t N, int64_t K, int64_t r) {
  if (dtype == UNO_F32) return r == 0 ? 0 : align_up(size_t(M) * size_t(r) * 4, 256);
  size_t bytes = 0;
  if (r > 0) {
    const int s = lora_down_splits(M, r, K);
    bytes += align_up(size_t(M) * size_t(r) * 2, 256) + align_up(size_t(s) * size_t(M) * size_t(r) * 4, 256);
  }
  const TileCfg c = choose_main_tile(M, N, K);
  if (c.splits > 1) bytes += align_up(size_t(c.splits) * size_t(M) * size_t(N) * 4, 256);
  return bytes;
}

size_t lora_down_part_bytes(int64_t M, int64_t n, int64_t K) {
  return align_up(size_t(lora_down_splits(M, n, K)) * size_t(M) * size_t(n) * 4, 256);
}

namespace {

bool is_dl_shape(int shape) { return shape == 15 || (shape >= 18 && shape <= 24); }

// The gathered LoRA-down (structured gate): over the M / 2 gated rows only,
// when those rows take a direct-to-LDS tile, the gate kernel's vector form
// applies and the partials fit the space sized for the full M rows.
bool lora_gather_ok(const LoraDownArgs& a) {
  if (a.gather_blk <= 0 || a.M % (2 * a.gather_blk) != 0) return false;
  if (!is_dl_shape(lora_down_cfg(a.M / 2, a.n, a.K).shape)) return false;
  if (a.n % 4 != 0 || (reinterpret_cast<uintptr_t>(a.part) & 15u) != 0 || (reinterpret_cast<uintptr_t>(a.t) & 7u) != 0)
    return false;
  return lora_down_part_bytes(a.M / 2, a.n, a.K) <= lora_down_part_bytes(a.M, a.n, a.K);
}

}  // namespace

// T[M][n] = bf16(s * g[m] * x A^T) for the n rows of A (one projection's r,
// or several projections' adapters stored back to back): split-K MFMA GEMM
// into fp32 partials, then lora_gate_kernel sums them in a fixed order.
hipError_t launch_lora_down(const LoraDownArgs& a, hipStream_t stream) {
  // rows the GEMM reads: all M, or only the gated M / 2 under the structured gate
  const bool gather = lora_gather_ok(a);
  const int64_t Mg = gather ? a.M / 2 : a.M;
  const int splits = lora_down_splits(Mg, a.n, a.K);
  GemmParams d{};
  d.M = int(Mg);
  d.N = int(a.n);
  d.K1 = int(a.K);
  d.K2 = 0;
  d.x = static_cast<const uint16_t*>(a.x);
  d.ldx = a.ldx;
  d.w = static_cast<const uint16_t*>(a.a);
  d.ldw = a.lda;
  d.t = d.x;
  d.ldt = d.ldx;
  d.b = d.w;
  d.ldb = d.ldw;
  d.part = static_cast<float*>(a.part);
  d.gather_blk = gather ? a.gather_blk : 0;
  TileCfg dc = lora_down_cfg(Mg, a.n, a.K);
  {
    // tuning build: per-shape override UNO_LORA_TILE_<n>_<K>="<shape name>/<splits>"
    char key[64];
    snprintf(key, sizeof(key), "UNO_LORA_TILE_%lld_%lld", (long long)a.n, (long long)a.K);
    const char* env = tuning_env(key);
    if (env) {
      char nm[32] = {0};
      const char* slash = strchr(env, '/');
      const size_t len = slash ? size_t(slash - env) : strlen(env);
      if (len < sizeof(nm)) {
        memcpy(nm, env, len);
        const int id = shape_index(nm);
        const int sp = slash ? atoi(slash + 1) : 1;
        if (id >= 0 && sp >= 1 && sp <= splits && (!gather || is_dl_shape(id))) dc = TileCfg{id, sp};
      }
    }
  }
  {
    // tuning override "<shape name>/<splits>" (sweeps only); the split count sizes the
    // partials, so it may not exceed the one the workspace was sized for
    const char* env = tuning_env("UNO_LORA_TILE");
    if (env) {
      char nm[32] = {0};
      const char* slash = strchr(env, '/');
      const size_t len = slash ? size_t(slash - env) : strlen(env);
      if (len < sizeof(nm)) {
        memcpy(nm, env, len);
        const int id = shape_index(nm);
        const int sp = slash ? atoi(slash + 1) : 1;
        if (id >= 0 && sp >= 1 && sp <= splits && (!gather || is_dl_shape(id))) dc = TileCfg{id, sp};
      }
    }
  }
  // the vector form needs 4-element rows and 16-byte aligned partials / 8-byte aligned T
  const bool vec = a.n % 4 == 0 && (reinterpret_cast<uintptr_t>(a.part) & 15u) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.t) & 7u) == 0;
  char pname[64] = "uno_lora_down_bf16", gname[64] = "uno_lora_gate";
#ifdef UNO_TUNING
  // tuning build: kernel timings named per shape
  snprintf(pname, sizeof(pname), "uno_lora_down_bf16_%lld_%lld", (long long)a.n, (long long)a.K);
  snprintf(gname, sizeof(gname), "uno_lora_gate_%lld_%lld", (long long)a.n, (long long)a.K);
#endif
  hipError_t e = launch_cfg<1>(dc, d, stream, pname);
  if (e != hipSuccess) return e;
  const int64_t n = a.M * a.n;
  ProfileScope ps(gname, stream);
  if (vec)
    hipLaunchKernelGGL(lora_gate4_kernel, dim3(unsigned((n / 4 + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const float*>(a.part), dc.splits, int(a.M), int(a.n), a.gate, a.lora_scale, a.t,
                       gather ? a.gather_blk : 0);
  else
    hipLaunchKernelGGL(lora_gate_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const float*>(a.part), dc.splits, int(a.M), int(a.n), a.gate, a.lora_scale, a.t);
  return hipGetLastError();
}

namespace {

void set_merged(GemmParams& g, int64_t M, int gate_block, const void* wm, const void* wm2) {
  g.K2 = 0;
  g.kr = 0;
  g.t = g.x;
  g.ldt = g.ldx;
  g.b = g.w;
  g.b2 = g.w2;
  g.ldb = g.ldw;
  g.merge_m = int(M / 2);
  g.row_blk = gate_block;
  g.wm = static_cast<const uint16_t*>(wm);
  g.wm2 = static_cast<const uint16_t*>(wm2);
}

bool swiglu_merged(const SwigluArgs& a) {
  return a.r > 0 && a.wg_merged && a.wu_merged && merged_rows_ok(a.M, a.gate_block, 256, 512);
}

GemmParams swiglu_params(const SwigluArgs& a) {
  GemmParams g{};
  const bool lora = a.r > 0 && !swiglu_merged(a);
  g.M = int(a.M);
  g.N = int(a.N);
  g.K1 = int(a.K);
  g.K2 = lora ? int(2 * a.r) : 0;
  g.x = static_cast<const uint16_t*>(a.x);
  g.ldx = a.ldx;
  g.w = static_cast<const uint16_t*>(a.wg);
  g.w2 = static_cast<const uint16_t*>(a.wu);
  g.ldw = a.ldw;
  g.t = lora ? static_cast<const uint16_t*>(a.t) : g.x;
  g.ldt = lora ? a.ldt : a.ldx;
  g.b = lora ? static_cast<const uint16_t*>(a.bg) : g.w;
  g.b2 = lora ? static_cast<const uint16_t*>(a.bu) : g.w2;
  g.ldb = lora ? a.ldb : a.ldw;
  g.kr = lora ? int(a.r / kBK) : 0;
  g.y = static_cast<uint16_t*>(a.y);
  g.ldy = a.ldy;
  g.y_vec = (a.ldy % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.y) & 7u) == 0);
  if (swiglu_merged(a)) set_merged(g, a.M, a.gate_block, a.wg_merged, a.wu_merged);
  return g;
}

}  // namespace

bool merged_rows_ok(int64_t M, int gate_block, int bm, int threads) {
  if (gate_block <= 0 || M % (2 * gate_block) != 0 || (M / 2) % bm != 0) return false;
  return (threads / kChunksPerRow) % gate_block == 0;
}

bool swiglu_fused_ok(const SwigluArgs& a) {
  if (a.K % kBK != 0 || a.r % kBK != 0) return false;
  if (a.r > 0 && !swiglu_merged(a) && (!a.t || a.ldt < 2 * a.r || !a.bg || !a.bu)) return false;
  return fast_ok(swiglu_params(a), 256, 256);
}

// gate and up projections in one launch (MODE 2 of gemm_bf16_kernel), y =
// bf16(silu(g) * u); the 256 x 256 tile with 8 waves on the buffer-load path
hipError_t launch_gated_lora_swiglu(const SwigluArgs& a, hipStream_t stream) {
  if (!swiglu_fused_ok(a)) return hipErrorNotSupported;
#ifdef UNO_TUNING
  if (const char* env = tuning_env("UNO_GEMM_DEFER"))   // tuning override: 0 = no deferred k-step
    if (atoi(env) == 0) return launch_tile_k<256, 256, 4, 2, 1, 0, 2, 1>(swiglu_params(a), 1, stream, "uno_gemm_bf16");
#endif
  return launch_tile_k<256, 256, 4, 2, 1, 2, 2, 1>(swiglu_params(a), 1, stream, "uno_gemm_bf16");
}

namespace {

// Gate-merged launch of one projection (pair: bm = 256 on 8 waves).
bool lora_merged(const GatedLoraArgs& a, int bm, int threads) {
  return a.dtype == UNO_BF16 && a.r > 0 && a.gate && a.w_merged && merged_rows_ok(a.M, a.gate_block, bm, threads);
}

GemmParams lora_params(const GatedLoraArgs& a, const uint16_t* t, int64_t ldt) {
  const bool lora = a.r > 0 && a.gate != nullptr;
  GemmParams g{};
  g.M = int(a.M);
  g.N = int(a.N);
  g.K1 = int(a.K);
  g.K2 = lora ? int(a.r) : 0;
  g.x = static_cast<const uint16_t*>(a.x);
  g.ldx = a.ldx;
  g.w = static_cast<const uint16_t*>(a.w);
  g.ldw = a.ldw;
  g.t = lora ? t : g.x;
  g.ldt = lora ? ldt : a.ldx;
  g.b = lora ? static_cast<const uint16_t*>(a.b) : g.w;
  g.ldb = lora ? a.ldb : a.ldw;
  g.y = static_cast<uint16_t*>(a.y);
  g.ldy = a.ldy;
  g.y_vec = (a.ldy % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.y) & 7u) == 0);
  return g;
}

}  // namespace

// Two projections of one input with the same shapes (k and v), each with T
// computed by the caller, as one launch over 2N output columns.
bool gated_lora_pair_ok(const GatedLoraArgs& a, const GatedLoraArgs& b) {
  const bool la = a.r > 0 && a.gate, lb = b.r > 0 && b.gate;
  if (a.dtype != UNO_BF16 || b.dtype != UNO_BF16 || la != lb) return false;
  if (a.M != b.M || a.N != b.N || a.K != b.K || a.r != b.r || a.x != b.x || a.ldx != b.ldx || a.ldw != b.ldw ||
      a.ldb != b.ldb || a.ldy != b.ldy || a.ldt_pre != b.ldt_pre || a.gate != b.gate)
    return false;
  const bool merged = lora_merged(a, 256, 512) && lora_merged(b, 256, 512) && a.gate_block == b.gate_block;
  if (la && !merged && (!a.t_pre || !b.t_pre)) return false;
  if (a.M < 2048 || a.N % 128 != 0 || a.N * 2 > 0x7fffffff) return false;
  GemmParams ga = lora_params(a, static_cast<const uint16_t*>(a.t_pre), a.ldt_pre);
  GemmParams gb = lora_params(b, static_cast<const uint16_t*>(b.t_pre), b.ldt_pre);
  if (merged) {
    set_merged(ga, a.M, a.gate_block, a.w_merged, b.w_merged);
    set_merged(gb, b.M, b.gate_block, b.w_merged, a.w_merged);
  }
  return fast_ok(ga, 256, 128) && fast_ok(gb, 256, 128) && ga.y_vec && gb.y_vec;
}

// Measured at 4096 rows, N = 1024 each (k and v): 256 x 128 tiles on 8 waves
// (2-deep prefetch), 256 tiles over 2N, 76 us against 2 x 53 us for two
// launches on 128 x 128 tiles.
hipError_t launch_gated_lora_pair(const GatedLoraArgs& a, const GatedLoraArgs& b, hipStream_t stream) {
  if (!gated_lora_pair_ok(a, b)) return hipErrorNotSupported;
  const bool merged = lora_merged(a, 256, 512) && lora_merged(b, 256, 512) && a.gate_block == b.gate_block;
  const bool lora = a.r > 0 && a.gate && !merged;
  GemmParams g = lora_params(a, static_cast<const uint16_t*>(a.t_pre), a.ldt_pre);
  g.N = int(2 * a.N);
  g.seg_n = int(a.N);
  g.w2 = static_cast<const uint16_t*>(b.w);
  g.b2 = lora ? static_cast<const uint16_t*>(b.b) : g.w2;
  g.t2_off = lora ? static_cast<const uint16_t*>(b.t_pre) - static_cast<const uint16_t*>(a.t_pre) : 0;
  g.y2 = static_cast<uint16_t*>(b.y);
  // merged: k rows read (w, w_merged of k), v rows (after the segment swap) those of v
  if (merged) set_merged(g, a.M, a.gate_block, a.w_merged, b.w_merged);
  return launch_tile_k<256, 128, 4, 2, 2, 0, 0, 1>(g, 1, stream, "uno_gemm_bf16");
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
                         static_cast<const float*>(a.x), a.ldx, static_cast<const float*>(a.a), a.lda, a.gate,
                         a.lora_scale, int(a.M), int(a.K), int(a.r), t);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    const int64_t n = a.M * a.N;
    ProfileScope ps("uno_gemm_f32", stream);
    hipLaunchKernelGGL(gemm_f32_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const float*>(a.x), a.ldx, static_cast<const float*>(a.w), a.ldw, t,
                       static_cast<const float*>(a.b), a.ldb, int(a.M), int(a.N), int(a.K), lora ? int(a.r) : 0,
                       static_cast<float*>(a.y), a.ldy);
    return hipGetLastError();
  }

  if (lora && a.w_merged && a.gate_block > 0) {
    // the gated rows against the merged weights: no LoRA-down, no adapter columns
    const TileCfg c = choose_main_tile(a.M, a.N, a.K);
    const int threads = kShapes[c.shape].waves * kWave;
    if (c.splits == 1 && lora_merged(a, kShapes[c.shape].bm, threads)) {
      GemmParams g = lora_params(a, nullptr, 0);
      set_merged(g, a.M, a.gate_block, a.w_merged, a.w_merged);
      if (fast_ok(g, kShapes[c.shape].bm, kShapes[c.shape].bn)) return launch_cfg<0>(c, g, stream, "uno_gemm_bf16");
    }
  }
  char* ws = static_cast<char*>(a.ws);
  const uint16_t* t = nullptr;
  int64_t ldt = a.r;
  if (lora && a.t_pre) {
    // T computed by the caller (a grouped LoRA-down over several projections)
    t = static_cast<const uint16_t*>(a.t_pre);
    ldt = a.ldt_pre;
  } else if (lora) {
    uint16_t* tw = reinterpret_cast<uint16_t*>(ws);
    ws += align_up(size_t(a.M) * a.r * 2, 256);
    LoraDownArgs ld{};
    ld.M = a.M;
    ld.K = a.K;
    ld.n = a.r;
    ld.x = a.x;
    ld.ldx = a.ldx;
    ld.a = a.a;
    ld.lda = a.lda;
    ld.gate = a.gate;
    ld.lora_scale = a.lora_scale;
    ld.t = tw;
    ld.part = ws;
    ld.gather_blk = a.gate_block;
    ws += align_up(size_t(lora_down_splits(a.M, a.r, a.K)) * size_t(a.M) * size_t(a.r) * 4, 256);
    hipError_t e = launch_lora_down(ld, stream);
    if (e != hipSuccess) return e;
    t = tw;
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
  g.t = lora ? t : g.x;
  g.ldt = lora ? ldt : a.ldx;
  g.b = lora ? static_cast<const uint16_t*>(a.b) : g.w;
  g.ldb = lora ? a.ldb : a.ldw;
  g.y = static_cast<uint16_t*>(a.y);
  g.ldy = a.ldy;
  g.y_vec = (a.ldy % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.y) & 7u) == 0);
  const TileCfg c = choose_main_tile(a.M, a.N, a.K);
  if (c.splits == 1) return launch_cfg<0>(c, g, stream, "uno_gemm_bf16");
  g.part = reinterpret_cast<float*>(ws);
  hipError_t e = launch_cfg<1>(c, g, stream, "uno_gemm_bf16_splitk");
  if (e != hipSuccess) return e;
  const int64_t quads = a.M * ((a.N + 3) / 4);
  ProfileScope ps("uno_gemm_reduce", stream);
  hipLaunchKernelGGL(gemm_reduce_kernel, dim3(unsigned((quads + 255) / 256)), dim3(256), 0, stream, g.part, c.splits,
                     int(a.M), int(a.N), g.y, g.ldy, g.y_vec);
  return hipGetLastError();
}

hipError_t launch_lora_merge(const LoraMergeArgs& m, hipStream_t stream) {
  const bool vec = m.ldw % 8 == 0 && m.lda % 8 == 0 && m.ldo % 8 == 0 &&
                   ((reinterpret_cast<uintptr_t>(m.w) | reinterpret_cast<uintptr_t>(m.a) |
                     reinterpret_cast<uintptr_t>(m.out)) & 15u) == 0;
  const dim3 grid(unsigned((m.K + 2047) / 2048), unsigned(m.N));
  ProfileScope ps("uno_lora_merge", stream);
  hipLaunchKernelGGL(lora_merge_kernel, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(m.w), m.ldw,
                     static_cast<const uint16_t*>(m.a), m.lda, static_cast<const uint16_t*>(m.b), m.ldb, m.scale,
                     int(m.K), int(m.r), static_cast<uint16_t*>(m.out), m.ldo, vec ? 1 : 0);
  return hipGetLastError();
}

}  // namespace uno
