// Block-masked grouped-query attention of a decode step over a long KV cache,
// gfx950.
//
// Method: Uno summary (hyper.ai, arXiv 2609.04010), section "方法" -- one
// forward pass over the concatenated clean and noisy rows of a block; section
// "实验" -- the clean (verify) and noisy (draft) rows share one KV cache.
// Mask (the pages give none; the reading used throughout): every row sees the
// whole cache; clean row i also sees clean rows 0..i; a noisy row sees all
// 2*block rows of its block.  With per-sequence cache lengths (a cache whose
// verified prefix grows by the kept rows of each step) sequence b sees its
// first ctx_lens[b] cache rows; its rows sit `ctx` (the capacity) rows apart.
//
// Work unit: 128 query rows of one (sequence, KV head), i.e. 4 waves x 32
// rows, where row r is (block row r / G, head g*G + r % G): the G query heads
// of a KV head and all block rows read every K/V byte once per workgroup.  At
// the decode-step shape (16 + 16 rows, G = 4) one workgroup covers a whole
// (sequence, KV head).  Keys are the cache rows then the block rows, in blocks
// of 32; when the grid is small the key blocks are split into contiguous
// ranges over several workgroups whose partials are merged by the shared
// combine kernel.
//
// K/V staging: each 32-key block (K 8 KB + V 8 KB) goes straight from global
// memory into LDS with global_load_lds_dwordx4 (one wave instruction fills
// 1 KB: lane l writes bytes 16 l .. 16 l + 15), through a 4-stage ring, so
// three blocks are in flight while one is computed.  Each lane loads the
// global chunk whose swizzled LDS slot it fills:
//   K: 16-byte chunk c of key row k at c ^ (k & 15)  -- the 16-byte fragment
//      reads of 8 or 16 consecutive keys then hit distinct banks;
//   V: chunk c of key row k at c ^ T[k & 3], T = {0, 6, 10, 12} -- the
//      transposed 8-byte reads of 4 consecutive keys x 32 bytes hit distinct
//      banks for both 16- and 32-lane LDS phases.
//
// Per key block, per wave (v_mfma_f32_32x32x16_bf16):
//   S^T[key][row] = K . Q^T: K fragments are 16-byte LDS reads, Q^T is held in
//                   registers for the whole loop;
//   online softmax in the log2 domain, lane l owning query row l % 32;
//   O^T[d][row] += V^T . P^T: the V^T operand needs 8 keys at a fixed d per
//                   lane; ds_read_b64_tr_b16 delivers 4 consecutive keys at
//                   d = lane's column from a row-major LDS tile (each 16-lane
//                   group addresses a 4-key x 16-d patch, lane j at key j / 4,
//                   d 4 (j % 4)), so no transposition pass is needed.
#include <stdlib.h>

#include "device_common.h"
#include "internal.h"

namespace uno {

namespace {

constexpr int kHD = 128;
constexpr int kKB = 32;                           // keys per block
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kRows = kWaves * 32;                // query rows per workgroup
constexpr int kStagesDefault = 4;
constexpr int kKBytes = kKB * kHD * 2;            // 8 KB of K per block
constexpr int kStageBytes = 2 * kKBytes;          // K + V
constexpr int kLpw = kStageBytes / 1024 / kWaves; // 1 KB load instructions per wave per stage
constexpr int kXcd = 8;
constexpr int kTargetWgs = 512;                   // 2 resident workgroups per CU
constexpr int kMinBlocksPerSplit = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;                      // log2 headroom of the lazily updated max

static_assert(kLpw * kWaves * 1024 == kStageBytes, "a stage is a whole number of wave loads");

__device__ __align__(16) const uint32_t kZero16[4] = {0u, 0u, 0u, 0u};
constexpr int kLoadNt = 2;   // cache-policy operand of a direct-to-LDS load: non-temporal

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt vmcnt(N) alone
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// two floats to packed bf16, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{lo, hi}, bf16x2v));
}

__host__ __device__ __forceinline__ int swz_v(int k) { return ((k & 1) ? 6 : 0) ^ ((k & 2) ? 10 : 0); }

struct BlkPlan {
  int tiles;    // 128-row tiles per (sequence, KV head)
  int ks;       // key splits
  int groups;   // batch * n_kv * ks
  int nblk;     // key blocks
  int per;      // key blocks per split
};

BlkPlan make_plan(int batch, int n, int ctx, int H, int Hkv) {
  BlkPlan p;
  const int G = H / Hkv;
  p.tiles = (n * G + kRows - 1) / kRows;
  p.nblk = (ctx + n + kKB - 1) / kKB;
  const int64_t base = int64_t(p.tiles) * Hkv * batch;
  int ks = 1;
  if (base < kTargetWgs) {
    ks = int(kTargetWgs / base);
    const int most = p.nblk / kMinBlocksPerSplit;
    if (ks > most) ks = most;
    if (ks < 1) ks = 1;
  }
  p.per = (p.nblk + ks - 1) / ks;
  p.ks = (p.nblk + p.per - 1) / p.per;   // no empty split
  p.groups = batch * Hkv * p.ks;
  return p;
}

typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));

// The eight transposed V reads of one 16-key step (2 halves x 4 d-blocks),
// written out so the compiler does not order them behind every pending
// direct-to-LDS load (its waitcnt pass cannot tell the two apart and would
// wait for all of them); the reads complete inside the block, and the stage
// they read is published by the explicit vmcnt wait and barrier of the loop.
__device__ __forceinline__ void read_vt(s16x4 (&t)[2][4], const uint32_t (&va)[2][4], int st) {
  if (st == 0) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\t"
        "ds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\t"
        "ds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t[0][0]), "=&v"(t[0][1]), "=&v"(t[0][2]), "=&v"(t[0][3]), "=&v"(t[1][0]), "=&v"(t[1][1]),
          "=&v"(t[1][2]), "=&v"(t[1][3])
        : "v"(va[0][0]), "v"(va[0][1]), "v"(va[0][2]), "v"(va[0][3]), "v"(va[1][0]), "v"(va[1][1]), "v"(va[1][2]),
          "v"(va[1][3])
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:4096\n\t"
        "ds_read_b64_tr_b16 %1, %9 offset:4096\n\t"
        "ds_read_b64_tr_b16 %2, %10 offset:4096\n\t"
        "ds_read_b64_tr_b16 %3, %11 offset:4096\n\t"
        "ds_read_b64_tr_b16 %4, %12 offset:4096\n\t"
        "ds_read_b64_tr_b16 %5, %13 offset:4096\n\t"
        "ds_read_b64_tr_b16 %6, %14 offset:4096\n\t"
        "ds_read_b64_tr_b16 %7, %15 offset:4096\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t[0][0]), "=&v"(t[0][1]), "=&v"(t[0][2]), "=&v"(t[0][3]), "=&v"(t[1][0]), "=&v"(t[1][1]),
          "=&v"(t[1][2]), "=&v"(t[1][3])
        : "v"(va[0][0]), "v"(va[0][1]), "v"(va[0][2]), "v"(va[0][3]), "v"(va[1][0]), "v"(va[1][1]), "v"(va[1][2]),
          "v"(va[1][3])
        : "memory");
  }
}

// The eight K fragments of a block (one per 16-dim step), issued together and
// waited for once: one LDS round trip instead of one per fragment.
__device__ __forceinline__ void read_k(bf16x8 (&kf)[8], const uint32_t (&ka)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b128 %2, %10\n\t"
      "ds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %12\n\t"
      "ds_read_b128 %5, %13\n\t"
      "ds_read_b128 %6, %14\n\t"
      "ds_read_b128 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(kf[2]), "=&v"(kf[3]), "=&v"(kf[4]), "=&v"(kf[5]), "=&v"(kf[6]),
        "=&v"(kf[7])
      : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(ka[4]), "v"(ka[5]), "v"(ka[6]), "v"(ka[7])
      : "memory");
}

// x combined with the value of lane l ^ 32: v_permlane32_swap exchanges the
// upper half of one register with the lower half of another, so swapping two
// copies of x leaves each lane with x and its partner in the two registers
// (no LDS round trip, unlike a cross-half shuffle).
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  asm volatile("s_nop 4\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 4" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float max_xor32(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_xor32(float x) {
  float a = x, b = x;
  swap_halves(a, b);
  return a + b;
}

template <int kStages>
__global__ __launch_bounds__(kThreads) void block_attn_kernel(TreeAttnArgs a, BlkPlan pl, float* part_o,
                                                              float2* part_ms) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  uint32_t lds_base = uint32_t(reinterpret_cast<uintptr_t>(smem_raw));
  asm volatile("" : "+s"(lds_base));

  // ---- work unit (XCD-grouped numbering; the grid is padded to a multiple of 8 groups)
  const int L = blockIdx.x;
  const int slot = L / kXcd;
  const int tile = slot % pl.tiles;
  const int grp = (slot / pl.tiles) * kXcd + L % kXcd;
  if (grp >= pl.groups) return;
  const int ksi = grp % pl.ks;
  const int g = (grp / pl.ks) % a.n_kv;
  const int b = grp / (pl.ks * a.n_kv);

  const int n = a.n_tree, cap = a.ctx, H = a.n_heads, Hkv = a.n_kv, blk = a.block;
  // valid cache rows of this sequence (rows cap apart in memory); the key
  // blocks past its cache and block rows are not visited
  const int ctx = a.ctx_lens ? __builtin_amdgcn_readfirstlane(min(max(a.ctx_lens[b], 0), cap)) : cap;
  const int G = H / Hkv;
  const int nrows = n * G;
  const int nkeys = ctx + n;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lrow = lane & 31, lh = lane >> 5;

  const int blk0 = ksi * pl.per;
  const int blk_end = min((nkeys + kKB - 1) / kKB, blk0 + pl.per);
  const int nb = blk_end - blk0;

  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
  const uint16_t* kt = static_cast<const uint16_t*>(a.k_tree);
  const uint16_t* vt = static_cast<const uint16_t*>(a.v_tree);

  // ---- this wave's query row and its Q^T fragments (issued before the K/V ring)
  const int r = tile * kRows + wave * 32 + lrow;
  const bool row_ok = r < nrows;
  const int node = row_ok ? r / G : 0;
  const int head = g * G + (row_ok ? r % G : 0);
  u32x4 qv[kHD / 16];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((int64_t(b) * n + node) * H + head) * kHD;
#pragma unroll
    for (int s = 0; s < kHD / 16; ++s) qv[s] = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * lh);
  }

  // ---- direct-load slots: instruction q of this wave fills 1 KB block qb = q * 4 + wave
  // of a stage (K blocks 0..7, V blocks 8..15); lane l: key row (qb & 7) * 4 + l / 16,
  // physical chunk l & 15.  Addresses are plain 64-bit integers and every choice is a
  // select, so a stage's loads form one basic block with no waits between them.
  const uint64_t row_bytes = uint64_t(Hkv) * kHD * 2;
  const uint64_t cache_k = reinterpret_cast<uint64_t>(kc) + (uint64_t(b) * cap * Hkv + g) * kHD * 2;
  const uint64_t cache_v = reinterpret_cast<uint64_t>(vc) + (uint64_t(b) * cap * Hkv + g) * kHD * 2;
  const uint64_t tree_k = reinterpret_cast<uint64_t>(kt) + (uint64_t(b) * n * Hkv + g) * kHD * 2;
  const uint64_t tree_v = reinterpret_cast<uint64_t>(vt) + (uint64_t(b) * n * Hkv + g) * kHD * 2;
  const uint64_t zaddr = reinterpret_cast<uint64_t>(&kZero16[0]);
  int krow[kLpw];
  uint64_t cbase[kLpw], tbase[kLpw], colb[kLpw];
#pragma unroll
  for (int q = 0; q < kLpw; ++q) {
    const int qb = q * kWaves + wave;
    const bool v = qb >= 8;
    krow[q] = (qb & 7) * 4 + (lane >> 4);
    colb[q] = uint64_t(16 * ((lane & 15) ^ (v ? swz_v(krow[q]) : (krow[q] & 15))));
    cbase[q] = v ? cache_v : cache_k;
    tbase[q] = v ? tree_v : tree_k;
  }
  // running address of this lane's chunk in the next block to issue (cache rows)
  uint64_t run[kLpw];
#pragma unroll
  for (int q = 0; q < kLpw; ++q) run[q] = cbase[q] + uint64_t(blk0 * kKB + krow[q]) * row_bytes + colb[q];
  const uint64_t run_step = uint64_t(kKB) * row_bytes;
  // blocks are issued in order blk0, blk0 + 1, ...
  auto issue = [&](int stage, int j) {
    // wave-uniform cases: past the split (zero chunks), all cache keys, or the tail
    const int mode = j >= blk_end ? 0 : ((j + 1) * kKB <= ctx ? 1 : 2);
#pragma unroll
    for (int q = 0; q < kLpw; ++q) {
      const int key = j * kKB + krow[q];
      uint64_t addr = zaddr;
      if (mode == 1) {
        addr = run[q];
      } else if (mode == 2) {
        const uint64_t at = key < ctx ? cbase[q] + uint64_t(key) * row_bytes
                                      : tbase[q] + uint64_t(key - ctx) * row_bytes;
        addr = key < nkeys ? at + colb[q] : zaddr;
      }
      run[q] += run_step;
      const uint32_t dst = lds_base + uint32_t(stage * kStageBytes + (q * kWaves + wave) * 1024);
      // non-temporal (each cache row is read once per step): a streaming probe
      // reads 6.9 TB/s this way against 6.3 with the default policy
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(addr),
                                       reinterpret_cast<__attribute__((address_space(3))) void*>(uintptr_t(dst)),
                                       16, 0, kLoadNt);
    }
  };

  bf16x8 qf[kHD / 16];
#pragma unroll
  for (int s = 0; s < kHD / 16; ++s) qf[s] = __builtin_bit_cast(bf16x8, row_ok ? qv[s] : u32x4{0u, 0u, 0u, 0u});

  const float sc = a.scale * kLog2e;
  float m = -INFINITY, ssum = 0.f;
  f32x16 o[kHD / 32];
#pragma unroll
  for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;

  // per-lane LDS byte offsets inside a stage
  const uint32_t koff_row = uint32_t(lrow * 256);
  uint32_t voff[2][4];   // [half][db]: key row 8 half + 4 lh + (lane & 15) / 4 of a 16-key step, d of this lane
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int db = 0; db < kHD / 32; ++db) {
      const int vr = 8 * half + 4 * lh + ((lane & 15) >> 2);     // + 16 st at use
      const int d = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      // swz_v depends on the key row's low 2 bits only, which 16 st does not change
      voff[half][db] = uint32_t(kKBytes + vr * 256 + (((d >> 3) ^ swz_v(vr)) << 4) + ((d & 7) << 1));
    }

  uint32_t kcol[kHD / 16];   // this lane's K fragment bytes of step st inside a stage
#pragma unroll
  for (int st = 0; st < kHD / 16; ++st) kcol[st] = koff_row + uint32_t(((2 * st + lh) ^ (lrow & 15)) << 4);

  auto compute = [&](int stage, int j) {
    const uint32_t sb = lds_base + uint32_t(stage * kStageBytes);
    // S^T = K . Q^T
    bf16x8 kf[kHD / 16];
    {
      uint32_t ka[kHD / 16];
#pragma unroll
      for (int st = 0; st < kHD / 16; ++st) ka[st] = sb + kcol[st];
      read_k(kf, ka);
    }
    f32x16 s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
    for (int st = 0; st < kHD / 16; ++st) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[st], s, 0, 0, 0);

    // scores: lane holds row lrow, keys 8 (e / 4) + 4 lh + e % 4 of the block
    const int kb = j * kKB;
    const bool full = kb + kKB <= ctx;   // every key of the block is a cache key: nothing is masked
    uint32_t okm = 0xffffu;              // bit e: score e visible
    float bmax;
    if (full) {
      float r = s[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) r = fmaxf(r, s[e]);
      bmax = r * sc;                     // sc > 0
    } else {
      okm = 0;
      bmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kb + 8 * (e >> 2) + 4 * lh + (e & 3);
        // cache keys always, block keys by the clean/noisy rule
        const bool ok = (key < nkeys) & ((key < ctx) | (node >= blk) | (key - ctx <= node));
        okm |= uint32_t(ok) << e;
        bmax = ok ? fmaxf(bmax, s[e] * sc) : bmax;
      }
    }
    bmax = max_xor32(bmax);
    // Lazy rescaling: the running max m moves only when a score exceeds it by
    // more than kLazy (log2 units), so P = 2^(y - m) <= 2^kLazy, and the
    // accumulator is rescaled only in the rare blocks where some row's max moved.
    const bool grow = bmax > m + kLazy;
    if (__ballot(grow) != 0) {
      const float mn = grow ? bmax : m;
      const float alpha = grow ? fexp2(m - mn) : 1.f;   // m = -inf: alpha = 0
      ssum *= alpha;
#pragma unroll
      for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
      m = mn;
    }
    const float nm = m == -INFINITY ? 0.f : -m;   // a row with nothing visible yet: P = 0
    float y[16];
    float psum = 0.f;
    if (full) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        y[e] = fexp2(fmaf(s[e], sc, nm));
        psum += y[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        y[e] = ((okm >> e) & 1u) ? fexp2(fmaf(s[e], sc, nm)) : 0.f;
        psum += y[e];
      }
    }
    psum = sum_xor32(psum);
    ssum += psum;
    bf16x8 pf[2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
      pf[st] = __builtin_bit_cast(bf16x8, u32x4{pk_bf16(y[8 * st + 0], y[8 * st + 1]), pk_bf16(y[8 * st + 2], y[8 * st + 3]),
                                                pk_bf16(y[8 * st + 4], y[8 * st + 5]), pk_bf16(y[8 * st + 6], y[8 * st + 7])});

    // O^T += V^T . P^T; the A fragment of (db, st) is keys 16 st + 4 lh + 0..3
    // (P elements 0..3) and 16 st + 8 + 4 lh + 0..3 (elements 4..7) at d = 32 db + lrow
    uint32_t va[2][kHD / 32];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int db = 0; db < kHD / 32; ++db) va[half][db] = sb + voff[half][db];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      s16x4 t[2][kHD / 32];
      read_vt(t, va, st);
#pragma unroll
      for (int db = 0; db < kHD / 32; ++db) {
        const s16x4 lo = t[0][db], hi = t[1][db];
        const short __attribute__((ext_vector_type(8))) v8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v8), pf[st], o[db], 0, 0, 0);
      }
    }
  };

  auto sync_stage = [&]() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  if (nb > 0) {
#pragma unroll
    for (int s = 0; s + 1 < kStages; ++s) issue(s, blk0 + s);
    wait_vm<(kStages - 2) * kLpw>();   // stage 0 landed (and the Q fragments before it)
    sync_stage();
    for (int i = 0; i < nb; ++i) {
      compute(i % kStages, blk0 + i);
      wait_vm<(kStages - 3) * kLpw>();   // stage i + 1 landed (past the end: zero loads)
      sync_stage();                      // every wave is done with stage i - 1 ...
      issue((i + kStages - 1) % kStages, blk0 + i + kStages - 1);   // ... which is refilled
    }
  }
  // drain the trailing (unused) loads before the workgroup exits
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));

  if (pl.ks > 1) {
    const int64_t prow = (int64_t(grp) * (pl.tiles * kWaves) + tile * kWaves + wave) * 32 + lrow;
    float* dst = part_o + prow * kHD;
#pragma unroll
    for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const f32x4 v = {o[db][4 * gq], o[db][4 * gq + 1], o[db][4 * gq + 2], o[db][4 * gq + 3]};
        *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * gq + 4 * lh) = v;
      }
    if (lh == 0) part_ms[prow] = make_float2(m, ssum);
    return;
  }
  if (row_ok) {
    const float inv = 1.f / ssum;
    uint16_t* orow = static_cast<uint16_t*>(a.out) + ((int64_t(b) * n + node) * H + head) * kHD;
#pragma unroll
    for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = 32 * db + 8 * gq + 4 * lh;
        const uint32_t lo = pack_bf16x2(o[db][4 * gq] * inv, o[db][4 * gq + 1] * inv);
        const uint32_t hi = pack_bf16x2(o[db][4 * gq + 2] * inv, o[db][4 * gq + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d) = make_uint2(lo, hi);
      }
    if (a.out_lse && lh == 0) a.out_lse[(int64_t(b) * n + node) * H + head] = (m + __log2f(ssum)) * kLn2;
  }
}

template <int S>
hipError_t launch_stages(const TreeAttnArgs& a, const BlkPlan& pl, int64_t nwg, float* part_o, float2* part_ms,
                         hipStream_t stream) {
  const size_t lds = size_t(S) * kStageBytes;
  static std::atomic<uint64_t> configured{0};
  {
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(block_attn_kernel<S>), int(lds), configured);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(block_attn_kernel<S>, dim3(unsigned(nwg)), dim3(kThreads), lds, stream, a, pl, part_o, part_ms);
  return hipGetLastError();
}

}  // namespace

size_t block_attention_workspace_bytes(int batch, int block, int ctx, int n_heads, int n_kv) {
  const BlkPlan pl = make_plan(batch, 2 * block, ctx, n_heads, n_kv);
  if (pl.ks == 1) return 0;
  return attn_part_bytes(batch, n_kv, pl.tiles * kWaves, pl.ks);
}

hipError_t launch_block_attention(const TreeAttnArgs& a, hipStream_t stream) {
  const BlkPlan pl = make_plan(a.batch, a.n_tree, a.ctx, a.n_heads, a.n_kv);
  const int64_t padded_groups = (int64_t(pl.groups) + kXcd - 1) / kXcd * kXcd;
  const int64_t nwg = padded_groups * pl.tiles;
  if (nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int tiles32 = pl.tiles * kWaves;
  float* part_o = nullptr;
  float2* part_ms = nullptr;
  if (pl.ks > 1) {
    const size_t rows = size_t(pl.groups) * tiles32 * 32;
    part_o = static_cast<float*>(a.ws);
    part_ms = reinterpret_cast<float2*>(static_cast<char*>(a.ws) + align_up(rows * kHD * sizeof(float), 256));
  }
  int stages = kStagesDefault;
  {
    const char* env = tuning_env("UNO_ATTN_STAGES");   // tuning override: 3..5
    if (env && atoi(env) >= 3 && atoi(env) <= 5) stages = atoi(env);
  }
  hipError_t e = hipSuccess;
  {
    ProfileScope ps("uno_block_attention", stream);
    switch (stages) {
      case 3: e = launch_stages<3>(a, pl, nwg, part_o, part_ms, stream); break;
      case 5: e = launch_stages<5>(a, pl, nwg, part_o, part_ms, stream); break;
      default: e = launch_stages<4>(a, pl, nwg, part_o, part_ms, stream); break;
    }
  }
  if (e != hipSuccess || pl.ks == 1) return e;
  return launch_attn_combine(a, tiles32, pl.ks, a.ws, stream, "uno_block_attention_combine");
}

}  // namespace uno
