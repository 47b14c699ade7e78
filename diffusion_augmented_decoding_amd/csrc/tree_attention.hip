// Tree-masked grouped-query attention for tree verification, gfx950.
//
// Method: Uno summary (hyper.ai, arXiv 2609.04010), section "方法", last
// paragraph -- the tree sampler verifies its candidates concurrently as a
// prefix tree using tree attention.  Node i attends to every cached position
// and to the tree nodes that are its ancestors or itself.
//
// Work unit: 32 query rows of one KV head's group.  Query row r of the group
// is (node r / G, head g*G + r % G), G = H / H_kv, so the G heads sharing a KV
// head share every K/V fetch.  Keys are the ctx cache rows followed by the n
// tree nodes, in blocks of 32.  The key blocks of a unit are split over KS
// workgroups (KS chosen so a decode-sized call still spreads over the chip,
// with every workgroup resident at once) and, inside a workgroup, over its 4
// waves.  All global loads of the set-up (parent ids, query rows, the first
// K/V block) are issued before any of them is used.  Waves
// merge their online-softmax states in LDS; with KS > 1 each workgroup writes
// its merged (max, sum, unnormalised O) to the workspace and a combine kernel
// merges the KS partials of every row in a fixed order.
//
// Per key block, per wave (all on v_mfma_f32_32x32x16_bf16):
//   S^T[key][row] = K_blk . Q^T : the K rows are head_dim-contiguous, so each
//                   lane's A operand is a direct 16-byte global load;
//   online softmax in the log2 domain, lane l owning query row l % 32 (the
//                   other 16 keys of the block are in lane l ^ 32);
//   O^T[d][row]  += V_blk^T . P^T : P is the lane's own scores (the key order
//                   inside a 16-key step is a permutation shared by both
//                   operands); V is staged transposed in a per-wave LDS tile
//                   so its operand is two 8-byte LDS reads.  Keeping O
//                   transposed leaves the rescale by exp2(m_old - m_new) local
//                   to the lane that owns the row.
// The tree mask is an ancestor-or-self bitset per node (<= 256 nodes) in LDS,
// built from the parent array staged in LDS.
//
// Workgroups are numbered so that the tiles sharing one (batch, KV head, key
// split) land on one XCD (hardware deals workgroups to the 8 XCDs round
// robin): their common K/V blocks are fetched into that XCD's L2 once.
#include <stdlib.h>

#include "device_common.h"
#include "internal.h"

namespace uno {

namespace {

constexpr int kHD = 128;
constexpr int kKB = 32;                 // keys per block
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kMaxNodes = 256;
static_assert(kMaxNodes <= kThreads, "one thread per tree node in the set-up");
constexpr int kVtStride = 36;           // bf16 per transposed-V row (32 keys + pad)
constexpr int kXcd = 8;
constexpr int kTargetWgs = 256;         // 1 resident workgroup per CU (register-bound with the prefetch)
constexpr int kMrgStride = kHD + 4;     // fp32 row stride of the merge buffer (bank spread)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

struct AttnPlan {
  int tiles;    // 32-row tiles per (batch, KV head)
  int ks;       // key splits
  int groups;   // batch * n_kv * ks
  int nblk;     // key blocks
};

AttnPlan make_plan(int batch, int n, int ctx, int H, int Hkv) {
  AttnPlan p;
  const int G = H / Hkv;
  p.tiles = (n * G + 31) / 32;
  p.nblk = (ctx + n + kKB - 1) / kKB;
  const int64_t base = int64_t(p.tiles) * Hkv * batch;
  int64_t target = kTargetWgs;
  if (const char* env = tuning_env("UNO_TREE_ATTN_WGS")) target = atoi(env);   // tuning build only
  int ks = 1;
  if (base < target) {
    ks = int(target / base);          // every workgroup resident at once
    const int most = (p.nblk + kWaves - 1) / kWaves;   // at least one block per wave
    if (ks > most) ks = most;
    if (ks < 1) ks = 1;
  }
  p.ks = ks;
  p.groups = batch * Hkv * ks;
  return p;
}

// Partial results of one split: [group][tile][32 rows] x (m, s) and
// x O[128] (fp32, unnormalised).
struct AttnPart {
  float* o;
  float2* ms;
};

AttnPart part_ws(void* base, const AttnPlan& p) {
  const size_t rows = size_t(p.groups) * p.tiles * 32;
  AttnPart w;
  w.o = static_cast<float*>(base);
  w.ms = reinterpret_cast<float2*>(static_cast<char*>(base) + align_up(rows * kHD * sizeof(float), 256));
  return w;
}

size_t part_bytes(const AttnPlan& p) {
  if (p.ks == 1) return 0;
  const size_t rows = size_t(p.groups) * p.tiles * 32;
  return align_up(rows * kHD * sizeof(float), 256) + align_up(rows * sizeof(float2), 256);
}

__global__ __launch_bounds__(kThreads) void tree_attn_kernel(TreeAttnArgs a, AttnPlan pl, AttnPart part) {
  __shared__ uint64_t anc[kMaxNodes][4];
  __shared__ int sh_par[kMaxNodes];
  __shared__ int sh_bad;
  __shared__ __align__(16) uint16_t vt[kWaves][kHD * kVtStride];   // 36 KB, reused for the merge
  __shared__ float mrg_m[kWaves][32], mrg_s[kWaves][32];

  // ---- work unit (XCD-grouped numbering; the grid is padded to a multiple of 8 groups)
  const int L = blockIdx.x;
  const int slot = L / kXcd;
  const int tile = slot % pl.tiles;
  const int grp = (slot / pl.tiles) * kXcd + L % kXcd;
  if (grp >= pl.groups) return;
  const int ksi = grp % pl.ks;
  const int g = (grp / pl.ks) % a.n_kv;
  const int b = grp / (pl.ks * a.n_kv);

  const int n = a.n_tree, ctx = a.ctx, H = a.n_heads, Hkv = a.n_kv;
  const int G = H / Hkv;
  const int nrows = n * G;
  const int row0 = tile * 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid / kWave;
  const int lrow = lane & 31, lh = lane >> 5;
  const int nkeys = ctx + n;

  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
  const uint16_t* kt = static_cast<const uint16_t*>(a.k_tree);
  const uint16_t* vtr = static_cast<const uint16_t*>(a.v_tree);

  // this wave's key blocks: j = ksi*4 + wave + i*(ks*4)
  const int stride = pl.ks * kWaves;
  const int j0 = ksi * kWaves + wave;
  const int nb = j0 < pl.nblk ? (pl.nblk - 1 - j0) / stride + 1 : 0;

  // K fragment rows of a block (key kb + lrow, dims 16 st + 8 lh) and the V
  // chunks (chunk lane + 64 t -> key (lane & 31), dims 8 ((lane >> 5) + 2 t));
  // keys past the end read the last key (finite values, masked scores).
  auto key_row = [&](const uint16_t* cache, const uint16_t* tree, int key) {
    key = min(key, nkeys - 1);
    return key < ctx ? cache + ((int64_t(b) * ctx + key) * Hkv + g) * kHD
                     : tree + ((int64_t(b) * n + (key - ctx)) * Hkv + g) * kHD;
  };
  auto load_block = [&](int j, u32x4 (&kr)[8], u32x4 (&vr)[8]) {
    const int kb = j * kKB;
    const uint16_t* krow = key_row(kc, kt, kb + lrow);
#pragma unroll
    for (int st = 0; st < 8; ++st) kr[st] = *reinterpret_cast<const u32x4*>(krow + 16 * st + 8 * lh);
    const uint16_t* vrow = key_row(vc, vtr, kb + lrow);
#pragma unroll
    for (int t = 0; t < 8; ++t) vr[t] = *reinterpret_cast<const u32x4*>(vrow + 8 * (lh + 2 * t));
  };

  // ---- every global load of the set-up is issued first: parent ids, this
  // lane's query row, the first K/V block
  const int par_i = tid < n ? a.parent[int64_t(b) * n + tid] : 0;   // n <= kThreads
  const int r = row0 + lrow;
  const bool row_ok = r < nrows;
  const int node = row_ok ? r / G : 0;
  const int head = g * G + (row_ok ? r % G : 0);
  u32x4 qv[kHD / 16];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((int64_t(b) * n + node) * H + head) * kHD;
#pragma unroll
    for (int s = 0; s < kHD / 16; ++s) qv[s] = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * lh);
  }
  u32x4 kr[8], vr[8];
  if (nb > 0) load_block(j0, kr, vr);

  // ---- parent array to LDS, then ancestor-or-self bitsets (one thread per node)
  if (tid == 0) sh_bad = 0;
  if (tid < n) sh_par[tid] = par_i;
  __syncthreads();
  if (tid < n) {
    const int i = tid;
    uint64_t w[4] = {0, 0, 0, 0};
    int j = i, steps = 0;
    bool bad = false;
    while (true) {
      w[j >> 6] |= uint64_t(1) << (j & 63);
      const int pj = sh_par[j];
      if (j == 0) {
        bad = (pj != -1);
        break;
      }
      if (pj < 0 || pj >= j || ++steps > n) {
        bad = true;
        break;
      }
      j = pj;
    }
    if (bad) sh_bad = 1;
    anc[i][0] = w[0];
    anc[i][1] = w[1];
    anc[i][2] = w[2];
    anc[i][3] = w[3];
  }
  __syncthreads();
  const bool bad_tree = sh_bad != 0;

  bf16x8 qf[kHD / 16];
#pragma unroll
  for (int s = 0; s < kHD / 16; ++s) qf[s] = __builtin_bit_cast(bf16x8, row_ok ? qv[s] : u32x4{0u, 0u, 0u, 0u});
  const uint64_t my_anc0 = anc[node][0], my_anc1 = anc[node][1], my_anc2 = anc[node][2], my_anc3 = anc[node][3];

  const float sc = a.scale * kLog2e;
  float m = -INFINITY, ssum = 0.f;
  f32x16 o[kHD / 32];
#pragma unroll
  for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;

  uint16_t* myvt = vt[wave];
  for (int i = 0, j = j0; i < nb; ++i, j += stride) {
    // the wave's next key block is loaded while this one is computed
    u32x4 kn[8], vn[8];
    if (i + 1 < nb) load_block(j + stride, kn, vn);
    const u32x4(&kcur)[8] = kr;
    const u32x4(&vcur)[8] = vr;
    const int kb = j * kKB;

    f32x16 s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
    for (int st = 0; st < kHD / 16; ++st)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kcur[st]), qf[st], s, 0, 0, 0);
    // ---- stage V transposed: chunk t holds key lrow, dims 8 (lh + 2t) .. +8
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int dc = lh + 2 * t;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        myvt[(8 * dc + 2 * e) * kVtStride + lrow] = uint16_t(vcur[t][e] & 0xffffu);
        myvt[(8 * dc + 2 * e + 1) * kVtStride + lrow] = uint16_t(vcur[t][e] >> 16);
      }
    }
    // ---- scores: lane holds row lrow, keys 8(e/4) + 4lh + e%4
    float y[16];
    float bmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kb + 8 * (e >> 2) + 4 * lh + (e & 3);
      bool ok = key < nkeys;
      if (ok && key >= ctx) {
        const int t = key - ctx;
        const uint64_t word = (t < 64) ? my_anc0 : (t < 128) ? my_anc1 : (t < 192) ? my_anc2 : my_anc3;
        ok = (word >> (t & 63)) & 1u;
      }
      y[e] = ok ? s[e] * sc : -INFINITY;
      bmax = fmaxf(bmax, y[e]);
    }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const float mn = fmaxf(m, bmax);
    float alpha = 1.f, psum = 0.f;
    bf16x8 pf[2];
    if (mn == -INFINITY) {
#pragma unroll
      for (int e = 0; e < 16; ++e) y[e] = 0.f;
    } else {
      alpha = fexp2(m - mn);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        y[e] = fexp2(y[e] - mn);
        psum += y[e];
      }
    }
    psum += __shfl_xor(psum, 32);
    ssum = ssum * alpha + psum;
    m = mn;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      uint32_t w0 = pack_bf16x2(y[8 * st + 0], y[8 * st + 1]);
      uint32_t w1 = pack_bf16x2(y[8 * st + 2], y[8 * st + 3]);
      uint32_t w2 = pack_bf16x2(y[8 * st + 4], y[8 * st + 5]);
      uint32_t w3 = pack_bf16x2(y[8 * st + 6], y[8 * st + 7]);
      pf[st] = __builtin_bit_cast(bf16x8, u32x4{w0, w1, w2, w3});
    }
#pragma unroll
    for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
    wave_sync_lds();
    // ---- O^T[d][row] += V^T[d][keys] P^T[keys][row]
#pragma unroll
    for (int db = 0; db < kHD / 32; ++db) {
      const int d = 32 * db + lrow;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const uint16_t* src = myvt + d * kVtStride + 16 * st + 4 * lh;
        const uint2 lo = *reinterpret_cast<const uint2*>(src);
        const uint2 hi = *reinterpret_cast<const uint2*>(src + 8);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[st], o[db], 0, 0, 0);
      }
    }
    wave_sync_lds();
    if (i + 1 < nb) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        kr[t] = kn[t];
        vr[t] = vn[t];
      }
    }
  }

  // ---- merge the 4 waves' states: (2,3) -> (0,1), then 1 -> 0; vt reused as fp32 [32 rows][128 d]
  __syncthreads();
  float* ob = reinterpret_cast<float*>(&vt[0][0]);    // room for 2 x 32 x kMrgStride floats
  static_assert(2 * 32 * kMrgStride * sizeof(float) <= sizeof(vt), "merge buffer fits in the V tiles");
#pragma unroll
  for (int round = 0; round < 2; ++round) {
    const int writers_lo = (round == 0) ? 2 : 1, writers_hi = (round == 0) ? 4 : 2;
    if (wave >= writers_lo && wave < writers_hi) {
      float* dst = ob + (wave - writers_lo) * 32 * kMrgStride;
      if (lh == 0) {
        mrg_m[wave][lrow] = m;
        mrg_s[wave][lrow] = ssum;
      }
#pragma unroll
      for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) dst[lrow * kMrgStride + 32 * db + 8 * (e >> 2) + 4 * lh + (e & 3)] = o[db][e];
    }
    __syncthreads();
    if (wave < writers_lo) {
      const int src_w = wave + writers_lo;
      const float* src = ob + wave * 32 * kMrgStride;
      const float m2 = mrg_m[src_w][lrow], s2 = mrg_s[src_w][lrow];
      const float mn = fmaxf(m, m2);
      const float a1 = (mn == -INFINITY) ? 0.f : fexp2(m - mn);
      const float a2 = (mn == -INFINITY) ? 0.f : fexp2(m2 - mn);
      ssum = ssum * a1 + s2 * a2;
      m = mn;
#pragma unroll
      for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          o[db][e] = o[db][e] * a1 + src[lrow * kMrgStride + 32 * db + 8 * (e >> 2) + 4 * lh + (e & 3)] * a2;
    }
    __syncthreads();
  }
  if (wave != 0) return;

  if (pl.ks > 1) {
    // partial of this split; a bad tree is passed on as a NaN max
    const int64_t prow = (int64_t(grp) * pl.tiles + tile) * 32 + lrow;
    float* dst = part.o + prow * kHD;
#pragma unroll
    for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const f32x4 v = {o[db][4 * gq], o[db][4 * gq + 1], o[db][4 * gq + 2], o[db][4 * gq + 3]};
        *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * gq + 4 * lh) = v;
      }
    if (lh == 0) part.ms[prow] = make_float2(bad_tree ? __builtin_nanf("") : m, ssum);
    return;
  }

  if (row_ok) {
    const float inv = bad_tree ? __builtin_nanf("") : 1.f / ssum;
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
    if (a.out_lse && lh == 0)
      a.out_lse[(int64_t(b) * n + node) * H + head] = bad_tree ? __builtin_nanf("") : (m + __log2f(ssum)) * kLn2;
  }
}

// Merge of the KS split partials of 8 rows per workgroup, ks ascending
// (the result is M = max m_k, S = sum s_k 2^(m_k - M),
// O = sum O_k 2^(m_k - M) / S).
// Thread t: row 8 * (blockIdx.x % 4) + t / 32 of the tile, dims 4 (t % 32) .. +4.
constexpr int kCombineThreads = 256;

__global__ __launch_bounds__(kCombineThreads) void tree_attn_combine_kernel(TreeAttnArgs a, AttnPlan pl,
                                                                            AttnPart part) {
  const int tile = blockIdx.x / 4, quarter = blockIdx.x % 4;
  const int g = blockIdx.y, b = blockIdx.z;
  const int G = a.n_heads / a.n_kv;
  const int rin = quarter * 8 + threadIdx.x / 32;
  const int r = tile * 32 + rin;
  if (r >= a.n_tree * G) return;
  const int d0 = 4 * (threadIdx.x % 32);
  const int node = r / G, head = g * G + r % G;
  const int64_t grp0 = (int64_t(b) * a.n_kv + g) * pl.ks;
  auto prow = [&](int k) { return ((grp0 + k) * pl.tiles + tile) * 32 + rin; };

  // online merge, 8 partials per step with all 16 loads of a step in flight
  float M = -INFINITY, S = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  bool bad = false;
  for (int k0 = 0; k0 < pl.ks; k0 += 8) {
    float2 ms[8];
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t pr = prow(min(k0 + u, pl.ks - 1));   // past the end: unused
      ms[u] = part.ms[pr];
      v[u] = *reinterpret_cast<const f32x4*>(part.o + pr * kHD + d0);
    }
    float mb = M;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (k0 + u < pl.ks) {
        bad |= __builtin_isnan(ms[u].x);
        mb = fmaxf(mb, ms[u].x);
      }
    const float resc = (M == -INFINITY) ? 0.f : fexp2(M - mb);
    S *= resc;
    acc *= resc;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (k0 + u < pl.ks) {
        const float w = (ms[u].x == -INFINITY) ? 0.f : fexp2(ms[u].x - mb);
        S += ms[u].y * w;
        acc += v[u] * w;
      }
    M = mb;
  }
  const float inv = bad ? __builtin_nanf("") : 1.f / S;
  uint16_t* orow = static_cast<uint16_t*>(a.out) + ((int64_t(b) * a.n_tree + node) * a.n_heads + head) * kHD;
  *reinterpret_cast<uint2*>(orow + d0) =
      make_uint2(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv));
  if (a.out_lse && d0 == 0)
    a.out_lse[(int64_t(b) * a.n_tree + node) * a.n_heads + head] =
        bad ? __builtin_nanf("") : (M + __log2f(S)) * kLn2;
}

}  // namespace

size_t attn_part_bytes(int batch, int n_kv, int tiles32, int ks) {
  AttnPlan pl{};
  pl.tiles = tiles32;
  pl.ks = ks;
  pl.groups = batch * n_kv * ks;
  return part_bytes(pl);
}

hipError_t launch_attn_combine(const TreeAttnArgs& a, int tiles32, int ks, void* ws, hipStream_t stream,
                               const char* name) {
  AttnPlan pl{};
  pl.tiles = tiles32;
  pl.ks = ks;
  pl.groups = a.batch * a.n_kv * ks;
  const AttnPart part = part_ws(ws, pl);
  ProfileScope ps(name, stream);
  hipLaunchKernelGGL(tree_attn_combine_kernel, dim3(tiles32 * 4, a.n_kv, a.batch), dim3(kCombineThreads), 0, stream,
                     a, pl, part);
  return hipGetLastError();
}

size_t tree_attention_workspace_bytes(int batch, int n_tree, int ctx, int n_heads, int n_kv, int) {
  return part_bytes(make_plan(batch, n_tree, ctx, n_heads, n_kv));
}

hipError_t launch_tree_attention(const TreeAttnArgs& a, hipStream_t stream) {
  const AttnPlan pl = make_plan(a.batch, a.n_tree, a.ctx, a.n_heads, a.n_kv);
  const AttnPart part = pl.ks > 1 ? part_ws(a.ws, pl) : AttnPart{nullptr, nullptr};
  const int64_t padded_groups = (int64_t(pl.groups) + kXcd - 1) / kXcd * kXcd;
  const int64_t nwg = padded_groups * pl.tiles;
  if (nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
  {
    ProfileScope ps("uno_tree_attention", stream);
    hipLaunchKernelGGL(tree_attn_kernel, dim3(unsigned(nwg)), dim3(kThreads), 0, stream, a, pl, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.ks == 1) return e;
  {
    ProfileScope ps("uno_tree_attention_combine", stream);
    hipLaunchKernelGGL(tree_attn_combine_kernel, dim3(pl.tiles * 4, a.n_kv, a.batch), dim3(kCombineThreads), 0,
                       stream, a, pl, part);
  }
  return hipGetLastError();
}

}  // namespace uno
