// Tree-masked grouped-query attention for tree verification, gfx950.
//
// Method: Uno summary (hyper.ai, arXiv 2609.04010), section "方法", last
// paragraph -- the tree sampler verifies its candidates concurrently as a
// prefix tree using tree attention.  Node i attends to every cached position
// and to the tree nodes that are its ancestors or itself.
//
// One workgroup per (32 query rows of one KV head's group, KV head, batch).
// Query row r of the group is (node r / G, head g*G + r % G), G = H / H_kv, so
// the G heads sharing a KV head share every K/V fetch.  Keys are the ctx cache
// rows followed by the n tree nodes, in blocks of 32; the 4 waves take every
// 4th block and merge their online-softmax states in LDS at the end.
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
// The tree mask is an ancestor-or-self bitset per node (<= 256 nodes) in LDS.
#include "device_common.h"
#include "internal.h"

namespace uno {

namespace {

constexpr int kHD = 128;
constexpr int kKB = 32;                 // keys per block
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kMaxNodes = 256;
constexpr int kVtStride = 36;           // bf16 per transposed-V row (32 keys + pad)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__global__ __launch_bounds__(kThreads) void tree_attn_kernel(TreeAttnArgs a) {
  __shared__ uint64_t anc[kMaxNodes][4];
  __shared__ int sh_bad;
  __shared__ __align__(16) uint16_t vt[kWaves][kHD * kVtStride];   // 36 KB, reused for the merge
  __shared__ float mrg_m[kWaves][32], mrg_s[kWaves][32];

  const int n = a.n_tree, ctx = a.ctx, H = a.n_heads, Hkv = a.n_kv;
  const int G = H / Hkv;
  const int nrows = n * G;
  const int row0 = blockIdx.x * 32;
  const int g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid / kWave;
  const int lrow = lane & 31, lh = lane >> 5;

  // ---- ancestor-or-self bitsets, one thread per node (walks its chain)
  if (tid == 0) sh_bad = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kThreads) {
    uint64_t w[4] = {0, 0, 0, 0};
    int j = i, steps = 0;
    bool bad = false;
    while (true) {
      w[j >> 6] |= uint64_t(1) << (j & 63);
      const int pj = a.parent[int64_t(b) * n + j];
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

  // ---- this lane's query row
  const int r = row0 + lrow;
  const bool row_ok = r < nrows;
  const int node = row_ok ? r / G : 0;
  const int head = g * G + (row_ok ? r % G : 0);
  bf16x8 qf[kHD / 16];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((int64_t(b) * n + node) * H + head) * kHD;
#pragma unroll
    for (int s = 0; s < kHD / 16; ++s) {
      u32x4 v = row_ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * lh) : u32x4{0u, 0u, 0u, 0u};
      qf[s] = __builtin_bit_cast(bf16x8, v);
    }
  }
  const uint64_t my_anc0 = anc[node][0], my_anc1 = anc[node][1], my_anc2 = anc[node][2], my_anc3 = anc[node][3];

  const float sc = a.scale * kLog2e;
  float m = -INFINITY, ssum = 0.f;
  f32x16 o[kHD / 32];
#pragma unroll
  for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;

  const int nkeys = ctx + n;
  const int nblk = (nkeys + kKB - 1) / kKB;
  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
  const uint16_t* kt = static_cast<const uint16_t*>(a.k_tree);
  const uint16_t* vtr = static_cast<const uint16_t*>(a.v_tree);
  uint16_t* myvt = vt[wave];

  for (int blk = wave; blk < nblk; blk += kWaves) {
    const int kb = blk * kKB;
    // ---- K fragments (A operand): key kb + lrow, dims 16s + 8lh .. +8
    const int kj = kb + lrow;
    const uint16_t* krow = nullptr;
    if (kj < ctx)
      krow = kc + ((int64_t(b) * ctx + kj) * Hkv + g) * kHD;
    else if (kj < nkeys)
      krow = kt + ((int64_t(b) * n + (kj - ctx)) * Hkv + g) * kHD;
    f32x16 s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
    for (int st = 0; st < kHD / 16; ++st) {
      u32x4 v = krow ? *reinterpret_cast<const u32x4*>(krow + 16 * st + 8 * lh) : u32x4{0u, 0u, 0u, 0u};
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v), qf[st], s, 0, 0, 0);
    }
    // ---- stage V block transposed: chunk id c = lane + 64 t -> key c % 32, dims 8 (c / 32) ..
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int cid = lane + kWave * t;
      const int key = cid & 31, dc = cid >> 5;
      const int vj = kb + key;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (vj < ctx)
        v = *reinterpret_cast<const u32x4*>(vc + ((int64_t(b) * ctx + vj) * Hkv + g) * kHD + 8 * dc);
      else if (vj < nkeys)
        v = *reinterpret_cast<const u32x4*>(vtr + ((int64_t(b) * n + (vj - ctx)) * Hkv + g) * kHD + 8 * dc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        myvt[(8 * dc + 2 * e) * kVtStride + key] = uint16_t(v[e] & 0xffffu);
        myvt[(8 * dc + 2 * e + 1) * kVtStride + key] = uint16_t(v[e] >> 16);
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
  }

  // ---- merge the 4 waves' states: (2,3) -> (0,1), then 1 -> 0; vt reused as fp32 [32 rows][128 d]
  __syncthreads();
  float* ob = reinterpret_cast<float*>(&vt[0][0]);    // room for 2 x 32 x 128 floats
#pragma unroll
  for (int round = 0; round < 2; ++round) {
    const int writers_lo = (round == 0) ? 2 : 1, writers_hi = (round == 0) ? 4 : 2;
    if (wave >= writers_lo && wave < writers_hi) {
      float* dst = ob + (wave - writers_lo) * 32 * kHD;
      if (lh == 0) {
        mrg_m[wave][lrow] = m;
        mrg_s[wave][lrow] = ssum;
      }
#pragma unroll
      for (int db = 0; db < kHD / 32; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) dst[lrow * kHD + 32 * db + 8 * (e >> 2) + 4 * lh + (e & 3)] = o[db][e];
    }
    __syncthreads();
    if (wave < writers_lo) {
      const int src_w = wave + writers_lo;
      const float* src = ob + wave * 32 * kHD;
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
          o[db][e] = o[db][e] * a1 + src[lrow * kHD + 32 * db + 8 * (e >> 2) + 4 * lh + (e & 3)] * a2;
    }
    __syncthreads();
  }

  if (wave == 0 && row_ok) {
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

}  // namespace

size_t tree_attention_workspace_bytes(int, int, int, int, int, int) { return 0; }

hipError_t launch_tree_attention(const TreeAttnArgs& a, hipStream_t stream) {
  const int G = a.n_heads / a.n_kv;
  const int rows = a.n_tree * G;
  dim3 grid((rows + 31) / 32, a.n_kv, a.batch);
  ProfileScope ps("uno_tree_attention", stream);
  hipLaunchKernelGGL(tree_attn_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace uno
