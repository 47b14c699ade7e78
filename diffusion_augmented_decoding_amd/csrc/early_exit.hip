// Psi-Spec linear verify with early exit, for gfx950.
//
// Method: Uno summary (hyper.ai, arXiv 2609.04010), section "方法", last
// paragraph -- rejection sampling of a drafted block against the AR
// distribution, longest accepted prefix, correction from the residual
// (standard speculative sampling, Leviathan et al. 2023).  Drafts are tested
// in order and the first rejection ends the block, so the rows of positions
// after it never influence the result; this variant does not read them.
//
// Same outputs as the full verify (accepted length, correction or bonus
// token, residual mass), up to the rounding of the row statistics, which
// are summed over 8192-element chunks here.  Two launches before the draw:
//  1. init: every published word set to its sentinel, position 0 of every
//     sequence live, the work counter and the error flag to 0;
//  2. flow: blocks take work items in increasing order from a counter.  For
//     each position i = 0..k in turn: one item per (sequence, row, chunk)
//     -- rows p_i and q_i (p_k alone at i = k) -- then one decision item
//     per sequence.  A chunk item first waits until its sequence's position
//     i is known to be live or dead; a live one publishes the chunk's
//     softmax partial (max, sum of 2^(y - max)) as one 64-bit word, a dead
//     one reads nothing.  The decision item of (sequence, i) merges the
//     partials in chunk order (one wave, fixed order), runs the accept test
//     of draft i, and publishes whether position i + 1 is live; at the first
//     rejection (or at i = k) it writes the accepted length and the
//     descriptor of the row pair the correction (or bonus) is drawn from.
//     An item waits only for words that items with smaller numbers publish,
//     and every counter hands out its items in increasing order (in claims of
//     consecutive items, each processed in order), so the item
//     with the smallest number in progress always has its inputs and the
//     launch finishes for any number of resident blocks (at least one per
//     counter: the grid is a multiple of the counter count).
//  3-4. the draw kernels of the full verify, on those descriptors.
#include <algorithm>

#include "sampler_common.h"

namespace uno {

namespace {

constexpr uint64_t kPartUnset = 0xbf80000000000000ull;   // s = -1.0f in the high word: not yet written
constexpr int kEeSpinMax = 1 << 22;                       // waits end long before; a bound, not a timeout
// Work counters: item it belongs to counter it % kQueues and is its
// (it / kQueues)-th item; block x takes items from counter x % kQueues.  One
// counter on one address serialises every block's atomic (~11 ns each); each
// counter sits on its own 128-byte line.
constexpr int kQueues = 16;
constexpr int kQueueStride = 32;   // ints per counter line
constexpr int kBatch = 8;          // consecutive items of a counter claimed by one atomic

struct EeWs {
  uint64_t* part;   // [batch][2k+1][nchunk]: (m, s) packed, low word m, high word s
  int* live;        // [batch][k+2]: -1 unknown, 0 dead, 1 live
  int* queue;       // work counters (kQueues lines); err: a wait ran past its bound (never expected)
  int* err;
  DrawDesc* desc;   // [batch]
  float* seg;
};

EeWs ee_ws(void* base, int batch, int k, int vocab) {
  const int nc = num_chunks(vocab);
  char* p = static_cast<char*>(base);
  EeWs w;
  w.part = reinterpret_cast<uint64_t*>(p);
  p += align_up(size_t(batch) * (2 * k + 1) * nc * sizeof(uint64_t), 256);
  w.live = reinterpret_cast<int*>(p);
  p += align_up(size_t(batch) * (k + 2) * sizeof(int), 256);
  w.queue = reinterpret_cast<int*>(p);
  w.err = w.queue + kQueues * kQueueStride;
  p += align_up(size_t(kQueues + 1) * kQueueStride * sizeof(int), 256);
  w.desc = reinterpret_cast<DrawDesc*>(p);
  p += align_up(size_t(batch) * sizeof(DrawDesc), 256);
  w.seg = reinterpret_cast<float*>(p);
  return w;
}

__device__ __forceinline__ uint64_t ld_word(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_word(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_int(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_int(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t pack_part(float2 r) {
  return (uint64_t(__float_as_uint(r.y)) << 32) | __float_as_uint(r.x);
}

__global__ __launch_bounds__(kChunkThreads) void ee_init_kernel(int batch, int k, int nc, EeWs w) {
  const int64_t nparts = int64_t(batch) * (2 * k + 1) * nc;
  const int64_t nlive = int64_t(batch) * (k + 2);
  const int64_t stride = int64_t(gridDim.x) * kChunkThreads;
  for (int64_t t = int64_t(blockIdx.x) * kChunkThreads + threadIdx.x; t < nparts + nlive; t += stride) {
    if (t < nparts)
      w.part[t] = kPartUnset;
    else
      w.live[t - nparts] = ((t - nparts) % (k + 2)) == 0 ? 1 : -1;   // position 0 of every sequence is live
  }
  // no draw until a decision writes the descriptor (a sequence whose decision
  // never came would get token -1, not a draw from stale pointers)
  for (int64_t t = int64_t(blockIdx.x) * kChunkThreads + threadIdx.x; t < batch; t += stride) {
    w.desc[t].prow = nullptr;
    w.desc[t].qrow = nullptr;
    w.desc[t].active = 0;
  }
  if (blockIdx.x == 0 && threadIdx.x <= kQueues) w.queue[threadIdx.x * kQueueStride] = 0;   // counters, then err
}

// Whether position i of sequence b is live, once the decision of position
// i - 1 has published it; the whole block calls it (thread 0 polls).
__device__ __forceinline__ bool wait_live(const EeWs& w, int k, int b, int i, int* sh) {
  if (threadIdx.x == 0) {
    const int* f = w.live + int64_t(b) * (k + 2) + i;
    int v = ld_int(f);
    for (int it = 0; v < 0; ++it) {
      if (it == kEeSpinMax) {
        atomicOr(w.err, 1);
        v = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
      v = ld_int(f);
    }
    *sh = v;
  }
  __syncthreads();
  const bool live = *sh > 0;
  __syncthreads();
  return live;
}

// Merge of one row's published chunk partials by one whole wave, once every
// one of them is written: lane l folds chunks l, l + 64, ... in order, then
// a butterfly (same bits in every lane).
__device__ __forceinline__ float2 wave_merge_published(const uint64_t* part, int nc, int* err) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int it = 0;; ++it) {
    bool missing = false;
    for (int c = lane; c < nc; c += kWave) missing |= ld_word(part + c) == kPartUnset;
    if (!wave_ballot(missing)) break;
    if (it == kEeSpinMax) {
      if (lane == 0) atomicOr(err, 1);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  float m = -INFINITY, s = 0.f;
  for (int c = lane; c < nc; c += kWave) {
    const uint64_t v = ld_word(part + c);
    lse2_merge(m, s, __uint_as_float(uint32_t(v)), __uint_as_float(uint32_t(v >> 32)));
  }
  wave_lse2(m, s);
  return make_float2(m, s);
}

template <typename T>
__device__ __forceinline__ const T* ee_row(const VerifyLinearArgs& a, int b, int r) {   // r <= k: p row r, else q row r - k - 1
  if (r <= a.k) return static_cast<const T*>(a.p) + int64_t(b) * a.p_seq + int64_t(r) * a.p_row;
  return static_cast<const T*>(a.q) + int64_t(b) * a.q_seq + int64_t(r - a.k - 1) * a.q_row;
}

// Decision of (sequence b, position i), by one whole wave (no barriers inside).
template <typename T>
__device__ __forceinline__ void decision_item(const VerifyLinearArgs& a, const EeWs& w, int b, int i) {
  const int k = a.k, V = a.vocab, nc = num_chunks(V), rps = 2 * k + 1;
  const int lane = threadIdx.x & (kWave - 1);
  const float sl2 = a.scale_log2;
  int* live_next = w.live + int64_t(b) * (k + 2) + i + 1;
  const int* live_here = w.live + int64_t(b) * (k + 2) + i;
  int lv = ld_int(live_here);   // published by a smaller item; bounded wait all the same
  for (int t = 0; lv < 0; ++t) {
    if (t == kEeSpinMax) {
      if (lane == 0) atomicOr(w.err, 1);
      lv = 0;
      break;
    }
    __builtin_amdgcn_s_sleep(2);
    lv = ld_int(live_here);
  }
  if (lv <= 0) {   // an earlier draft was rejected: position i + 1 is dead too
    if (lane == 0) {
      if (i < k) {
        if (a.out_pd) a.out_pd[int64_t(b) * k + i] = __builtin_nanf("");
        if (a.out_qd) a.out_qd[int64_t(b) * k + i] = __builtin_nanf("");
      }
      st_int(live_next, 0);
    }
    return;
  }
  const float2 sp = wave_merge_published(w.part + (int64_t(b) * rps + i) * nc, nc, w.err);
  const float2 sq = i < k ? wave_merge_published(w.part + (int64_t(b) * rps + k + 1 + i) * nc, nc, w.err)
                          : make_float2(0.f, 0.f);
  if (lane != 0) return;
  bool rej = false;
  if (i < k) {
    const int d = a.drafts[int64_t(b) * a.drafts_seq + i];
    const bool in_range = d >= 0 && d < V;
    const float xp = in_range ? load_logit<T>(ee_row<T>(a, b, i), d) : -INFINITY;
    const float xq = in_range ? load_logit<T>(ee_row<T>(a, b, k + 1 + i), d) : -INFINITY;
    const float pd = fast_exp2(fmaf(xp, sl2, -sp.x)) / sp.y;
    const float qd = fast_exp2(fmaf(xq, sl2, -sq.x)) / sq.y;
    rej = !(a.u_acc[int64_t(b) * k + i] * qd < pd);
    if (a.out_pd) a.out_pd[int64_t(b) * k + i] = pd;
    if (a.out_qd) a.out_qd[int64_t(b) * k + i] = qd;
  }
  if (rej || i == k) {   // the block ends here: L = i
    a.out_len[b] = i;
    DrawDesc dd;
    dd.prow = ee_row<T>(a, b, i);
    dd.mp = sp.x;
    dd.inv_sp = 1.f / sp.y;
    if (i < k) {
      dd.qrow = ee_row<T>(a, b, k + 1 + i);
      dd.mq = sq.x;
      dd.inv_sq = 1.f / sq.y;
      dd.c = 1.f;
    } else {
      dd.qrow = dd.prow;
      dd.mq = 0.f;
      dd.inv_sq = 0.f;
      dd.c = 0.f;
    }
    dd.active = 1;
    w.desc[b] = dd;
  }
  if (i < k) st_int(live_next, rej ? 0 : 1);
}

// Every item is one structured branch of the loop body, closed by one block
// barrier: no `continue` out of lane- or wave-divergent code, so every wave
// of the block passes the same barriers in the same order.
template <typename T>
__global__ __launch_bounds__(kChunkThreads) void ee_flow_kernel(VerifyLinearArgs a, EeWs w) {
  __shared__ int sh_item, sh_live;
  const int B = a.batch, k = a.k, V = a.vocab, nc = num_chunks(V);
  const int rps = 2 * k + 1;
  // position i < k: B * 2 * nc chunk items, then B decisions; position k: B * nc, then B
  const int per_pos = B * 2 * nc + B;
  const int total = k * per_pos + B * nc + B;
  const int qid = blockIdx.x % kQueues;
  int* counter = w.queue + qid * kQueueStride;
  if (threadIdx.x == 0) sh_item = atomicAdd(counter, 1);
  __syncthreads();
  // the live flag of the last (sequence, position) this block saw: a
  // published flag never changes, and a counter's consecutive items mostly
  // share one (sequence, position)
  int cached_b = -1, cached_i = -1, cached_live = 0;
  while (true) {
    // one atomic claims kBatch consecutive items of this counter, processed
    // in increasing order; the next claim is fetched under them
    const int claim = __builtin_amdgcn_readfirstlane(sh_item);
    if (claim * kBatch * kQueues + qid >= total) break;
    int nxt = 0;
    if (threadIdx.x == 0) nxt = atomicAdd(counter, 1);
    for (int u = 0; u < kBatch; ++u) {
    const int it = (claim * kBatch + u) * kQueues + qid;
    if (it >= total) break;
    const int i = it < k * per_pos ? it / per_pos : k;
    const int rem = it - i * per_pos;
    const int nrow = i < k ? 2 : 1;
    if (rem < B * nrow * nc) {
      // ---- chunk item: (sequence b, row p_i or q_i, chunk c); past the
      // first rejection nothing is read
      const int b = rem / (nrow * nc), r = (rem / nc) % nrow, c = rem % nc;
      if (b != cached_b || i != cached_i) {
        cached_live = __builtin_amdgcn_readfirstlane(int(wait_live(w, k, b, i, &sh_live)));
        cached_b = b;
        cached_i = i;
      }
      if (cached_live) {
        const int row = r == 0 ? i : k + 1 + i;
        const int lo = c * kChunk, hi = min(V, lo + kChunk);
        const float2 st = range_stats<T>(ee_row<T>(a, b, row), lo, hi, a.scale_log2);
        if (threadIdx.x == 0) st_word(w.part + (int64_t(b) * rps + row) * nc + c, pack_part(st));
      }
    } else if (threadIdx.x < kWave) {
      decision_item<T>(a, w, rem - B * nrow * nc, i);
    }
    __syncthreads();   // the item's LDS is reused by the next one
    }
    if (threadIdx.x == 0) sh_item = nxt;
    __syncthreads();
  }
}

template <typename T>
hipError_t launch_ee(const VerifyLinearArgs& a, hipStream_t stream) {
  const int nc = num_chunks(a.vocab);
  EeWs w = ee_ws(a.ws, a.batch, a.k, a.vocab);
  {
    const int64_t n = int64_t(a.batch) * (2 * a.k + 1) * nc + int64_t(a.batch) * (a.k + 2);
    const unsigned blocks = unsigned(std::min<int64_t>((n + kChunkThreads - 1) / kChunkThreads, 1024));
    ProfileScope ps("uno_ee_init", stream);
    hipLaunchKernelGGL(ee_init_kernel, dim3(blocks), dim3(kChunkThreads), 0, stream, a.batch, a.k, nc, w);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    // every block that can be resident at once takes items (2 per CU)
    int dev = 0, cus = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    ProfileScope ps("uno_ee_flow", stream);
    const int blocks = (2 * std::max(cus, 1) + kQueues - 1) / kQueues * kQueues;
    hipLaunchKernelGGL(ee_flow_kernel<T>, dim3(unsigned(blocks)), dim3(kChunkThreads), 0, stream, a, w);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_draw<T>(w.desc, a.batch, a.vocab, a.scale_log2, w.seg, a.u_s, a.out_tok, a.out_mass, stream,
                        "uno_draw_seg", "uno_draw_resolve");
}

}  // namespace

size_t verify_linear_ee_workspace_bytes(int batch, int k, int vocab) {
  const int nc = num_chunks(vocab);
  return align_up(size_t(batch) * (2 * k + 1) * nc * sizeof(uint64_t), 256) +
         align_up(size_t(batch) * (k + 2) * sizeof(int), 256) +
         align_up(size_t(kQueues + 1) * kQueueStride * sizeof(int), 256) +
         align_up(size_t(batch) * sizeof(DrawDesc), 256) + draw_seg_bytes(batch, vocab);
}

hipError_t launch_verify_linear_ee(const VerifyLinearArgs& a, hipStream_t stream) {
  return a.dtype == UNO_BF16 ? launch_ee<uint16_t>(a, stream) : launch_ee<float>(a, stream);
}

}  // namespace uno
