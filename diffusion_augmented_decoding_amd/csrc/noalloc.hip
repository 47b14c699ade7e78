// Allocation-free linear verify: the same kernels as
// uno_psi_spec_verify_linear, with their scratch in a file-scope device
// array instead of a caller-provided workspace, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops).
//
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Host code never passes the array's name to a kernel (in
// host code that name is a host-side stand-in, not a device address): the
// device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and is kept per device.  Every call on a GPU shares
// that GPU's array: calls that overlap on one GPU (concurrent streams,
// threads) race on it.  Nothing in it has to start at zero: each call writes
// every scratch value it reads (the row partials, the draft logits, one draw
// descriptor per sequence, the segment masses).
#include <mutex>

#include "internal.h"

namespace uno {

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;   // 16 MiB: batch 4096 x 64 drafts at V = 151,936
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// The current device's address of `scratch` (looked up on the first call on
// that device).
uno_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return check_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(UNO_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return check_hip(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(UNO_ERR_INTERNAL, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return UNO_OK;
}

}  // namespace

}  // namespace uno

using namespace uno;

extern "C" uno_status uno_psi_spec_verify_linear_noalloc(
    hipStream_t stream, uno_dtype logit_dtype, int32_t batch, int32_t k, int32_t vocab, const void* p_logits,
    int64_t p_seq_stride, int64_t p_row_stride, const void* q_logits, int64_t q_seq_stride, int64_t q_row_stride,
    const int32_t* draft_tokens, const float* u_accept, const float* u_sample, float temperature,
    int32_t* out_accept_len, int32_t* out_token, float* out_p_draft, float* out_q_draft, float* out_residual_mass) {
  UNO_GUARD_BEGIN
  VerifyLinearArgs a{};
  uno_status s = verify_linear_args(logit_dtype, batch, k, vocab, p_logits, p_seq_stride, p_row_stride, q_logits,
                                    q_seq_stride, q_row_stride, draft_tokens, u_accept, u_sample, temperature,
                                    out_accept_len, out_token, out_p_draft, out_q_draft, out_residual_mass, &a);
  if (s != UNO_OK) return s;
  s = debug_check_verify_linear(stream, a);
  if (s != UNO_OK) return s;
  const size_t need = verify_linear_workspace_bytes(batch, k, vocab);
  if (need > kScratchBytes)
    return fail(UNO_ERR_UNSUPPORTED, "scratch of %zu bytes needed, the allocation-free call has %zu (use "
                "uno_psi_spec_verify_linear with a workspace)", need, kScratchBytes);
  void* ws = nullptr;
  s = scratch_address(&ws);
  if (s != UNO_OK) return s;
  a.ws = ws;
  return check_hip(launch_verify_linear(a, stream), "uno_psi_spec_verify_linear_noalloc launch");
  UNO_GUARD_END
}
