// Allocation-free variant of the attention backward, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  gpt2_op_attention_backward takes its
// scratch -- rowsum(dO * O) and the base-2 log-sum-exp of every query row,
// 2 x B*H*T floats -- from a caller workspace; this variant keeps it in a
// file-scope device array of fixed size instead.  Each GPU the library runs
// on holds its own copy of the array until the process ends; its address on
// a device is looked up once (hipGetSymbolAddress, with that device current)
// and kept.  The host-side name of the array is only a stand-in for the
// symbol and is never passed to a kernel.

#include <mutex>

#include "../../include/gpt2.h"
#include "../../include/gpt2_ops.h"
#include "kernels.h"

namespace {

constexpr size_t kScratchBytes = GPT2_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call there).
int scratch_address(void** out) {
  int dev = -1;
  GPT2_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices)
    return gpt2_internal_fail(GPT2_E_INVALID_ARG, "device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    GPT2_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return gpt2_internal_fail(GPT2_E_HIP, "hipGetSymbolAddress returned no address for the scratch array");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return GPT2_OK;
}

}  // namespace

extern "C" int gpt2_op_attention_backward_noalloc(int dtype, int B, int T, int H, int hd, const void* qkv,
                                                  const void* out, const void* dout, const float* lse, void* dqkv,
                                                  void* stream) {
  try {
    if (B < 0 || T < 0 || H <= 0 || hd <= 0)
      return gpt2_internal_fail(GPT2_E_INVALID_ARG, "attention_backward_noalloc: bad shape (B=%d, T=%d, H=%d, hd=%d)",
                                B, T, H, hd);
    const size_t need = gpt2k::attention_backward_workspace_bytes(B, T, H, hd);
    if (need > kScratchBytes)
      return gpt2_internal_fail(GPT2_E_INVALID_ARG,
                                "attention_backward_noalloc: B*H*T = %lld rows need %zu bytes of scratch; the "
                                "allocation-free variant holds at most %zu (use gpt2_op_attention_backward with a "
                                "workspace)",
                                (long long)B * H * T, need, kScratchBytes);
    if (!qkv || !out || !dout || !lse || !dqkv)
      return gpt2_internal_fail(GPT2_E_INVALID_ARG, "attention_backward_noalloc: NULL buffer");
    if (B == 0 || T == 0) return GPT2_OK;
    void* ws = nullptr;
    const int rc = scratch_address(&ws);
    if (rc) return rc;
    return gpt2k::attention_backward(dtype, B, T, H, hd, qkv, out, dout, lse, dqkv, ws, kScratchBytes,
                                     (hipStream_t)stream);
  } catch (...) {
    return gpt2_internal_fail(GPT2_E_INTERNAL, "attention_backward_noalloc: unexpected C++ exception");
  }
}
