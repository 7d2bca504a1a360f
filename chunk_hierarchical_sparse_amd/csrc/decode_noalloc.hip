// decode_noalloc.hip - hsa_decode for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  The decode's scratch (slice candidates, the selection,
// partial chunk outputs) lives in a fixed device array of
// HSA_DECODE_NOALLOC_SCRATCH_BYTES that each GPU holds from its first use to
// the end of the process; the computation is hsa_decode's, kernel for
// kernel.
//
// In host code `scratch` names a host-side stand-in, not device memory, so
// it is never passed to a kernel or a copy: its device address is looked up
// once per device with hipGetSymbolAddress (with that device current) and
// that address is used instead.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "hsa_attn.h"
#include "kernels.h"

namespace {

constexpr size_t kScratchBytes = HSA_DECODE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (looked up on the
// first call on that device).
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" hsa_status_t hsa_decode_noalloc(const void* q, const void* Kc, const void* Vc,
                                           const float* lmk, int64_t n_ctx, int64_t n_max,
                                           void* o, int32_t* sel_idx, float* sel_w, int B,
                                           int Hq, int Hkv, int d, int S, int topk,
                                           hsa_dtype_t dtype, hsa_stream_t stream) {
  // the size hsa_decode needs; 0 means the shape is invalid, and hsa_decode
  // (given no workspace) reports why before touching the device
  const size_t need = hsa_decode_workspace_size(B, Hq, Hkv, d, S, topk, n_ctx);
  if (need == 0)
    return hsa_decode(q, Kc, Vc, lmk, n_ctx, n_max, o, sel_idx, sel_w, B, Hq, Hkv, d, S, topk,
                      dtype, nullptr, 0, stream);
  if (need > kScratchBytes) {
    const std::string msg = "hsa_decode_noalloc: this shape needs " + std::to_string(need) +
                            " bytes of scratch, above the fixed " +
                            std::to_string(kScratchBytes) +
                            " bytes; call hsa_decode with a workspace instead";
    return (hsa_status_t)hsa::api_error(HSA_ERR_UNSUPPORTED, msg.c_str());
  }
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) {
    const std::string msg = std::string("hsa_decode_noalloc: scratch address: ") +
                            hipGetErrorString(e);
    return (hsa_status_t)hsa::api_error(HSA_ERR_HIP, msg.c_str());
  }
  return hsa_decode(q, Kc, Vc, lmk, n_ctx, n_max, o, sel_idx, sel_w, B, Hq, Hkv, d, S, topk,
                    dtype, ws, kScratchBytes, stream);
}
