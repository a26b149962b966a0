// mla_decode_run_noalloc: mla_decode_run for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The work list and the split partials that
// mla_decode_run keeps in the plan's workspace live here in one file-scope
// device array per GPU instead, of a fixed maximum size.
//
// In host code `scratch` names a host-side stand-in, not device memory: the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken once
// per device (with that device current) on the first call there, and only
// that address is handed to copies and kernels.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <string>

#include "../../include/mla_decode.h"
#include "plan_internal.h"

namespace {

constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

std::mutex g_mu;
uint8_t* g_scratch[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

// Device address of this device's scratch array (looked up once per device).
mla_status scratch_of_current_device(uint8_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return mla_abi::hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    mla_abi::set_last_error("mla_decode_run_noalloc: device index out of range");
    return MLA_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return mla_abi::hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch[dev] = static_cast<uint8_t*>(ptr);
  }
  *out = g_scratch[dev];
  return MLA_OK;
}

}  // namespace

extern "C" mla_status mla_decode_run_noalloc(mla_plan_t p, const void* q_nope, const void* q_pe,
                                             const void* ckv, const void* kpe,
                                             const float* kv_scale, const int32_t* kv_indptr,
                                             const int32_t* kv_indices,
                                             const int32_t* kv_last_page_len, float sm_scale,
                                             void* o, float* lse, void* stream) {
  if (!p) return MLA_ERR_INVALID_ARG;
  if (p->batch == 0) return MLA_OK;
  if (p->layout.total > kScratchBytes) {  // checked before any device call
    mla_abi::set_last_error("mla_decode_run_noalloc: the plan needs " +
                            std::to_string(p->layout.total) +
                            " bytes of work list and partials; the library's scratch holds " +
                            std::to_string(kScratchBytes));
    return MLA_ERR_WORKSPACE_TOO_SMALL;
  }
  uint8_t* ws = nullptr;
  mla_status st = scratch_of_current_device(&ws);
  if (st != MLA_OK) return st;
  // this plan's work list, ahead of the kernels on the same stream (the last
  // call's contents may still be there; partials need no clearing, every
  // slot a run reads was written by that run's decode kernel)
  if (!p->host_meta.empty()) {
    hipError_t e = hipMemcpyAsync(ws, p->host_meta.data(), p->host_meta.size(),
                                  hipMemcpyHostToDevice, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return mla_abi::hip_fail(e, "hipMemcpyAsync(work list)");
  }
  return mla_abi::run_on_workspace(p, ws, q_nope, q_pe, ckv, kpe, kv_scale, kv_indptr,
                                   kv_indices, kv_last_page_len, sm_scale, o, lse, stream);
}
