// Plan object and run path shared by the C ABI's entry points (internal to the
// library; the public interface is include/mla_decode.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/mla_decode.h"
#include "kernels.h"
#include "planner.h"

namespace mla_abi {

// Byte offsets of the regions of a plan's device workspace:
// segments (32 B each) | worker_ptr | combine list (16 B per split request) |
// partial LSE | partial O.  The first meta_bytes are the work list the plan
// uploads; the partial regions are written and read by every run.
struct Layout {
  size_t segs, wptr, clist, plse, po, total, meta_bytes;
  size_t pscale;  // the partials' block scales, inside the partial-O area (after the fp16 data)
};

// Records the text returned by mla_last_error on this thread.
void set_last_error(const std::string& what);
mla_status hip_fail(hipError_t e, const char* what);

}  // namespace mla_abi

struct mla_plan_s {
  int32_t batch = 0, heads = 0, page_size = 0, page_shift = 0, kv_dtype = 0;
  int32_t qo_len = 1, head_split = 1, kernel_heads = 0;
  mla_gpu::DecodeConfig cfg{};
  mla::Plan plan;
  int32_t max_splits = 0;  // most chunks of one split request
  int32_t one_seg = 0;     // every worker runs exactly the segment of its own index
  int32_t req_div = 0;     // with one_seg: segment i reads request i / req_div (0: no such c)
  int32_t req_deal = 0;    // X > 0: the workers were dealt to X L2 domains and segment i
                           // reads request rank(i) / req_div, rank(i) = (i % X) * (n / X) + i / X
  mla_abi::Layout layout{};
  std::vector<uint8_t> host_meta;  // staged work list (kept alive for the async copy)
  uint8_t* workspace = nullptr;
  hipEvent_t ev_before = nullptr, ev_after = nullptr;
};

namespace mla_abi {

// The launches of mla_decode_run for plan p with its work list and partials
// in `ws` (a device buffer of at least p->layout.total bytes that already
// holds p's work list).  Validates the pointers; launches the decode kernel
// and, for split requests, the merge.
mla_status run_on_workspace(mla_plan_s* p, uint8_t* ws, const void* q_nope, const void* q_pe,
                            const void* ckv, const void* kpe, const float* kv_scale,
                            const int32_t* kv_indptr, const int32_t* kv_indices,
                            const int32_t* kv_last_page_len, float sm_scale, void* o, float* lse,
                            void* stream);

}  // namespace mla_abi
