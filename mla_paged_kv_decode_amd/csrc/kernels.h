// Launch interface of the gfx950 decode kernel (internal to the
// library; the public C ABI is include/mla_decode.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla_gpu {

struct DecodeArgs {
  const uint16_t* q_nope;  // bf16 [B, H, 512]
  const uint16_t* q_pe;    // bf16 [B, H, 64]
  const uint8_t* ckv;      // [pages, P, 512] bf16 or 8-bit codes
  const uint8_t* kpe;      // [pages, P, 64]
  const float* kv_scale;   // [pages, P] for 8-bit caches
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* kv_last_page_len;
  const int4* segs;           // 8 ints each: row, begin, end, slot, split index,
                              // first slot, number of chunks, request (row / rows_per_req)
  const int32_t* worker_ptr;  // grid + 1
  uint16_t* o;                // bf16 [B, H, 512]
  float* lse;                 // [B, H]
  float* part_o;              // partial O: fp16 [slots, H, 512] (typed float* for the
                              // workspace's fp32 sizing; the scales follow the fp16 data)
  float* part_lse;            // [slots, H]
  float* part_scale;          // power-of-two scale of each 128-column block of part_o
                              // [slots, H, 4]: the partial is fp16 value x scale
  const int4* clist;          // 4 ints per split request: row, first slot, chunks, 0
  float scale_log2;           // sm_scale * log2(e)
  int32_t o_fp16;             // 1: o is fp16 (fp16 cache and queries), 0: bf16
  int32_t page_shift;         // log2(page_size)
  int32_t rows_per_req;       // kernel rows per request: row b of q/o/lse (kernel-width
                              // groups of query vectors) reads the latent cache of request
                              // b / rows_per_req
  int32_t qo_len;             // queries per request: query vector j of a request is head
  int32_t head_log2;          // j & (2^head_log2 - 1) of query j >> head_log2, and sees the
                              // first L_b - (qo_len - 1 - (j >> head_log2)) tokens
  int32_t one_seg;            // 1: worker w runs segment w alone (worker_ptr is the
                              // identity), so a workgroup skips that load
  int32_t req_div;            // > 0 (only with one_seg): segment i reads the latent cache of
                              // request i / req_div, so its page-table loads need not wait
                              // for the segment record
  int32_t req_deal;           // > 0 (only with req_div): the workers were dealt to req_deal
                              // L2 domains, and segment i reads request rank(i) / req_div,
                              // rank(i) = (i % X) * (grid / X) + i / X (X = req_deal)
};

struct DecodeConfig {
  int32_t waves;  // waves per workgroup
  int32_t tile;   // tokens per KV tile = split granularity
  int32_t lds_bytes;  // LDS per workgroup
};

// Kernel for `heads` heads per workgroup and a cache of `kv_dtype` (mla_kv_dtype:
// 0 bf16, 1 / 2 fp8 / int8, 3 / 4 fp8 / int8 ckv with bf16 kpe, 5 fp16): returns -1 when
// no kernel serves the pair.
int decode_config(int heads, int kv_dtype, DecodeConfig* cfg);
// Workgroups of that kernel resident on one CU (HIP occupancy query on the
// current device; an LDS-based estimate if the query fails).
int decode_blocks_per_cu(int heads, int kv_dtype);
// start / stop (either may be null): events the launch takes from its own
// dispatch, the start and the end of the kernel's execution
// (hipExtLaunchKernel), so that no marker between kernels adds to what they
// measure.
hipError_t launch_decode(int heads, int kv_dtype, const DecodeArgs& a, int grid,
                         hipStream_t stream, hipEvent_t start = nullptr,
                         hipEvent_t stop = nullptr);
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
// Merge of the ncomb split requests listed in a.clist, each cut into at most
// max_splits chunks, after the decode kernel (which leaves their partials):
// writes o and lse of those rows.
hipError_t launch_combine(int heads, const DecodeArgs& a, int ncomb, int max_splits,
                          hipStream_t stream);
// Up to this many chunks per request, one thread per (head, 8 columns) merges
// a request; more chunks are spread over several workgroups per head.
constexpr int kCombineFewMax = 4;

}  // namespace mla_gpu
