// Split-KV work planner (host only, no HIP calls).
//
// FlashMLA PR 233, "What is added", describes a balanced scheduler with a
// deterministic combine whose metadata is computed ahead of the launch.  This
// planner cuts each request into token chunks and assigns the chunks to a
// fixed number of workgroups ("workers") so that the largest per-worker cost is
// small; requests cut into several chunks get consecutive partial slots that
// the combine step merges in chunk order.
#pragma once

#include <cstdint>
#include <vector>

namespace mla {

struct PlanParams {
  int32_t num_heads = 0;
  int32_t page_size = 0;
  int32_t num_workers = 0;   // grid size to balance over
  int32_t granularity = 64;  // chunk boundaries are multiples of this many tokens
  int32_t force_splits = 0;  // > 0: every request cut into this many chunks (at most)
  int32_t max_splits = 256;  // chunks per request at most (what the merge launch weighs)
  int32_t head_split = 1;    // > 1: each request's heads run as this many sub-requests
                             // (rows b * head_split + g of q/o viewed with H / head_split heads)
  int32_t xcd_count = 8;     // workgroups are dealt round-robin to this many L2 domains
};

struct Segment {
  int32_t request;  // q/o row block (a sub-request when heads are split)
  int32_t begin;  // first logical token
  int32_t end;    // one past the last token
  int32_t slot;   // partial slot, or -1 when this segment is the whole request
  int32_t split_request;  // index of the request among the split ones, or -1
  int32_t first_slot;     // first partial slot of the request (split requests)
  int32_t num_splits;     // chunks of the request (1 when not split)
  int32_t last;           // 1 for the last chunk of its request (end = the request's length)
};

struct Plan {
  int32_t batch = 0;
  int32_t num_workers = 0;           // workers that received work (grid size)
  std::vector<Segment> segments;     // grouped by worker
  std::vector<int32_t> worker_ptr;   // num_workers + 1 offsets into segments
  std::vector<int32_t> combine;      // 4 per split request: request, first slot, count, 0
  int32_t num_partials = 0;
};

// Returns 0 on success, -1 for a malformed page table (kv_indptr not starting at
// 0 or decreasing, kv_last_page_len outside [1, page_size] for a request with
// pages, or more than 2^31 - 1 tokens in one request).
int32_t build_plan(const int32_t* kv_indptr, const int32_t* kv_last_page_len, int32_t batch,
                   const PlanParams& params, Plan* out);

// Upper bound of segments and partial slots for any plan of `batch` requests
// (counting sub-requests when heads are split).
int64_t max_segments(int32_t batch, const PlanParams& params);
int64_t max_partials(int32_t batch, const PlanParams& params);

}  // namespace mla
