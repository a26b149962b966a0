// C ABI of the paged MLA decode library (declared in include/mla_decode.h).
//
// mla_decode_plan runs the split-KV planner on the host copies of the page
// table and copies the work list into the caller's workspace; mla_decode_run
// only launches kernels: the decode kernel and, when the plan split requests
// into chunks, the merge of their partials.
// It allocates and synchronises nothing, so it is safe to capture in a HIP
// graph.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/mla_decode.h"
#include "append.h"
#include "kernels.h"
#include "plan_internal.h"
#include "planner.h"

namespace {

thread_local std::string g_last_error;

}  // namespace

namespace mla_abi {

void set_last_error(const std::string& what) { g_last_error = what; }

mla_status hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return MLA_ERR_HIP;
}

}  // namespace mla_abi

namespace {

using mla_abi::hip_fail;
using mla_abi::Layout;

bool supported_heads(int32_t h) { return h == 16 || h == 32 || h == 64 || h == 128; }

int page_shift_of(int32_t p) {
  switch (p) {
    case 16: return 4;
    case 32: return 5;
    case 64: return 6;
    default: return -1;
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// workspace: segments (32 B each) | worker_ptr | combine list (16 B per split
// request) | partial LSE | partial O (sized as fp32 [parts, heads, 512]; held
// as fp16, followed by one fp32 scale per 128-column block)
Layout layout_for(int64_t nseg, int64_t workers, int64_t ncomb, int64_t nparts, int32_t heads) {
  Layout L;
  L.segs = 0;
  L.wptr = align256(L.segs + (size_t)nseg * 32);
  L.clist = align256(L.wptr + (size_t)(workers + 1) * 4);
  L.meta_bytes = L.clist + (size_t)ncomb * 16;
  L.plse = align256(L.meta_bytes);
  L.po = align256(L.plse + (size_t)nparts * heads * 4);
  L.pscale = L.po + (size_t)nparts * heads * 512 * 2;
  L.total = align256(L.po + (size_t)nparts * heads * 512 * 4);
  return L;
}

// Workgroups to balance over: CUs x decode workgroups resident per CU, for
// the kernel that serves `kernel_heads` heads.  With an explicit
// opts->num_cus (host-only planning) the per-CU count comes from the kernel's
// LDS footprint; on a device it comes from the occupancy query.
mla_status worker_count(const mla_plan_opts* opts, int32_t kernel_heads, int32_t kv_dtype,
                        int32_t* workers) {
  int32_t cus = opts ? opts->num_cus : 0;
  if (cus < 0) return MLA_ERR_INVALID_ARG;
  mla_gpu::DecodeConfig cfg{};
  if (mla_gpu::decode_config(kernel_heads, kv_dtype, &cfg) != 0) return MLA_ERR_UNSUPPORTED;
  int32_t per_cu = std::max(1, (160 * 1024) / cfg.lds_bytes);
  if (cus == 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    per_cu = mla_gpu::decode_blocks_per_cu(kernel_heads, kv_dtype);
  }
  int32_t w = cus * per_cu;
  if (opts && opts->max_workers > 0) w = std::min(w, opts->max_workers);
  if (w <= 0) return MLA_ERR_INVALID_ARG;
  *workers = w;
  return MLA_OK;
}

int log2_exact(int32_t x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return (1 << s) == x ? s : -1;
}

constexpr int32_t kMaxQoLen = 64;

// Queries per request from the options (0 = 1); -1 if out of range.
int32_t qo_len_of(const mla_plan_opts* opts) {
  const int32_t q = opts ? opts->qo_len : 0;
  if (q < 0 || q > kMaxQoLen) return -1;
  return q == 0 ? 1 : q;
}

// Head split for a batch: explicit (opts->head_split) or automatic.  The
// qo_len * num_heads query vectors of a request share its latent stream; they
// run as head_split rows of the largest width a kernel serves that divides
// them (bf16: 16 to 128; 8-bit: 16 and 128), so that a request takes as few
// passes over its cache as possible.  Rows of one request are placed on one
// XCD by the planner, so that the latent cache is read from HBM about once.
mla_status choose_head_split(int32_t num_heads, int32_t qo_len, int32_t kv_dtype,
                             const mla_plan_opts* opts, int32_t* head_split) {
  const int32_t req = opts ? opts->head_split : 0;
  if (req < 0) return MLA_ERR_INVALID_ARG;
  const int32_t nq = num_heads * qo_len;
  mla_gpu::DecodeConfig cfg{};
  if (req > 0) {
    if (nq % req != 0 || mla_gpu::decode_config(nq / req, kv_dtype, &cfg) != 0)
      return MLA_ERR_UNSUPPORTED;
    *head_split = req;
    return MLA_OK;
  }
  for (int32_t w = 128; w >= 16; w /= 2) {
    if (nq % w == 0 && mla_gpu::decode_config(w, kv_dtype, &cfg) == 0) {
      *head_split = nq / w;
      return MLA_OK;
    }
  }
  return MLA_ERR_UNSUPPORTED;
}

mla::PlanParams plan_params(int32_t num_queries, int32_t head_split, int32_t workers,
                            const mla_gpu::DecodeConfig& cfg, const mla_plan_opts* opts) {
  mla::PlanParams pp;
  pp.num_heads = num_queries / head_split;
  pp.num_workers = workers;
  pp.granularity = cfg.tile;
  pp.force_splits = opts ? opts->force_splits : 0;
  pp.head_split = head_split;
  if (opts && opts->l2_domains > 0) pp.xcd_count = opts->l2_domains;
  // the merge launch weighs up to 256 chunks of one request (one LDS weight each)
  pp.max_splits = 256;
  return pp;
}

}  // namespace

namespace mla_abi {

mla_status run_on_workspace(mla_plan_s* p, uint8_t* ws, const void* q_nope, const void* q_pe,
                            const void* ckv, const void* kpe, const float* kv_scale,
                            const int32_t* kv_indptr, const int32_t* kv_indices,
                            const int32_t* kv_last_page_len, float sm_scale, void* o, float* lse,
                            void* stream) {
  if (p->batch == 0) return MLA_OK;
  if (!q_nope || !q_pe || !ckv || !kpe || !kv_indptr || !kv_indices || !kv_last_page_len || !o ||
      !lse)
    return MLA_ERR_INVALID_ARG;
  const bool scaled = p->kv_dtype != MLA_KV_BF16 && p->kv_dtype != MLA_KV_FP16;
  if (scaled != (kv_scale != nullptr)) return MLA_ERR_INVALID_ARG;
  if (!(sm_scale == sm_scale)) return MLA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);

  mla_gpu::DecodeArgs a;
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.ckv = static_cast<const uint8_t*>(ckv);
  a.kpe = static_cast<const uint8_t*>(kpe);
  a.kv_scale = kv_scale;
  a.kv_indptr = kv_indptr;
  a.kv_indices = kv_indices;
  a.kv_last_page_len = kv_last_page_len;
  a.segs = reinterpret_cast<const int4*>(ws + p->layout.segs);
  a.worker_ptr = reinterpret_cast<const int32_t*>(ws + p->layout.wptr);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.part_o = reinterpret_cast<float*>(ws + p->layout.po);
  a.part_lse = reinterpret_cast<float*>(ws + p->layout.plse);
  a.part_scale = reinterpret_cast<float*>(ws + p->layout.pscale);
  a.clist = reinterpret_cast<const int4*>(ws + p->layout.clist);
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.o_fp16 = p->kv_dtype == MLA_KV_FP16 ? 1 : 0;
  a.page_shift = p->page_shift;
  a.rows_per_req = p->head_split;
  a.qo_len = p->qo_len;
  a.head_log2 = log2_exact(p->heads);
  a.one_seg = p->one_seg;
  a.req_div = p->req_div;
  a.req_deal = p->req_deal;
  if (p->plan.num_workers > 0) {
    // the events (if set) take the decode kernel's own start and end, without
    // the merge below
    hipError_t e = mla_gpu::launch_decode(p->kernel_heads, p->kv_dtype, a, p->plan.num_workers, s,
                                          p->ev_before, p->ev_after);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
  } else {
    // no decode launch: the events are recorded back to back
    for (hipEvent_t ev : {p->ev_before, p->ev_after}) {
      if (!ev) continue;
      hipError_t e = hipEventRecord(ev, s);
      if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
  }
  const int ncomb = (int)(p->plan.combine.size() / 4);
  if (p->plan.num_workers > 0 && ncomb > 0) {
    hipError_t e = mla_gpu::launch_combine(p->kernel_heads, a, ncomb, p->max_splits, s);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
  }
  return MLA_OK;
}

}  // namespace mla_abi

extern "C" {

const char* mla_status_string(int32_t s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MLA_ERR_HIP: return "HIP runtime error";
    case MLA_ERR_NOT_UPLOADED: return "plan has no device workspace";
    default: return "unknown status";
  }
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

size_t mla_decode_workspace_bytes(int32_t batch, int32_t num_heads, const mla_plan_opts* opts) {
  if (batch < 0 || !supported_heads(num_heads)) return 0;
  if (opts && (opts->force_splits < 0 || opts->head_split < 0)) return 0;
  const int32_t qo_len = qo_len_of(opts);
  if (qo_len < 1) return 0;
  const int32_t nq = num_heads * qo_len;
  // bound over every row width and cache dtype the plan may choose
  size_t best = 0;
  for (int32_t kvd = 0; kvd <= MLA_KV_FP16; ++kvd)
  for (int32_t w = 16; w <= 128; w *= 2) {
    if (nq % w != 0) continue;
    const int32_t hs = nq / w;
    if (opts && opts->head_split > 0 && hs != opts->head_split) continue;
    mla_gpu::DecodeConfig cfg{};
    if (mla_gpu::decode_config(w, kvd, &cfg) != 0) continue;
    int32_t workers = 0;
    if (worker_count(opts, w, kvd, &workers) != MLA_OK) return 0;
    const mla::PlanParams pp = plan_params(nq, hs, workers, cfg, opts);
    const int64_t nseg = mla::max_segments(batch, pp);
    const int64_t nparts = mla::max_partials(batch, pp);
    best = std::max(best, layout_for(nseg, workers, (int64_t)batch * hs, nparts, pp.num_heads).total);
  }
  return best;
}

mla_status mla_decode_plan(mla_plan_t* out, const int32_t* kv_indptr_host,
                           const int32_t* kv_last_page_len_host, int32_t batch, int32_t num_heads,
                           int32_t page_size, int32_t kv_dtype, const mla_plan_opts* opts,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!out) return MLA_ERR_INVALID_ARG;
  *out = nullptr;
  if (batch < 0 || !kv_indptr_host || (batch > 0 && !kv_last_page_len_host))
    return MLA_ERR_INVALID_ARG;
  if (!supported_heads(num_heads) || page_shift_of(page_size) < 0) return MLA_ERR_UNSUPPORTED;
  if (kv_dtype < MLA_KV_BF16 || kv_dtype > MLA_KV_FP16) return MLA_ERR_UNSUPPORTED;
  if (opts && (opts->force_splits < 0 || opts->max_workers < 0 || opts->l2_domains < 0))
    return MLA_ERR_INVALID_ARG;

  if (opts && opts->head_split < 0) return MLA_ERR_INVALID_ARG;
  const int32_t qo_len = qo_len_of(opts);
  if (qo_len < 1) return MLA_ERR_INVALID_ARG;
  if ((int64_t)batch * qo_len * num_heads / 16 > INT32_MAX) return MLA_ERR_INVALID_ARG;  // rows
  int32_t head_split = 1;
  mla_status st = choose_head_split(num_heads, qo_len, kv_dtype, opts, &head_split);
  if (st != MLA_OK) return st;
  const int32_t kernel_heads = num_heads * qo_len / head_split;

  mla_plan_s* p = new (std::nothrow) mla_plan_s();
  if (!p) return MLA_ERR_INVALID_ARG;
  p->batch = batch;
  p->heads = num_heads;
  p->qo_len = qo_len;
  p->head_split = head_split;
  p->kernel_heads = kernel_heads;
  p->page_size = page_size;
  p->page_shift = page_shift_of(page_size);
  p->kv_dtype = kv_dtype;
  if (mla_gpu::decode_config(kernel_heads, kv_dtype, &p->cfg) != 0) {
    delete p;
    return MLA_ERR_UNSUPPORTED;
  }
  int32_t workers = 0;
  st = worker_count(opts, kernel_heads, kv_dtype, &workers);
  if (st != MLA_OK) {
    delete p;
    return st;
  }
  mla::PlanParams pp = plan_params(num_heads * qo_len, head_split, workers, p->cfg, opts);
  pp.page_size = page_size;
  static const int32_t kZero = 0;
  if (mla::build_plan(kv_indptr_host, batch > 0 ? kv_last_page_len_host : &kZero, batch, pp,
                      &p->plan) != 0) {
    delete p;
    return MLA_ERR_INVALID_ARG;
  }
  const mla::Plan& pl = p->plan;
  for (size_t i = 2; i < pl.combine.size(); i += 4)
    p->max_splits = std::max(p->max_splits, pl.combine[i]);
  p->one_seg = (int64_t)pl.segments.size() == (int64_t)pl.num_workers ? 1 : 0;
  for (size_t w = 0; p->one_seg && w < pl.worker_ptr.size(); ++w)
    if (pl.worker_ptr[w] != (int32_t)w) p->one_seg = 0;
  if (p->one_seg && !pl.segments.empty()) {
    // Segment i reads request rank(i) / c, with rank(i) = i (launch order) or,
    // when the planner dealt the workers to X L2 domains (domain d taking
    // ranks d * per .. d * per + per - 1 at launch positions d, d + X, ...,
    // per = n / X), rank(i) = (i % X) * per + i / X.
    const int64_t n = (int64_t)pl.segments.size();
    for (int32_t deal : {0, pp.xcd_count}) {
      if (deal == 1 || (deal > 1 && n % deal != 0)) continue;
      const int64_t per = deal > 1 ? n / deal : n;
      auto req_of_rank = [&](int64_t r) {
        const int64_t pos = deal > 1 ? r / per + deal * (r % per) : r;
        return pl.segments[(size_t)pos].request / head_split;
      };
      const int32_t first = req_of_rank(0);
      int32_t c = 0;
      while (c < n && req_of_rank(c) == first) ++c;
      bool ok = true;
      for (int64_t r = 0; ok && r < n; ++r) ok = req_of_rank(r) == (int32_t)(r / c);
      if (ok) {
        p->req_div = c;
        p->req_deal = deal;
        break;
      }
    }
  }
  const int64_t ncomb = (int64_t)pl.combine.size() / 4;
  p->layout = layout_for((int64_t)pl.segments.size(), pl.num_workers, ncomb, pl.num_partials,
                         kernel_heads);

  // stage the work list: segments | worker_ptr | combine list.  The last chunk
  // of every request ends at INT32_MAX, i.e. at the request's length as the
  // device page table gives it when a run reads it (the kernels clamp every
  // chunk to that length): tokens appended after planning are decoded by the
  // same plan, and only the balance of the work depends on the plan-time lengths.
  p->host_meta.assign(p->layout.meta_bytes, 0);
  for (size_t i = 0; i < pl.segments.size(); ++i) {
    const mla::Segment& g = pl.segments[i];
    const int32_t end = g.last ? INT32_MAX : g.end;
    const int32_t v[8] = {g.request, g.begin, end, g.slot, g.split_request, g.first_slot,
                          g.num_splits, g.request / head_split};
    std::memcpy(p->host_meta.data() + p->layout.segs + i * 32, v, 32);
  }
  std::memcpy(p->host_meta.data() + p->layout.wptr, pl.worker_ptr.data(),
              pl.worker_ptr.size() * 4);
  if (ncomb > 0)
    std::memcpy(p->host_meta.data() + p->layout.clist, pl.combine.data(), (size_t)ncomb * 16);

  if (workspace) {
    if (workspace_bytes < p->layout.total) {
      delete p;
      return MLA_ERR_WORKSPACE_TOO_SMALL;
    }
    p->workspace = static_cast<uint8_t*>(workspace);
    hipError_t e = hipMemcpyAsync(p->workspace, p->host_meta.data(), p->host_meta.size(),
                                  hipMemcpyHostToDevice, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
      delete p;
      return hip_fail(e, "hipMemcpyAsync(work list)");
    }
  }
  *out = p;
  return MLA_OK;
}

mla_status mla_decode_run(mla_plan_t p, const void* q_nope, const void* q_pe, const void* ckv,
                          const void* kpe, const float* kv_scale, const int32_t* kv_indptr,
                          const int32_t* kv_indices, const int32_t* kv_last_page_len,
                          float sm_scale, void* o, float* lse, void* stream) {
  if (!p) return MLA_ERR_INVALID_ARG;
  if (!p->workspace) return MLA_ERR_NOT_UPLOADED;
  return mla_abi::run_on_workspace(p, p->workspace, q_nope, q_pe, ckv, kpe, kv_scale, kv_indptr,
                                   kv_indices, kv_last_page_len, sm_scale, o, lse, stream);
}

void mla_decode_plan_destroy(mla_plan_t p) { delete p; }

mla_status mla_decode_plan_set_events(mla_plan_t p, void* before, void* after) {
  if (!p || ((before == nullptr) != (after == nullptr))) return MLA_ERR_INVALID_ARG;
  p->ev_before = static_cast<hipEvent_t>(before);
  p->ev_after = static_cast<hipEvent_t>(after);
  return MLA_OK;
}

mla_status mla_decode_plan_info(mla_plan_t p, int32_t info[16]) {
  if (!p || !info) return MLA_ERR_INVALID_ARG;
  info[0] = p->batch;
  info[1] = p->heads;
  info[2] = p->page_size;
  info[3] = p->kv_dtype;
  info[4] = p->plan.num_workers;
  info[5] = (int32_t)p->plan.segments.size();
  info[6] = p->plan.num_partials;
  info[7] = (int32_t)(p->plan.combine.size() / 4);
  info[8] = p->cfg.tile;
  info[9] = p->cfg.waves;
  info[10] = p->head_split;
  info[11] = p->kernel_heads;
  info[12] = p->qo_len;
  info[13] = p->one_seg;
  info[14] = p->req_div;
  info[15] = p->req_deal;
  return MLA_OK;
}

mla_status mla_decode_plan_segments(mla_plan_t p, int32_t* seg, int32_t* worker_ptr) {
  if (!p || !seg || !worker_ptr) return MLA_ERR_INVALID_ARG;
  for (size_t i = 0; i < p->plan.segments.size(); ++i) {
    seg[4 * i + 0] = p->plan.segments[i].request;
    seg[4 * i + 1] = p->plan.segments[i].begin;
    seg[4 * i + 2] = p->plan.segments[i].end;
    seg[4 * i + 3] = p->plan.segments[i].slot;
  }
  std::memcpy(worker_ptr, p->plan.worker_ptr.data(), p->plan.worker_ptr.size() * 4);
  return MLA_OK;
}

mla_status mla_cache_append(const void* ckv_new, const void* kpe_new, const int64_t* slots,
                            int32_t n, int32_t kv_dtype, void* ckv, void* kpe,
                            float* kv_scale, void* stream) {
  if (n < 0) return MLA_ERR_INVALID_ARG;
  if (kv_dtype < MLA_KV_BF16 || kv_dtype > MLA_KV_FP16) return MLA_ERR_UNSUPPORTED;
  if (n == 0) return MLA_OK;
  if (!ckv_new || !kpe_new || !slots || !ckv || !kpe) return MLA_ERR_INVALID_ARG;
  const bool scaled = kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP16;
  if (scaled != (kv_scale != nullptr)) return MLA_ERR_INVALID_ARG;
  hipError_t e = mla_gpu::launch_cache_append(
      kv_dtype, static_cast<const uint16_t*>(ckv_new), static_cast<const uint16_t*>(kpe_new),
      slots, n, static_cast<uint8_t*>(ckv), static_cast<uint8_t*>(kpe), kv_scale,
      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "cache append launch");
  return MLA_OK;
}

}  // extern "C"
