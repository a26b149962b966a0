/*
 * mla_decode.h - C ABI of the MI355X (gfx950) paged MLA decode library.
 *
 * The operation (absorbed-MQA multi-head latent attention decode):
 *   For request b with H query heads and kv_len L_b latent tokens, gathered
 *   through a paged cache,
 *     s[h,t]   = sm_scale * (q_nope[b,h,:] . ckv_t + q_pe[b,h,:] . kpe_t)
 *     o[b,h,:] = sum_t softmax_t(s[h,:]) * ckv_t              (512 values)
 *     lse[b,h] = ln sum_t exp(s[h,t])
 *   Sources:
 *   - "Benchmarking MLA" (flashinfer issue 700), comments on the
 *     matrix-absorbed decode: score dims 512 (ckv) + 64 (kpe), value dims 512,
 *     the ckv cache doubles as key and value, and all query heads share one
 *     latent stream (MQA, group size up to 128).  The same page lists the
 *     operands of a decode call: q_nope, q_pe, ckv, kpe, kv_indptr,
 *     kv_indices, kv_last_page_len, and the output o.
 *   - "perf: MLA decode kernel implemented by CuTe targeted to SM80"
 *     (flashinfer PR 844): the tensor shapes q_nope [B*qo_len, H, 512],
 *     q_pe [B*qo_len, H, 64], ckv [pages, P, 512], kpe [pages, P, 64].
 *   - FlashMLA PR 233, "What is added": page sizes 16/32/64, an 8-bit cache
 *     (FP8 e4m3 or INT8) with one scale per token dequantised in the kernel,
 *     a balanced split scheduler with a deterministic combine, and an API
 *     whose scheduling metadata is computed before graph capture.
 *   lse is this library's addition: the natural-log log-sum-exp of the same
 *   scaled scores that enter the softmax, so that callers can merge results.
 *
 * Conventions for every entry point:
 *   - All tensors are caller-owned, contiguous and row-major.  "device"
 *     pointers are HIP device allocations on the current device; "host"
 *     pointers are ordinary CPU memory.
 *   - Functions return an mla_status and never throw or abort; a HIP failure
 *     is reported as MLA_ERR_HIP and the text of the last error is available
 *     from mla_last_error().
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).
 *   - kv_dtype and status arguments are int32_t holding a value of
 *     mla_kv_dtype / mla_status, so that any integer a caller passes is
 *     checked rather than read as an out-of-range enum.
 *   - qo_len (mla_plan_opts.qo_len, default 1) queries per request: q_nope is
 *     [batch * qo_len, H, 512], q_pe [batch * qo_len, H, 64], o
 *     [batch * qo_len, H, 512], lse [batch * qo_len, H]; row b * qo_len + i is
 *     query i of request b.  The queries are the request's last qo_len
 *     positions: query i attends to the first L_b - (qo_len - 1 - i) tokens
 *     (the causal mask with Q at the end of the score matrix, for
 *     N_Q != N_K, of FlashMLA PR 76's forward kernel notes); a query with
 *     no visible token gets o = 0, lse = -inf.  All qo_len * H query vectors
 *     of a request share its latent stream, so they are folded into the
 *     kernel's head dimension (flashinfer issue 700 notes that fusing the
 *     query length with the heads raises the work per KV byte).
 *   - A cache "row" is one token slot: row = page * page_size + position.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1,          /* null pointer, bad size, malformed page table */
  MLA_ERR_UNSUPPORTED = -2,          /* head count / page size / dtype not built */
  MLA_ERR_WORKSPACE_TOO_SMALL = -3,  /* workspace_bytes below what the plan needs */
  MLA_ERR_HIP = -4,                  /* a HIP runtime call failed */
  MLA_ERR_NOT_UPLOADED = -5          /* run() on a plan made without a workspace */
} mla_status;

typedef enum {
  MLA_KV_BF16 = 0,      /* ckv/kpe are bf16; kv_scale must be NULL */
  MLA_KV_FP8_E4M3 = 1,  /* ckv/kpe are OCP fp8 e4m3 codes; kv_scale [pages, P] fp32
                           scales both (580 bytes per token) */
  MLA_KV_INT8 = 2,      /* ckv/kpe are int8 codes; kv_scale [pages, P] fp32 scales both */
  /* The 644-byte token record of FlashMLA PR 233 ("What is added": 644
     instead of 1152 bytes per token): 512 one-byte ckv codes, 64 bf16 kpe
     values and one fp32 scale, which applies to ckv only.  ckv [pages, P, 512]
     codes, kpe [pages, P, 64] bf16, kv_scale [pages, P] fp32. */
  MLA_KV_FP8_E4M3_KPE_BF16 = 3,
  MLA_KV_INT8_KPE_BF16 = 4,
  /* fp16 inputs (FlashMLA PR 233: the v2 kernel takes bf16 or fp16): ckv/kpe fp16,
     and q_nope, q_pe and o are fp16 too; kv_scale must be NULL. */
  MLA_KV_FP16 = 5
} mla_kv_dtype;

/* Scheduling options; zero-initialise for defaults. */
typedef struct {
  int32_t num_cus;      /* compute units to balance over; 0 = query the current device */
  int32_t force_splits; /* > 0: cut every request into this many near-equal chunks (testing) */
  int32_t max_workers;  /* > 0: cap on the number of workgroups; 0 = library default */
  int32_t head_split;   /* 0 = automatic; n >= 1: run each request's qo_len * num_heads query
                           vectors as n groups of qo_len * num_heads / n sharing the
                           request's latent cache (n = 1: all in one workgroup).  The group
                           width must be one the kernels serve: 16, 32, 64 or 128 (bf16),
                           16, 64 or 128 (fp16), 16 or 128 (8-bit caches). */
  int32_t qo_len;       /* queries per request, 1..64; 0 means 1 */
  int32_t l2_domains;   /* L2 domains (XCDs) that workgroups are dealt to round-robin in
                           launch order; the rows of one request, with all their token
                           chunks, are placed in one of them so that they share its latent
                           cache and query rows through one L2.  0 = 8 (a whole MI355X);
                           1 = no placement (e.g. a one-XCD partition). */
} mla_plan_opts;

typedef struct mla_plan_s* mla_plan_t;

/* Supported shapes: num_heads in {16, 32, 64, 128}; page_size in {16, 32, 64};
   every kv_dtype (8-bit caches run 16- and 128-wide rows, fp16 16-, 64- and
   128-wide rows);
   qo_len in 1..64.  The automatic group width is the largest served width that
   divides qo_len * num_heads. */

/*
 * Upper bound, in bytes, of the device workspace that mla_decode_plan needs
 * for any page table of `batch` requests with these heads and options.
 * Returns 0 for unsupported or invalid arguments (or, when opts->num_cus is
 * 0, if no HIP device can be queried).
 */
size_t mla_decode_workspace_bytes(int32_t batch, int32_t num_heads, const mla_plan_opts* opts);

/*
 * Build the split-KV schedule for one batch (the balanced scheduler; runs on
 * the host, launches no kernel).  FlashMLA PR 233, "What is added": a
 * scheduler that balances requests of different lengths over the GPU's
 * compute units, with its metadata computed before the decode launch so that
 * the launch can be captured in a graph.  The run of a batch-decode wrapper
 * is what "Benchmarking MLA" times; this split keeps all host work out of
 * that run.  A request whose qo_len * num_heads query
 * vectors are wider than one workgroup serves (see head_split) runs as
 * several rows of the served width; the workgroups of those rows are placed
 * on one XCD so that the request's latent cache is fetched from HBM about
 * once.
 *   kv_indptr_host        [batch + 1] int32, host: page-list offsets, non-decreasing, from 0.
 *   kv_last_page_len_host [batch] int32, host: valid slots of each request's last page,
 *                          in [1, page_size] when the request has pages (ignored otherwise).
 *   Request b holds L_b = (n_b - 1) * page_size + kv_last_page_len[b] tokens,
 *   n_b = kv_indptr[b+1] - kv_indptr[b]; a request without pages is empty
 *   (its output row is o = 0, lse = -inf).
 *   workspace             device buffer of workspace_bytes, caller-owned.  The plan
 *                          copies its work list there with hipMemcpyAsync on `stream`;
 *                          the workspace must stay allocated, and must not be used by
 *                          another plan, while runs of this plan may execute.
 *                          workspace == NULL makes a host-only plan that can be
 *                          inspected but not run.
 *   *out receives a new plan owned by the caller (free with mla_decode_plan_destroy).
 * Errors: MLA_ERR_INVALID_ARG for a malformed page table or null pointers,
 * MLA_ERR_UNSUPPORTED for shapes outside the supported set,
 * MLA_ERR_WORKSPACE_TOO_SMALL, MLA_ERR_HIP.
 */
mla_status mla_decode_plan(mla_plan_t* out, const int32_t* kv_indptr_host,
                           const int32_t* kv_last_page_len_host, int32_t batch, int32_t num_heads,
                           int32_t page_size, int32_t kv_dtype, const mla_plan_opts* opts,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Run the decode for a plan on `stream`: the decode kernel and, when the plan
 * split requests into chunks (up to 256 per request), a second launch that
 * merges their partials over the whole GPU.  The operands are those of the
 * decode call in "Benchmarking MLA" (nvbench snippet: q_nope, q_pe, ckv, kpe,
 * kv_indptr, kv_indices, kv_last_page_len, o) with the shapes of flashinfer
 * PR 844; the merge is the deterministic LSE-weighted combine of FlashMLA PR
 * 233, "What is added".  Every merge sums in a fixed
 * order, so reruns are bit-identical.  Allocates nothing, never
 * synchronises and never reads device memory from the host, so it may be
 * captured in a HIP graph and replayed.  A plan stays valid while requests
 * grow: the chunk boundaries are fixed at plan time, but the last chunk of
 * every request (and the one chunk of a request that was empty) runs to the
 * request's length as the device page table gives it at run time, so tokens
 * appended after planning (new slots, new pages, later pages renumbered in
 * kv_indptr) are decoded by the same plan and graph; only the balance of the
 * work across CUs reflects the plan-time lengths.  A request must not become
 * shorter than it was at plan time.
 *   q_nope  device bf16 [batch * qo_len, H, 512]   q_pe device bf16 [batch * qo_len, H, 64]
 *           (fp16 for MLA_KV_FP16, as are ckv, kpe and o)
 *   ckv     device [pages, P, 512]           kpe  device [pages, P, 64]
 *           (bf16, or 8-bit codes per the plan's kv_dtype)
 *   kv_scale device fp32 [pages, P] for 8-bit caches, NULL for bf16
 *   kv_indptr [batch+1], kv_indices [n], kv_last_page_len [batch]: device int32
 *           page table of the plan's batch as it stands at run time (the one the
 *           plan was made from, or the same requests grown since).  The kernel
 *           never reads past a request's device-side length; kv_indices entries
 *           must be valid page numbers (not checked on the device).
 *   sm_scale softmax scale applied to the whole 576-wide score
 *   o       device bf16 [batch * qo_len, H, 512] (written)
 *   lse     device fp32 [batch * qo_len, H] (written)
 * Results are bit-identical across runs of the same plan and inputs.
 * Errors: MLA_ERR_INVALID_ARG (null pointers, kv_scale inconsistent with the
 * dtype), MLA_ERR_NOT_UPLOADED, MLA_ERR_HIP (launch failure).
 */
mla_status mla_decode_run(mla_plan_t plan, const void* q_nope, const void* q_pe, const void* ckv,
                          const void* kpe, const float* kv_scale, const int32_t* kv_indptr,
                          const int32_t* kv_indices, const int32_t* kv_last_page_len,
                          float sm_scale, void* o, float* lse, void* stream);

/*
 * mla_decode_run without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The plan's work list and the split partials go to a
 * device array that the library holds on each GPU it runs on (one per GPU,
 * for the life of the process) of MLA_NOALLOC_SCRATCH_BYTES; each call first
 * copies the plan's work list there (hipMemcpyAsync on `stream`, from the
 * plan's host memory, which must stay alive while the call may execute),
 * then launches what mla_decode_run launches.  Nothing is allocated on the
 * device or the host.
 *   p: any plan, also one made without a workspace (workspace == NULL in
 *   mla_decode_plan); its own workspace, if any, is not used.  The other
 *   arguments, results and determinism are those of mla_decode_run.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that may overlap on one GPU (other streams, other threads,
 * other plans in flight) race and give wrong results.  Calls in order on one
 * stream are safe.
 * Errors: those of mla_decode_run (MLA_ERR_NOT_UPLOADED aside), and
 * MLA_ERR_WORKSPACE_TOO_SMALL (nothing launched; mla_last_error() gives the
 * sizes) when the plan needs more than MLA_NOALLOC_SCRATCH_BYTES, e.g. more
 * than 256 partial chunks at 128 heads.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)72 << 20)
mla_status mla_decode_run_noalloc(mla_plan_t plan, const void* q_nope, const void* q_pe,
                                  const void* ckv, const void* kpe, const float* kv_scale,
                                  const int32_t* kv_indptr, const int32_t* kv_indices,
                                  const int32_t* kv_last_page_len, float sm_scale, void* o,
                                  float* lse, void* stream);

/*
 * Optional instrumentation for measuring the decode kernel on its own: when
 * set, mla_decode_run (and mla_decode_run_noalloc) launches the decode kernel
 * so that `before` takes the start and `after` the end of that kernel's
 * execution, from its own dispatch (hipExtLaunchKernel), not the merge launch
 * of split requests that follows; a run with no decode launch records them
 * on its stream back to back.  hipEvent_t values passed as void*; the caller
 * owns them.  Passing NULL for both turns it off.  Host-only call.
 */
mla_status mla_decode_plan_set_events(mla_plan_t plan, void* before, void* after);

/* Free a plan (host memory only; the workspace stays the caller's). NULL is a no-op. */
void mla_decode_plan_destroy(mla_plan_t plan);

/* Static description of a status code. */
const char* mla_status_string(int32_t status);

/* Text of the last HIP error seen by this library on the calling thread ("" if none). */
const char* mla_last_error(void);

/*
 * Plan inspection (for tests and tools).
 *   info[0] batch, [1] num_heads, [2] page_size, [3] kv_dtype, [4] num_workers
 *   (grid size), [5] num_segments, [6] num_partials (split partial slots),
 *   [7] num_split_requests, [8] split granularity in tokens, [9] waves per
 *   workgroup, [10] head split, [11] query vectors per workgroup, [12]
 *   qo_len, [13] 1 when every workgroup runs exactly the segment of its own
 *   index (the kernels then skip the worker_ptr load), [14] c > 0 when, in
 *   addition, segment i reads the latent cache of request i / c (the kernels
 *   then load the segment record and the request's page-table entries in one
 *   round trip), else 0, [15] X > 0 when [14] applies to the rank of the
 *   segment before the workgroups were dealt to X L2 domains, rank(i) =
 *   (i % X) * (info[4] / X) + i / X, rather than to i itself.  With a head
 *   split n > 1, segment requests count groups: row r
 *   covers query vectors (r % n) * W .. (r % n) * W + W - 1 (W = info[11]) of
 *   request r / n, where query vector j is head j % num_heads of query
 *   j / num_heads.
 * mla_decode_plan_segments copies the work list: seg[4*i..4*i+3] =
 * {request, token_begin, token_end, partial_slot (-1 = writes o/lse directly)}
 * for i < num_segments (token_end as planned; a run takes the last chunk of
 * each request to the request's run-time length), and worker_ptr[w], worker_ptr[w+1] delimit the
 * segments of workgroup w (worker_ptr has num_workers + 1 entries).
 */
mla_status mla_decode_plan_info(mla_plan_t plan, int32_t info[16]);
mla_status mla_decode_plan_segments(mla_plan_t plan, int32_t* seg, int32_t* worker_ptr);

/*
 * mla_cache_append writes n new latent tokens into the paged cache, quantising
 * them when the cache is 8-bit (FlashMLA PR 233, "What is added": an FP8 e4m3
 * or INT8 latent cache with one fp32 scale per token; the layer's prologue
 * writes the cache before the decode reads it).
 *   ckv_new  device bf16 [n, 512]; kpe_new device bf16 [n, 64] (fp16 for MLA_KV_FP16)
 *   slots    device int64 [n]: destination row page * page_size + position of
 *            the cache viewed as [pages * page_size, ...]; a negative entry
 *            skips that token.  Destinations must be distinct and inside the
 *            cache (not checked on the device).
 *   ckv, kpe device cache [pages, page_size, 512] and [.., 64] of kv_dtype
 *   kv_scale device fp32 [pages, page_size] for 8-bit caches, NULL for bf16 / fp16
 * bf16 and fp16 caches: the rows are copied (ckv_new / kpe_new are then fp16 for
 * an fp16 cache).  8-bit, per token over its 576 values (ckv then kpe):
 * amax = max |x|; scale = amax / 448 (fp8) or amax / 127 (int8) in binary32,
 * 1 for an all-zero token; code = the representable value nearest to
 * x / scale (binary32 division), ties to even, saturated to +-448 / +-127.
 * The 644-byte layouts quantise the 512 ckv values the same way (amax over
 * them alone) and copy kpe as bf16 (kpe is then [pages, P, 64] bf16).
 * Errors: MLA_ERR_INVALID_ARG for n < 0, a null pointer (n > 0) or kv_scale
 * not matching kv_dtype; MLA_ERR_UNSUPPORTED for another kv_dtype.  One kernel
 * launch on stream; nothing is allocated or synchronised.
 */
mla_status mla_cache_append(const void* ckv_new, const void* kpe_new, const int64_t* slots,
                            int32_t n, int32_t kv_dtype, void* ckv, void* kpe,
                            float* kv_scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
