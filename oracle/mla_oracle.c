/*
 * Plain fp64 CPU oracle for absorbed-MQA paged MLA decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the GPU path, and the GPU path never calls it.
 *
 * What is computed (one request b, one query head h), following the pages:
 *  - "Benchmarking MLA" (flashinfer issue 700), the comments on the
 *    matrix-absorbed form: the score contraction runs over
 *    (kpe-dim + ckv-dim) = 64 + 512, the value head dim is 512 and the ckv
 *    cache serves as both key and value; the query heads all share one latent
 *    KV stream (MQA with a group size of up to 128).
 *  - same page, nvbench byte accounting: the inputs are q_nope, q_pe, ckv,
 *    kpe, kv_indptr, kv_indices and kv_last_page_len; the output is o.
 *  - FlashMLA PR 233, "What is added": paged caches with page sizes 16/32/64,
 *    and an 8-bit cache (FP8 e4m3 or INT8) with one scale per token that is
 *    dequantised before use.
 *
 *   n_b  = kv_indptr[b+1] - kv_indptr[b]                       (pages)
 *   L_b  = 0 if n_b == 0 else (n_b - 1) * P + kv_last_page_len[b]
 *   token t < L_b lives in page kv_indices[kv_indptr[b] + t / P], slot t % P
 *   K_t  = dec(ckv[page, slot, :]) * sigma_t   (512 values)
 *   R_t  = dec(kpe[page, slot, :]) * sigma_t   (64 values)
 *          sigma_t = kv_scale[page, slot] for 8-bit caches, 1 for bf16
 *   s_t  = sm_scale * (q_nope[b,h,:] . K_t + q_pe[b,h,:] . R_t)
 *   m    = max_t s_t,  Z = sum_t exp(s_t - m)
 *   LSE  = m + ln Z                     (natural log of the scaled scores)
 *   O    = sum_t (exp(s_t - m) / Z) * K_t   (512 values)
 *   An empty request (L_b = 0) gives O = 0 and LSE = -inf.
 *
 * Several queries per request (qo_len > 1, e.g. speculative tokens): the
 * query tensors are [batch * qo_len, H, *] ("perf: MLA decode kernel
 * implemented by CuTe targeted to SM80", the test's tensor shapes), query i
 * of request b is row b * qo_len + i, and the sums above run over its
 * visible tokens t < L_b - (qo_len - 1 - i) only: the queries are the last
 * qo_len positions of the sequence, the causal mask with Q at the end of the
 * score matrix ("FlashMLA SM100", the forward kernel notes on N_Q != N_K).
 * A query with no visible token gets O = 0 and LSE = -inf.
 *
 * The softmax is taken in two plain passes (max first, then sums), in logical
 * token order, in fp64, with no online rescaling, no blocking and no
 * reordering.  The split-KV merge (one partial (O_i, LSE_i) per token chunk,
 * merged with weights exp(LSE_i - LSE)) is a separate function, used only to
 * check that merging partials reproduces the unsplit result.
 *
 * Decoders (written from the format definitions, not from any library):
 *   bf16      : the upper 16 bits of an IEEE binary32.
 *   e4m3fn    : OCP 8-bit float, 1 sign, 4 exponent (bias 7), 3 mantissa bits;
 *               exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there
 *               is no infinity; the largest finite value is 448.
 *   int8      : two's complement.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define D_CKV 512
#define D_KPE 64

/*
 * Cache layouts.  BF16: ckv and kpe bf16.  FP8_E4M3 / INT8: ckv and kpe both
 * 8-bit codes, one fp32 scale per token over all 576 values (580 B / token).
 * FP8_KPE16 / INT8_KPE16: the 644-byte token record of "FlashMLA Ampere v2"
 * ("What is added", 644 instead of 1152 bytes per token), read as 512 8-bit
 * ckv codes + 64 bf16 kpe values + one fp32 scale that applies to ckv only
 * (512 + 128 + 4 = 644).  FP16: ckv and kpe fp16, and the queries are fp16 too
 * (the same page's v2 kernel takes bf16 or fp16 inputs).
 */
enum {
  ORC_BF16 = 0,
  ORC_FP8_E4M3 = 1,
  ORC_INT8 = 2,
  ORC_FP8_KPE16 = 3,
  ORC_INT8_KPE16 = 4,
  ORC_FP16 = 5
};

static int ckv_fp8(int32_t kv_dtype) { return kv_dtype == ORC_FP8_E4M3 || kv_dtype == ORC_FP8_KPE16; }
static int kpe_bf16(int32_t kv_dtype) {
  return kv_dtype == ORC_BF16 || kv_dtype == ORC_FP8_KPE16 || kv_dtype == ORC_INT8_KPE16;
}
static int valid_dtype(int32_t kv_dtype) { return kv_dtype >= ORC_BF16 && kv_dtype <= ORC_FP16; }

double oracle_dec_bf16(uint16_t bits) {
  uint32_t w = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

double oracle_dec_e4m3fn(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

double oracle_dec_int8(uint8_t code) { return (double)(int8_t)code; }

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits; exponent 0 is
   subnormal (m / 1024 * 2^-14); exponent 31 is infinity (m = 0) or NaN. */
double oracle_dec_fp16(uint16_t bits) {
  int sign = (bits >> 15) & 1;
  int e = (bits >> 10) & 31;
  int m = bits & 1023;
  double v;
  if (e == 31) return m ? NAN : (sign ? -INFINITY : INFINITY);
  if (e == 0)
    v = ldexp((double)m / 1024.0, -14);
  else
    v = ldexp(1.0 + (double)m / 1024.0, e - 15);
  return sign ? -v : v;
}

/* The 16-bit element type of q (and of a 16-bit cache) for a layout. */
static double dec16(int32_t kv_dtype, uint16_t bits) {
  return kv_dtype == ORC_FP16 ? oracle_dec_fp16(bits) : oracle_dec_bf16(bits);
}

/* Number of tokens of request b. */
int64_t oracle_kv_len(const int32_t* kv_indptr, const int32_t* kv_last_page_len, int32_t page_size,
                      int32_t b) {
  int64_t n = (int64_t)kv_indptr[b + 1] - (int64_t)kv_indptr[b];
  if (n <= 0) return 0;
  return (n - 1) * (int64_t)page_size + (int64_t)kv_last_page_len[b];
}

typedef struct {
  int32_t batch, qo_len, num_heads, page_size, kv_dtype;
  const uint16_t* q_nope; /* bf16 bits [B * qo_len, H, 512] */
  const uint16_t* q_pe;   /* bf16 bits [B * qo_len, H, 64] */
  const void* ckv;        /* [pages, P, 512] bf16 bits or 8-bit codes */
  const void* kpe;        /* [pages, P, 64]  bf16 bits or 8-bit codes */
  const float* kv_scale;  /* [pages, P] or NULL for bf16 */
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* kv_last_page_len;
  double sm_scale;
} oracle_inputs;

/* Decoded latent row of logical token t of request b: K (512) and R (64). */
static void load_token(const oracle_inputs* in, int32_t b, int64_t t, double* K, double* R) {
  int64_t P = in->page_size;
  int64_t page = in->kv_indices[(int64_t)in->kv_indptr[b] + t / P];
  int64_t slot = t % P;
  int64_t row = page * P + slot;
  double sigma = 1.0;
  int i;
  if (in->kv_dtype == ORC_BF16 || in->kv_dtype == ORC_FP16) {
    const uint16_t* c = (const uint16_t*)in->ckv + row * D_CKV;
    const uint16_t* k = (const uint16_t*)in->kpe + row * D_KPE;
    for (i = 0; i < D_CKV; ++i) K[i] = dec16(in->kv_dtype, c[i]);
    for (i = 0; i < D_KPE; ++i) R[i] = dec16(in->kv_dtype, k[i]);
    return;
  }
  sigma = (double)in->kv_scale[row];
  {
    const uint8_t* c = (const uint8_t*)in->ckv + row * D_CKV;
    for (i = 0; i < D_CKV; ++i)
      K[i] = (ckv_fp8(in->kv_dtype) ? oracle_dec_e4m3fn(c[i]) : oracle_dec_int8(c[i])) * sigma;
  }
  if (kpe_bf16(in->kv_dtype)) {
    const uint16_t* k = (const uint16_t*)in->kpe + row * D_KPE;
    for (i = 0; i < D_KPE; ++i) R[i] = oracle_dec_bf16(k[i]);
  } else {
    const uint8_t* k = (const uint8_t*)in->kpe + row * D_KPE;
    for (i = 0; i < D_KPE; ++i)
      R[i] = (ckv_fp8(in->kv_dtype) ? oracle_dec_e4m3fn(k[i]) : oracle_dec_int8(k[i])) * sigma;
  }
}

/*
 * Tokens that query i (0 <= i < qo_len) of request b may attend to: the
 * first V = L_b - (qo_len - 1 - i) tokens (none if that is not positive).
 * The qo_len queries of a request are its last qo_len positions, so the
 * causal mask is aligned to the bottom-right corner of the score matrix (the
 * "Q at the end" causal mask for N_Q != N_K that the FlashMLA SM100 release
 * notes name).  With qo_len = 1 every query sees all L_b tokens.
 */
static int64_t visible_len(const oracle_inputs* in, int32_t b, int32_t qi) {
  int64_t v = oracle_kv_len(in->kv_indptr, in->kv_last_page_len, in->page_size, b) -
              (int64_t)(in->qo_len - 1 - qi);
  return v > 0 ? v : 0;
}

/*
 * Attention of head h of query i of request b over the logical token range
 * [t0, t1) (t1 <= L_b).  The query vector is row b * qo_len + i of q_nope /
 * q_pe.  Writes the normalised output (512) and the log-sum-exp.  An empty
 * range gives O = 0, LSE = -inf.  Returns 0, or -1 on allocation failure.
 */
static int attend_range(const oracle_inputs* in, int32_t b, int32_t qi, int32_t h, int64_t t0,
                        int64_t t1, double* o, double* lse) {
  const int64_t qrow = (int64_t)b * in->qo_len + qi;
  const uint16_t* qn = in->q_nope + (qrow * in->num_heads + h) * D_CKV;
  const uint16_t* qp = in->q_pe + (qrow * in->num_heads + h) * D_KPE;
  double q[D_CKV + D_KPE];
  double K[D_CKV], R[D_KPE];
  int64_t n = t1 - t0, t;
  double* s;
  double m, Z;
  int i;

  for (i = 0; i < D_CKV; ++i) o[i] = 0.0;
  if (n <= 0) {
    *lse = -INFINITY;
    return 0;
  }
  for (i = 0; i < D_CKV; ++i) q[i] = dec16(in->kv_dtype, qn[i]);
  for (i = 0; i < D_KPE; ++i) q[D_CKV + i] = dec16(in->kv_dtype, qp[i]);

  s = (double*)malloc((size_t)n * sizeof(double));
  if (!s) return -1;

  /* pass 1: scores */
  for (t = 0; t < n; ++t) {
    double dot = 0.0;
    load_token(in, b, t0 + t, K, R);
    for (i = 0; i < D_CKV; ++i) dot += q[i] * K[i];
    for (i = 0; i < D_KPE; ++i) dot += q[D_CKV + i] * R[i];
    s[t] = in->sm_scale * dot;
  }
  /* max, normaliser, log-sum-exp */
  m = s[0];
  for (t = 1; t < n; ++t)
    if (s[t] > m) m = s[t];
  Z = 0.0;
  for (t = 0; t < n; ++t) Z += exp(s[t] - m);
  *lse = m + log(Z);
  /* pass 2: probability-weighted sum of the ckv rows */
  for (t = 0; t < n; ++t) {
    double p = exp(s[t] - m) / Z;
    load_token(in, b, t0 + t, K, R);
    for (i = 0; i < D_CKV; ++i) o[i] += p * K[i];
  }
  free(s);
  return 0;
}

typedef struct {
  const oracle_inputs* in;
  const int32_t* rows; /* flattened (b * qo_len + i) * H + h, or NULL for all */
  int64_t n_rows;
  double* o;
  double* lse;
  int64_t begin, end;
  int status;
} worker_arg;

static void* worker(void* p) {
  worker_arg* w = (worker_arg*)p;
  int64_t r;
  for (r = w->begin; r < w->end; ++r) {
    int64_t flat = w->rows ? (int64_t)w->rows[r] : r;
    int64_t qrow = flat / w->in->num_heads;
    int32_t h = (int32_t)(flat % w->in->num_heads);
    int32_t b = (int32_t)(qrow / w->in->qo_len);
    int32_t qi = (int32_t)(qrow % w->in->qo_len);
    int64_t V = visible_len(w->in, b, qi);
    if (attend_range(w->in, b, qi, h, 0, V, w->o + r * D_CKV, w->lse + r) != 0) w->status = -1;
  }
  return NULL;
}

/*
 * Full decode (or a selected list of query rows) of qo_len queries per
 * request (qo_len = 1: one new token per request).
 *   rows == NULL: all B*qo_len*H rows; o_out is [B*qo_len*H, 512], lse_out
 *                 [B*qo_len*H].
 *   rows != NULL: n_rows entries of (b * qo_len + i) * H + h; o_out is
 *                 [n_rows, 512].
 * Rows are distributed over num_threads threads in contiguous blocks; each
 * row's arithmetic is independent of the thread count.
 * Returns 0 on success, -1 on bad arguments or allocation failure.
 */
int mla_oracle_decode(int32_t batch, int32_t qo_len, int32_t num_heads, int32_t page_size,
                      int32_t kv_dtype,
                      const uint16_t* q_nope, const uint16_t* q_pe, const void* ckv, const void* kpe,
                      const float* kv_scale, const int32_t* kv_indptr, const int32_t* kv_indices,
                      const int32_t* kv_last_page_len, double sm_scale, const int32_t* rows,
                      int64_t n_rows, double* o_out, double* lse_out, int32_t num_threads) {
  oracle_inputs in;
  int64_t total, per, i;
  pthread_t* th;
  worker_arg* args;
  int status = 0;

  if (batch < 0 || qo_len < 1 || num_heads <= 0 || page_size <= 0 || !o_out || !lse_out)
    return -1;
  if (!valid_dtype(kv_dtype)) return -1;
  if (kv_dtype != ORC_BF16 && kv_dtype != ORC_FP16 && !kv_scale) return -1;
  in.batch = batch;
  in.qo_len = qo_len;
  in.num_heads = num_heads;
  in.page_size = page_size;
  in.kv_dtype = kv_dtype;
  in.q_nope = q_nope;
  in.q_pe = q_pe;
  in.ckv = ckv;
  in.kpe = kpe;
  in.kv_scale = kv_scale;
  in.kv_indptr = kv_indptr;
  in.kv_indices = kv_indices;
  in.kv_last_page_len = kv_last_page_len;
  in.sm_scale = sm_scale;

  total = rows ? n_rows : (int64_t)batch * qo_len * num_heads;
  if (total == 0) return 0;
  if (num_threads < 1) num_threads = 1;
  if (num_threads > total) num_threads = (int32_t)total;
  th = (pthread_t*)calloc((size_t)num_threads, sizeof(pthread_t));
  args = (worker_arg*)calloc((size_t)num_threads, sizeof(worker_arg));
  if (!th || !args) {
    free(th);
    free(args);
    return -1;
  }
  per = (total + num_threads - 1) / num_threads;
  for (i = 0; i < num_threads; ++i) {
    args[i].in = &in;
    args[i].rows = rows;
    args[i].n_rows = n_rows;
    args[i].o = o_out;
    args[i].lse = lse_out;
    args[i].begin = i * per < total ? i * per : total;
    args[i].end = (i + 1) * per < total ? (i + 1) * per : total;
    args[i].status = 0;
    if (num_threads == 1) {
      worker(&args[i]);
    } else if (pthread_create(&th[i], NULL, worker, &args[i]) != 0) {
      args[i].status = -1;
      th[i] = 0;
    }
  }
  if (num_threads > 1)
    for (i = 0; i < num_threads; ++i)
      if (th[i]) pthread_join(th[i], NULL);
  for (i = 0; i < num_threads; ++i)
    if (args[i].status != 0) status = -1;
  free(th);
  free(args);
  return status;
}

/*
 * Attention of one (b, i, h) over the logical token range [t0, t1) only,
 * giving the partial (O_i, LSE_i) of a split-KV chunk; tokens past the
 * query's causal limit (visible_len) carry no weight.  Returns -1 if the
 * range is outside [0, L_b].
 */
int mla_oracle_partial(int32_t batch, int32_t qo_len, int32_t num_heads, int32_t page_size,
                       int32_t kv_dtype,
                       const uint16_t* q_nope, const uint16_t* q_pe, const void* ckv, const void* kpe,
                       const float* kv_scale, const int32_t* kv_indptr, const int32_t* kv_indices,
                       const int32_t* kv_last_page_len, double sm_scale, int32_t b, int32_t qi,
                       int32_t h, int64_t t0, int64_t t1, double* o_out, double* lse_out) {
  oracle_inputs in;
  int64_t L, V;
  if (b < 0 || b >= batch || qo_len < 1 || qi < 0 || qi >= qo_len || h < 0 || h >= num_heads)
    return -1;
  if (!valid_dtype(kv_dtype) || (kv_dtype != ORC_BF16 && kv_dtype != ORC_FP16 && !kv_scale))
    return -1;
  L = oracle_kv_len(kv_indptr, kv_last_page_len, page_size, b);
  if (t0 < 0 || t1 < t0 || t1 > L) return -1;
  in.batch = batch;
  in.qo_len = qo_len;
  in.num_heads = num_heads;
  in.page_size = page_size;
  in.kv_dtype = kv_dtype;
  in.q_nope = q_nope;
  in.q_pe = q_pe;
  in.ckv = ckv;
  in.kpe = kpe;
  in.kv_scale = kv_scale;
  in.kv_indptr = kv_indptr;
  in.kv_indices = kv_indices;
  in.kv_last_page_len = kv_last_page_len;
  in.sm_scale = sm_scale;
  V = visible_len(&in, b, qi);
  return attend_range(&in, b, qi, h, t0, t1 < V ? t1 : (t0 > V ? t0 : V), o_out, lse_out);
}

/*
 * Merge of n split-KV partials of one (b, h), in the fixed order i = 0..n-1
 * (FlashMLA PR 233, "What is added": split work with a deterministic
 * combine).  With M = max_i LSE_i:
 *   LSE = M + ln sum_i exp(LSE_i - M),   O = sum_i exp(LSE_i - LSE) * O_i.
 * Partials with LSE_i = -inf (empty chunks) carry zero weight; if every
 * partial is empty the result is O = 0, LSE = -inf.
 */
void mla_oracle_combine(int32_t n, const double* lse_parts, const double* o_parts, double* o_out,
                        double* lse_out) {
  double M = -INFINITY, sum = 0.0, lse;
  int32_t i;
  int j;
  for (j = 0; j < D_CKV; ++j) o_out[j] = 0.0;
  for (i = 0; i < n; ++i)
    if (lse_parts[i] > M) M = lse_parts[i];
  if (n == 0 || M == -INFINITY) {
    *lse_out = -INFINITY;
    return;
  }
  for (i = 0; i < n; ++i) sum += exp(lse_parts[i] - M);
  lse = M + log(sum);
  for (i = 0; i < n; ++i) {
    double w = exp(lse_parts[i] - lse);
    for (j = 0; j < D_CKV; ++j) o_out[j] += w * o_parts[(int64_t)i * D_CKV + j];
  }
  *lse_out = lse;
}

/*
 * Cache append with quantisation on write (the cache-write part of the fused
 * prologue in FlashMLA PR 233, "What is added": an 8-bit latent cache, FP8
 * e4m3 or INT8, with one scale per token).  For each new token j the 576
 * values (512 ckv, then 64 kpe) are bf16; for an 8-bit cache
 *   amax  = max_i |x_i|                          (exact in binary32)
 *   scale = amax / qmax in binary32 (qmax = 448 for e4m3, 127 for int8);
 *           scale = 1 for an all-zero token
 *   v_i   = x_i / scale in binary32
 *   code_i = the e4m3 value nearest to v_i, ties to even mantissa, saturated
 *           to +-448 (never NaN); or round-to-nearest-even integer of v_i
 *           clamped to [-127, 127]
 * The divisions are the IEEE binary32 ones (the rounding of the reading that
 * both sides compute them in binary32).  For the 644-byte layouts (FP8_KPE16,
 * INT8_KPE16) only the 512 ckv values are quantised: amax runs over them
 * alone and kpe stays bf16 (kpe_codes is not written and may be NULL).  The encoder below works from the
 * format definition in the header: it finds the binade of |v| with frexp and
 * rounds the scaled value to the 3-bit mantissa grid with nearbyint (default
 * rounding mode: to nearest, ties to even).
 */
static uint8_t encode_e4m3fn(float v) {
  const int neg = signbit(v) ? 1 : 0;
  const double a = fabs((double)v);
  int code;
  if (a >= 448.0) {
    code = 0x7E;
  } else if (a < ldexp(1.0, -6)) {
    code = (int)nearbyint(a / ldexp(1.0, -9)); /* subnormal grid m/8 * 2^-6; 8 is 2^-6 */
  } else {
    int k;
    int E;
    double r;
    (void)frexp(a, &k); /* a = f 2^k, f in [0.5, 1) */
    E = k - 1;          /* a in [2^E, 2^(E+1)) */
    r = nearbyint(a / ldexp(1.0, E - 3)); /* 8 .. 16 */
    if (r >= 16.0) {
      r = 8.0;
      E += 1;
    }
    code = ((E + 7) << 3) | ((int)r - 8); /* a < 448 keeps this at or below 0x7E */
  }
  return (uint8_t)(code | (neg << 7));
}

int mla_oracle_quantize(int32_t n, int32_t kv_dtype, const uint16_t* ckv_new,
                        const uint16_t* kpe_new, uint8_t* ckv_codes, uint8_t* kpe_codes,
                        float* scales) {
  int32_t j;
  int i;
  if (!valid_dtype(kv_dtype) || kv_dtype == ORC_BF16 || kv_dtype == ORC_FP16) return -1;
  for (j = 0; j < n; ++j) {
    float x[D_CKV + D_KPE];
    float amax = 0.0f, scale;
    const float qmax = ckv_fp8(kv_dtype) ? 448.0f : 127.0f;
    const int nq = kpe_bf16(kv_dtype) ? D_CKV : D_CKV + D_KPE; /* values quantised */
    for (i = 0; i < nq; ++i) {
      const uint16_t bits = i < D_CKV ? ckv_new[(int64_t)j * D_CKV + i]
                                      : kpe_new[(int64_t)j * D_KPE + i - D_CKV];
      x[i] = (float)oracle_dec_bf16(bits);
      if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
    }
    scale = amax > 0.0f ? amax / qmax : 1.0f;
    scales[j] = scale;
    for (i = 0; i < nq; ++i) {
      const float v = x[i] / scale;
      uint8_t c;
      if (ckv_fp8(kv_dtype)) {
        c = encode_e4m3fn(v);
      } else {
        float r = nearbyintf(v);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        c = (uint8_t)(int8_t)r;
      }
      if (i < D_CKV)
        ckv_codes[(int64_t)j * D_CKV + i] = c;
      else
        kpe_codes[(int64_t)j * D_KPE + i - D_CKV] = c;
    }
  }
  return 0;
}

/* the encoder on its own, for its pins */
uint8_t oracle_enc_e4m3fn(float v) { return encode_e4m3fn(v); }
