// gfx950 kernels for paged MLA decode in its absorbed-MQA form.
//
// What is computed ("Benchmarking MLA", flashinfer issue 700: the score
// contraction runs over kpe-dim + ckv-dim = 64 + 512, ckv is both key and
// value, v dim 512, all query heads share one latent stream):
//   S^T[t, h] = sum_d K[t, d] * Q[h, d]          (d over 576 = ckv | kpe)
//   online softmax over t (log2 domain, scale * log2 e folded into the scores)
//   O^T[c, h] += sum_t ckv[t, c] * P^T[t, h]      (c over 512)
//
// Workgroup organisation (all query heads of a request in one workgroup, so
// every KV tile crosses HBM once):
//   * HG head groups of 16 heads; each wave owns one head group and TS waves
//     share a head group by splitting the tile's tokens (each keeps its own
//     softmax state; they are merged through LDS at the end of a segment).
//   * A tile of T tokens = T/16 row groups.  Each row group lives in one page
//     (row groups start on multiples of 16 and page sizes are multiples of 16),
//     so its page number is a single scalar load.
//   * KV rows stream HBM -> LDS with 16-byte direct-to-LDS loads into an
//     NSTAGE-deep ring.  Each 1 KiB LDS block holds 8 rows x 8 chunks of 16 B;
//     the chunk position inside a row is XOR-swizzled with the row so that the
//     QK operand reads (ds_read_b128) and the transposing PV operand reads
//     (ds_read_b64_tr_b16) are free of bank conflicts.
//   * QK: v_mfma_f32_16x16x32_bf16 with A = K rows (16 tokens x 8 dims per
//     lane) and B = Q^T held in registers for the whole segment, producing S^T
//     (token rows, head columns) so that every lane owns one head.
//   * PV: O^T = V^T P^T.  P^T is the S^T accumulator converted to bf16 in
//     place (no shuffles); V^T comes from LDS through the transpose read.
//     The O^T accumulator keeps each head in one lane, so the softmax rescale
//     is lane-local.
//
// Output: each segment is either a whole request (o bf16 and lse fp32 written
// directly) or a chunk of one (normalised partial O in fp16 with a power-of-two
// scale per 128-column block, and its fp32 LSE, written to a partial slot with
// plain stores).  A second launch after the decode kernel
// (mla_combine_kernel / mla_combine_many_kernel) merges the chunks of every
// split request in chunk order, weighting each by exp(LSE_i - LSE), so results
// are deterministic and no state survives from one launch to the next.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels.h"

namespace mla_gpu {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// The 16-bit element type of q, of a 16-bit cache, of P and of O is bf16, or
// fp16 with an fp16 cache (cache layout 5; "FlashMLA Ampere v2" takes bf16 or
// fp16 inputs).  Values travel in bf16-typed registers either way; these
// pick the conversion and the MFMA for the type (F16 = fp16).
template <bool F16>
__device__ __forceinline__ __bf16 to16(float x) {
  if constexpr (F16)
    return __builtin_bit_cast(__bf16, (_Float16)x);
  else
    return (__bf16)x;
}
template <bool F16>
__device__ __forceinline__ f32x4 mma_16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
template <bool F16>
__device__ __forceinline__ f32x4 mma_16x16x16(const s16x4& a, const s16x4& b, const f32x4& c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
template <bool F16>
__device__ __forceinline__ f32x16 mma_32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

#define LDS_AS __attribute__((address_space(3)))

constexpr int kRowBytes = 1152;     // 512 + 64 bf16 per latent token
constexpr int kGroupBytes = 16 * kRowBytes;  // one 16-row group = 18 blocks of 1 KiB
constexpr int kHalfGroupBytes = 8 * kRowBytes;  // rows 8..15 of a group (9 blocks)
constexpr float kLn2 = 0.69314718055994530942f;

// Wait until at most n vector-memory operations of this wave are outstanding.
// s_waitcnt needs an immediate; gfx9 encodes vmcnt in bits [3:0] and [15:14],
// expcnt [6:4] and lgkmcnt [11:8] (7 and 15 = do not wait on those).
template <int N>
__device__ __forceinline__ void vm_wait_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until tile `it` has landed in LDS, given that `later` tiles were issued
// after it, each with ITEMS loads from this wave.
template <int ITEMS, int MAXLATER>
__device__ __forceinline__ void wait_tile(int later) {
  static_assert(MAXLATER * ITEMS < 64, "vmcnt range");
  if constexpr (MAXLATER >= 3) {
    if (later >= 3) {
      vm_wait_n<3 * ITEMS>();
      return;
    }
  }
  if constexpr (MAXLATER >= 2) {
    if (later == 2) {
      vm_wait_n<2 * ITEMS>();
      return;
    }
  }
  if (later == 1)
    vm_wait_n<ITEMS>();
  else
    vm_wait_n<0>();
}

// Workgroup barrier for LDS hand-off.  __syncthreads() also fences global
// memory, which makes the compiler drain every outstanding vector load (the
// KV prefetch) first; LDS-DMA completion is tracked explicitly with wait_tile
// instead, so only this wave's LDS operations are waited for here.  The
// signal fences keep the compiler from moving memory operations across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Loads of read-only metadata through the constant address space: a
// wave-uniform address then becomes a scalar load (lgkmcnt), which does not
// queue behind the KV prefetch on vmcnt.
template <class T>
__device__ __forceinline__ T ld_const(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

// Token limit of one query column with several queries per request: column
// `col` of kernel row b (width W) is query vector j = (b - kvb R) W + col of
// request kvb, i.e. head j % H of query i = j / H, and the qo_len queries are
// the request's last positions, so query i sees tokens t < ldev - (qo_len -
// 1 - i) (the causal mask with Q at the end of the score matrix).  With
// qo_len = 1 the limit is ldev.
template <int W>
__device__ __forceinline__ int causal_limit(const DecodeArgs& a, int b, int kvb, int col,
                                            int ldev) {
  const int j = (b - kvb * a.rows_per_req) * W + col;
  return ldev - (a.qo_len - 1 - (j >> a.head_log2));
}

// 16-byte direct global -> LDS load: lane i's 16 bytes land at
// lds_base + 16 * i.  Issued as inline assembly so that the compiler does not
// treat every later LDS read as dependent on the in-flight copy (which makes it
// drain vmcnt); completion is tracked explicitly with wait_tile().
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  // one wait state between the SALU write of m0 and the LDS-DMA that reads it
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_base)
               : "memory", "m0");
}

// The same with the source split into a wave-uniform base (SGPRs) and a
// 32-bit per-lane byte offset from it.
__device__ __forceinline__ void dma16_s(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(lds_base)
               : "memory", "m0");
}

// A 16-byte global load into registers, as assembly: the compiler neither
// tracks it nor waits for it, so the caller waits (vm_wait_n, counting it
// with the direct-to-LDS loads in issue order) before any use of the result
// and before the result's registers can go out of use.
__device__ __forceinline__ bf16x8 load16_untracked(const void* p) {
  bf16x8 v;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(p));
  return v;
}

// The same for lanes 0..7 only (128 bytes at lds_base).  The exec mask is set
// and restored inside the one asm statement, so the compiler sees no divergent
// region (a register spilled and reloaded under a partial exec mask would keep
// stale values in the other lanes).
__device__ __forceinline__ void dma16_lanes8(const void* src, uint32_t lds_base) {
  uint64_t saved;
  asm volatile(
      "s_mov_b64 %0, exec\n\ts_mov_b64 exec, 0xff\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\ts_mov_b64 exec, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_base)
      : "memory", "m0");
}

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ (r >> 3); }

__device__ __forceinline__ float wave_max_16(float v) {
  // reduce over lanes that share (lane & 15): lane, lane^16, lane^32, lane^48
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float wave_sum_16(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// End of a segment, one 16-head block: normalise (merging the TS token-split
// waves of the block through LDS), then write o/lse for a whole request or the
// partial of a chunk.  acc holds O^T (lane = head lane & 15, columns
// 16 cb + 4 (lane >> 4) + i), m_run the log2-domain reference max, l_run this
// lane's share of the running sum.
constexpr int kMergeStride = 512 + 4;  // floats per head row in the merge area

template <int H, int HG, int TS>
constexpr int merge_bytes() {
  return TS > 1 ? HG * TS * 16 * kMergeStride * 4 + HG * TS * 16 * 8 : 0;
}

// Partials of split chunks are stored in fp16 with one power-of-two scale per
// (head, 128-column block): scale_exp(m) for the block's largest |value| m is
// the e with m * 2^-e in [2^14, 2^15), so every value keeps 2^-11 of m,
// relative, and cannot overflow; the stored scale is 2^e (value = fp16 x 2^e).
__device__ __forceinline__ int scale_exp(float m) {
  return min(max(__builtin_amdgcn_frexp_expf(m) - 15, -126), 127);
}

// HG here is the number of merge-slot columns: a call merges slot (ts, hg) ->
// ts * HG + hg; `hblock` is the 16-head block of the output rows it writes.
template <int H, int HG, int TS, bool F16 = false>
__device__ __forceinline__ void write_head_block(const DecodeArgs& a, f32x4 (&acc)[32],
                                                 float m_run, float l_run, int b, int slot,
                                                 int hblock, int hg, int ts, int lane,
                                                 uint8_t* smem) {
  constexpr int kWaves = HG * TS;  // merge slots: (ts, hg) -> ts * HG + hg
  const int qr = lane & 15;
  const int head = hblock * 16 + qr;
  const int mslot = ts * HG + hg;
  const float l_tot = wave_sum_16(l_run);
  if constexpr (TS == 1) {
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.f / l_tot;
    const float lse_v = empty ? -INFINITY : (m_run + __log2f(l_tot)) * kLn2;
    const size_t orow = (size_t)b * H + head;
    if (slot < 0) {
      uint16_t* op = a.o + orow * 512;
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = to16<F16>(acc[cb][i] * inv);
        *reinterpret_cast<bf16x4*>(op + cb * 16 + 4 * (lane >> 4)) = v;
      }
      if (lane < 16) a.lse[orow] = lse_v;
    } else {
      // fp16 with a scale per 128-column block k = columns 16 cb + ..., cb in
      // [8k, 8k + 8), held by the 4 lanes of this head
      uint16_t* po = reinterpret_cast<uint16_t*>(a.part_o) + ((size_t)slot * H + head) * 512 +
                     4 * (lane >> 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float mx = 0.f;
#pragma unroll
        for (int cb = 8 * k; cb < 8 * k + 8; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(acc[cb][i]));
        const int ex = scale_exp(wave_max_16(mx) * inv);
        const float mult = __builtin_amdgcn_ldexpf(inv, -ex);
#pragma unroll
        for (int cb = 8 * k; cb < 8 * k + 8; ++cb) {
          f16x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (_Float16)(acc[cb][i] * mult);
          *reinterpret_cast<f16x4*>(po + cb * 16) = v;
        }
        if (lane < 16)
          a.part_scale[((size_t)slot * H + head) * 4 + k] = __builtin_amdgcn_ldexpf(1.f, ex);
      }
      if (lane < 16) a.part_lse[(size_t)slot * H + head] = lse_v;
    }
  } else {
    // merge the TS token-split waves of each head group through LDS
    float* mo = reinterpret_cast<float*>(smem);
    float* mstat = mo + kWaves * 16 * kMergeStride;  // [wave][16][2] (m, l)
    float* mine = mo + mslot * 16 * kMergeStride;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb)
      *reinterpret_cast<f32x4*>(mine + qr * kMergeStride + cb * 16 + 4 * (lane >> 4)) =
          acc[cb];
    if (lane < 16) {
      mstat[(mslot * 16 + lane) * 2 + 0] = m_run;
      mstat[(mslot * 16 + lane) * 2 + 1] = l_tot;
    }
    lds_barrier();
    // wave (hg, ts) finalises columns [128*ts, 128*ts + 128) of its 16 heads
    constexpr int kCols = 512 / TS;
    constexpr int kIters = 16 * kCols / 8 / 64;
#pragma unroll
    for (int k = 0; k < kIters; ++k) {
      const int e = k * 64 + lane;
      const int hh = e / (kCols / 8);
      const int col = ts * kCols + (e % (kCols / 8)) * 8;
      float mw[TS];
      float M = -INFINITY;
#pragma unroll
      for (int u = 0; u < TS; ++u) {
        mw[u] = mstat[((u * HG + hg) * 16 + hh) * 2 + 0];
        M = fmaxf(M, mw[u]);
      }
      const float Mu = M == -INFINITY ? 0.f : M;
      float L = 0.f;
      float o8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o8[i] = 0.f;
#pragma unroll
      for (int u = 0; u < TS; ++u) {
        const float w = __builtin_amdgcn_exp2f(mw[u] - Mu);
        L += w * mstat[((u * HG + hg) * 16 + hh) * 2 + 1];
        const float* src = mo + (u * HG + hg) * 16 * kMergeStride + hh * kMergeStride + col;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o8[i] += w * x0[i];
          o8[4 + i] += w * x1[i];
        }
      }
      const bool empty = !(L > 0.f);
      const float inv = empty ? 0.f : 1.f / L;
      const float lse_v = empty ? -INFINITY : (M + __log2f(L)) * kLn2;
      const int hd = hblock * 16 + hh;
      if (slot < 0) {
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = to16<F16>(o8[i] * inv);
        *reinterpret_cast<bf16x8*>(a.o + ((size_t)b * H + hd) * 512 + col) = v;
        if (ts == 0 && (e % (kCols / 8)) == 0) a.lse[(size_t)b * H + hd] = lse_v;
      } else {
        // fp16 with a scale per 128-column block: its 16 threads of 8 columns
        // are 16 consecutive lanes, aligned (kCols / 8 items per head, a
        // multiple of 16)
        static_assert((kCols / 8) % 16 == 0, "whole 128-column blocks per head and wave");
        float mx = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(o8[i]));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        const int ex = scale_exp(mx * inv);
        const float mult = __builtin_amdgcn_ldexpf(inv, -ex);
        f16x8 y;
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = (_Float16)(o8[i] * mult);
        *reinterpret_cast<f16x8*>(reinterpret_cast<uint16_t*>(a.part_o) +
                                  ((size_t)slot * H + hd) * 512 + col) = y;
        if ((e & 15) == 0)
          a.part_scale[((size_t)slot * H + hd) * 4 + (col >> 7)] = __builtin_amdgcn_ldexpf(1.f, ex);
        if (ts == 0 && (e % (kCols / 8)) == 0) a.part_lse[(size_t)slot * H + hd] = lse_v;
      }
    }
    lds_barrier();  // merge area free before the next segment's loads
  }
}

// ---------------------------------------------------------------------------
// LDS-ring kernel (32 or more query heads).
//   HG   16-head blocks of the request (H = 16 HG), all in this workgroup;
//   HB   16-head blocks per wave: a wave reads each K / V operand from LDS once
//        and feeds HB MFMAs with it (HB = 2 halves the LDS traffic per flop);
//   TS   waves splitting a tile's tokens (own softmax state, merged at the end);
//   MB   16-row groups per wave per tile (MB = 2 lets PV use the 32-deep MFMA);
//   NSTAGE depth of the HBM -> LDS ring.
// Waves = (HG / HB) * TS.  Online softmax rescales lazily: the reference max
// only moves when a score exceeds it by more than 2^8, so the accumulators
// (in AGPRs when HB = 2) are rarely touched outside the MFMAs.
// ---------------------------------------------------------------------------
constexpr float kRescaleSlack = 8.f;  // log2 units

template <int HG, int HB, int TS, int MB, int NSTAGE>
struct RingShape {
  static constexpr int kWaveHeads = HG / HB;  // waves per token slice
  static constexpr int kWaves = kWaveHeads * TS;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kHeads = 16 * HG;
  static constexpr int kTile = TS * MB * 16;
  static constexpr int kGroups = kTile / 16;
  static constexpr int kItems = kGroups * 18;  // 1 KiB load blocks per tile
  // waves issue whole half groups (9 blocks): wave w takes w, w + kWaves, ...
  static constexpr int kItemsMin = 9 * ((2 * kGroups) / kWaves);
  static constexpr int kItemsRem = (2 * kGroups) % kWaves;  // waves < this take one more
  static constexpr int kStageBytes = kTile * kRowBytes;
  static constexpr int kMergeBytes = merge_bytes<16 * HG, HG, TS>();
  static constexpr int kLdsBytes =
      (NSTAGE * kStageBytes > kMergeBytes) ? NSTAGE * kStageBytes : kMergeBytes;
  static constexpr bool kOneBarrier = NSTAGE >= 3;
  static constexpr int kPvBatch = kWaves > 4 ? 2 : (HB == 2 ? 4 : 8);  // PV reads in flight
  static constexpr int kQkBatch = kWaves > 4 ? 3 : 6;                   // QK reads in flight
  static_assert(HG % HB == 0, "head blocks per wave");
  static_assert(MB == 1 || MB % 2 == 0, "MB must be 1 or even");
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

// Metadata of segment si: its record (request row, token range, partial slot)
// and the device page-table entries of the request whose latent cache it reads.
// When the plan fixes that request as r / req_div, where r is si or, with the
// workgroups dealt to req_deal L2 domains, the rank si had before the dealing,
// the page-table loads do not wait for the record, so all of them arrive in
// one memory round trip; the last-page length is loaded unconditionally (in
// bounds for every request).
struct SegMeta {
  int b, t0, send, slot, kvb, pbeg, npg, last_len;
};
__device__ __forceinline__ SegMeta load_seg(const DecodeArgs& a, int si) {
  const int* sgp = reinterpret_cast<const int*>(a.segs) + si * 8;
  SegMeta m;
  if (a.req_div > 0) {
    // One asm statement issues the three scalar loads and waits for them, so
    // the compiler can neither sink the record load below the others nor read
    // a destination before the wait.
    int rank = si;
    if (a.req_deal > 0) {
      const int per = (int)gridDim.x / a.req_deal;
      rank = (si % a.req_deal) * per + si / a.req_deal;
    }
    m.kvb = rank / a.req_div;
    typedef int i32x4s __attribute__((ext_vector_type(4)));
    typedef int i32x2s __attribute__((ext_vector_type(2)));
    i32x4s rec;
    i32x2s ip;
    int last;
    asm volatile(
        "s_load_dwordx4 %0, %3, 0x0\n\t"
        "s_load_dwordx2 %1, %4, 0x0\n\t"
        "s_load_dword %2, %5, 0x0\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&s"(rec), "=&s"(ip), "=&s"(last)
        : "s"(sgp), "s"(a.kv_indptr + m.kvb), "s"(a.kv_last_page_len + m.kvb)
        : "memory");
    m.b = rec.x;
    m.t0 = rec.y;
    m.send = rec.z;
    m.slot = rec.w;
    m.pbeg = ip.x;
    m.npg = ip.y - ip.x;
    m.last_len = last;
  } else {
    m.b = ld_const(sgp + 0);
    m.t0 = ld_const(sgp + 1);
    m.send = ld_const(sgp + 2);
    m.slot = ld_const(sgp + 3);
    m.kvb = ld_const(sgp + 7);
    m.pbeg = ld_const(a.kv_indptr + m.kvb);
    m.npg = ld_const(a.kv_indptr + m.kvb + 1) - m.pbeg;
    m.last_len = ld_const(a.kv_last_page_len + m.kvb);
  }
  return m;
}

template <int HG, int HB, int TS, int MB, int NSTAGE>
__global__ void __launch_bounds__(64 * (HG / HB) * TS)
    mla_decode_ring_kernel(const DecodeArgs a) {
  using S = RingShape<HG, HB, TS, MB, NSTAGE>;
  constexpr int H = S::kHeads;
  constexpr int T = S::kTile;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S::kLdsBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int lane = tid & 63;
  const int wh = wave % S::kWaveHeads;  // this wave's heads: blocks wh * HB .. wh * HB + HB - 1
  const int ts = wave / S::kWaveHeads;
  const int my_items = S::kItemsMin + (wave < S::kItemsRem ? 9 : 0);
  const int page_shift = a.page_shift;
  const int page_mask = (1 << page_shift) - 1;

  // ---- per-lane constant LDS offsets -------------------------------------
  // Loader: lane writes LDS slot `lane` of a block: row r = rh*8 + lane/8,
  // logical chunk = cb*8 + ((lane & 7) ^ swz(r)).
  const int ld_r_lo = lane >> 3;
  // QK operand: token row r = lane & 15, chunk c = 4*s + (lane >> 4).
  const int qr = lane & 15;
  const int qk_base = (qr >> 3) * kHalfGroupBytes + (qr & 7) * 128;
  const int qk_off_even = ((lane >> 4) ^ swz(qr)) * 16;       // s even: c & 7 = g
  const int qk_off_odd = ((4 + (lane >> 4)) ^ swz(qr)) * 16;  // s odd:  c & 7 = 4 + g
  // PV operand (transpose read): source lane s = 16G + 4j + q reads row 4G + j,
  // 8 bytes at columns c0 + 4q .. c0 + 4q + 3 of a 16-column block c0.
  const int tr_r = 4 * (lane >> 4) + ((lane >> 2) & 3);
  const int tr_q = lane & 3;
  const int tr_base = (tr_r >> 3) * kHalfGroupBytes + (tr_r & 7) * 128 + (tr_q & 1) * 8;
  int tr_off[4];
#pragma unroll
  for (int A = 0; A < 4; ++A) tr_off[A] = tr_base + (((2 * A) | (tr_q >> 1)) ^ swz(tr_r)) * 16;

  const int seg_begin = a.one_seg ? (int)blockIdx.x : ld_const(a.worker_ptr + blockIdx.x);
  const int seg_end = a.one_seg ? seg_begin + 1 : ld_const(a.worker_ptr + blockIdx.x + 1);

  for (int si = seg_begin; si < seg_end; ++si) {
    const SegMeta sm = load_seg(a, si);
    const int b = sm.b, t0 = sm.t0, send = sm.send, slot = sm.slot;
    const int kvb = sm.kvb, pbeg = sm.pbeg;
    const int ldev = sm.npg > 0 ? ((sm.npg - 1) << page_shift) + sm.last_len : 0;
    const int t1 = min(send, ldev);
    // score rows at or past tlim[hb] are masked (end of chunk, or causal limit)
    int tlim[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
      tlim[hb] = min(t1, causal_limit<H>(a, b, kvb, (wh * HB + hb) * 16 + (lane & 15), ldev));
    const int ntiles = t1 > t0 ? (t1 - t0 + T - 1) / T : 0;

    // Page numbers of the row groups of tile k (one scalar load per group;
    // a group past the end reuses the group of the last valid token).
    const int last_group = t1 > 0 ? ((t1 - 1) >> 4) << 4 : 0;
    int pg_next[S::kGroups];
    auto tile_pages = [&](int k) {
      const int tile_start = t0 + k * T;
#pragma unroll
      for (int g = 0; g < S::kGroups; ++g) {
        const int gs = min(tile_start + 16 * g, last_group);
        pg_next[g] = ld_const(a.kv_indices + pbeg + (gs >> page_shift));
      }
    };

    // Issue the direct-to-LDS loads of tile k into stage st, then prefetch the
    // page numbers of tile k + 1 so that the next issue does not wait on them.
    // Wave w loads half groups w, w + waves, ...: 9 blocks of 1 KiB (8 rows x
    // 8 chunks of ckv, then the kpe chunk) whose lane addresses differ only by
    // immediate 128-byte steps along one row.
    auto issue_tile = [&](int k, int st) {
      const int tile_start = t0 + k * T;
      int pg[S::kGroups];
#pragma unroll
      for (int g = 0; g < S::kGroups; ++g) pg[g] = pg_next[g];
      if (k + 1 < ntiles) tile_pages(k + 1);
      uint8_t* stage = smem + st * S::kStageBytes;
      for (int hh = wave; hh < 2 * S::kGroups; hh += S::kWaves) {
        const int g = hh >> 1;
        const int rh = hh & 1;
        int page = pg[0];
#pragma unroll
        for (int gg = 1; gg < S::kGroups; ++gg) page = g == gg ? pg[gg] : page;
        const int gs = min(tile_start + 16 * g, last_group);
        const int r = rh * 8 + ld_r_lo;
        const int tok = min(gs + r, t1 - 1);
        const size_t row = ((size_t)page << page_shift) + (tok & page_mask);
        const int sw = ((lane & 7) ^ swz(r)) * 16;
        const uint8_t* cbase = a.ckv + row * 1024 + sw;
        const uint8_t* kbase = a.kpe + row * 128 + sw;
        const uint32_t dst = __builtin_amdgcn_readfirstlane(
            (uint32_t)(uintptr_t)(LDS_AS uint8_t*)(stage + g * kGroupBytes + rh * 9 * 1024));
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) dma16(cbase + cb * 128, dst + cb * 1024);
        dma16(kbase, dst + 8 * 1024);
      }
    };

    auto wait_for = [&](int later) {
      constexpr int kMaxLater = S::kOneBarrier ? NSTAGE - 2 : NSTAGE - 1;
      if (my_items == S::kItemsMin)
        wait_tile<S::kItemsMin, kMaxLater>(later);
      else
        wait_tile<S::kItemsMin + 9, kMaxLater>(later);
    };

    if (ntiles > 0) tile_pages(0);
    for (int k = 0; k < NSTAGE - 1 && k < ntiles; ++k) issue_tile(k, k);

    // ---- Q^T operands of this wave's HB head blocks: 18 x 8 dims each -------
    bf16x8 qf[HB][18];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int head = (wh * HB + hb) * 16 + qr;
      const bf16x8* qn = reinterpret_cast<const bf16x8*>(a.q_nope + ((size_t)b * H + head) * 512);
      const bf16x8* qp = reinterpret_cast<const bf16x8*>(a.q_pe + ((size_t)b * H + head) * 64);
#pragma unroll
      for (int s = 0; s < 18; ++s) {
        const int c = 4 * s + (lane >> 4);
        qf[hb][s] = s < 16 ? qn[c] : qp[c - 64];
      }
    }
    // Q (and the previous segment's stores) complete before the tile loop; the
    // explicit full wait also tells the compiler that no vector load is
    // pending, so it adds no waits inside the loop (where only the LDS DMA,
    // which it does not see, is in flight).
    vm_wait_n<0>();

    float m_ref[HB], l_run[HB];
    f32x4 acc[HB][32];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      m_ref[hb] = -INFINITY;
      l_run[hb] = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) acc[hb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int it = 0; it < ntiles; ++it) {
      const int st = it % NSTAGE;
      if constexpr (!S::kOneBarrier) {
        const int nxt = it + NSTAGE - 1;
        if (nxt < ntiles) issue_tile(nxt, nxt % NSTAGE);
        wait_for(min(NSTAGE - 1, ntiles - 1 - it));
        lds_barrier();
      } else {
        wait_for(min(NSTAGE - 2, ntiles - 1 - it));
        lds_barrier();
        const int nxt = it + NSTAGE - 1;
        if (nxt < ntiles) issue_tile(nxt, nxt % NSTAGE);
      }

      const uint8_t* stage = smem + st * S::kStageBytes;
      const int tile_start = t0 + it * T;

      // ---- QK: S^T for this wave's MB row groups and HB head blocks ----------
      f32x4 sacc[HB][MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const uint8_t* gbase = stage + (ts * MB + mb) * kGroupBytes + qk_base;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) sacc[hb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s0 = 0; s0 < 18; s0 += S::kQkBatch) {
          bf16x8 kf[S::kQkBatch];
#pragma unroll
          for (int u = 0; u < S::kQkBatch; ++u) {
            const int s = s0 + u;
            kf[u] = *reinterpret_cast<const LDS_AS bf16x8*>(
                (const LDS_AS uint8_t*)(gbase + (s >> 1) * 1024 + ((s & 1) ? qk_off_odd : qk_off_even)));
          }
#pragma unroll
          for (int u = 0; u < S::kQkBatch; ++u)
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
              sacc[hb][mb] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[u], qf[hb][s0 + u], sacc[hb][mb], 0, 0, 0);
        }
      }

      // ---- online softmax (log2 domain, lazy rescale) ----------------------
      bf16x4 pb[HB][MB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        float tmax = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int row0 = tile_start + (ts * MB + mb) * 16 + 4 * (lane >> 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = (row0 + i < tlim[hb]) ? sacc[hb][mb][i] * a.scale_log2 : -INFINITY;
            sacc[hb][mb][i] = x;
            tmax = fmaxf(tmax, x);
          }
        }
        tmax = wave_max_16(tmax);
        if (__builtin_amdgcn_ballot_w64(tmax > m_ref[hb] + kRescaleSlack) != 0) {
          const float m_new = fmaxf(m_ref[hb], tmax);
          const float alpha = __builtin_amdgcn_exp2f(m_ref[hb] - m_new);  // 0 when m_ref = -inf
          l_run[hb] *= alpha;
#pragma unroll
          for (int i = 0; i < 32; ++i) acc[hb][i] *= alpha;
          m_ref[hb] = m_new;
        }
        const float m_use = m_ref[hb] == -INFINITY ? 0.f : m_ref[hb];
        float psum = 0.f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = __builtin_amdgcn_exp2f(sacc[hb][mb][i] - m_use);
            psum += p;
            pb[hb][mb][i] = (__bf16)p;
          }
        }
        l_run[hb] += psum;
      }

      // ---- PV: O^T[c, h] += V^T[c, t] P^T[t, h] ----------------------------
      if constexpr (MB == 1) {
        const uint8_t* gbase = stage + (ts * MB) * kGroupBytes;
#pragma unroll
        for (int c8 = 0; c8 < 32; c8 += S::kPvBatch) {
          s16x4 vf[S::kPvBatch];
#pragma unroll
          for (int u = 0; u < S::kPvBatch; ++u) {
            const int cb = c8 + u;
            vf[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (LDS_AS s16x4*)((LDS_AS uint8_t*)(gbase + (cb >> 2) * 1024 + tr_off[cb & 3])));
          }
#pragma unroll
          for (int u = 0; u < S::kPvBatch; ++u)
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
              acc[hb][c8 + u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                  vf[u], __builtin_bit_cast(s16x4, pb[hb][0]), acc[hb][c8 + u], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int mp = 0; mp < MB; mp += 2) {
          const uint8_t* g0 = stage + (ts * MB + mp) * kGroupBytes;
          const uint8_t* g1 = g0 + kGroupBytes;
          bf16x8 pv[HB];
#pragma unroll
          for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              pv[hb][i] = pb[hb][mp][i];
              pv[hb][4 + i] = pb[hb][mp + 1][i];
            }
#pragma unroll
          for (int c8 = 0; c8 < 32; c8 += S::kPvBatch) {
            bf16x8 vf[S::kPvBatch];
#pragma unroll
            for (int u = 0; u < S::kPvBatch; ++u) {
              const int off = ((c8 + u) >> 2) * 1024 + tr_off[(c8 + u) & 3];
              const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (LDS_AS s16x4*)((LDS_AS uint8_t*)(g0 + off)));
              const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (LDS_AS s16x4*)((LDS_AS uint8_t*)(g1 + off)));
              const bf16x4 a0 = __builtin_bit_cast(bf16x4, v0);
              const bf16x4 a1 = __builtin_bit_cast(bf16x4, v1);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                vf[u][i] = a0[i];
                vf[u][4 + i] = a1[i];
              }
            }
#pragma unroll
            for (int u = 0; u < S::kPvBatch; ++u)
#pragma unroll
              for (int hb = 0; hb < HB; ++hb)
                acc[hb][c8 + u] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[u], pv[hb], acc[hb][c8 + u], 0, 0, 0);
          }
        }
      }
      if constexpr (!S::kOneBarrier) lds_barrier();
    }
    if constexpr (S::kOneBarrier) lds_barrier();  // ring free before the merge / next segment

    // ---- epilogue -----------------------------------------------------------
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
      write_head_block<H, HG, TS>(a, acc[hb], m_ref[hb], l_run[hb], b, slot, wh * HB + hb,
                                  wh * HB + hb, ts, lane, smem);
  }
}

// ---------------------------------------------------------------------------
// Register-staged kernel for 16 or 32 heads per workgroup (HB 16-head blocks),
// with a bf16, fp8-e4m3 or int8 latent cache (KVT 0 / 1 / 2), or the 644-byte
// record with fp8 / int8 ckv and bf16 kpe (KVT 3 / 4).  At these head
// counts the work is memory bound, so what matters is the number of bytes in
// flight per CU and keeping the waves out of each other's way:
//   * NW waves (4, or 8 for int8) split a segment's 16-token groups
//     round-robin (wave w takes groups w, w + NW, ...); each wave runs its own
//     pipeline with no workgroup barrier until the end of the segment;
//   * a group is fetched with coalesced 16-byte loads per lane into registers,
//     NB groups ahead (2 with 4 waves, 1 with 8), so the vector register file
//     (not LDS) holds the data in flight;
//   * the group is then written to a wave-private 18 KiB LDS buffer in the
//     swizzled bf16 layout of the LDS ring (8-bit codes are converted exactly
//     to bf16 on the way) and consumed by the QK and PV MFMAs;
//   * Q^T (HB x 16 heads x 576) sits in LDS once per segment, [chunk][head]
//     (in registers with the fp8 580-byte and int8 644-byte records; its kpe
//     part in registers with eight waves).
// 8-bit caches (FlashMLA Ampere v2, "What is added": FP8 e4m3 or INT8 with one
// scale per token, dequantised in the kernel): codes become bf16 exactly; the
// token's scale multiplies its score (after QK, in fp32) and its probability
// (before P is rounded to bf16 for PV), which is the same as dequantising the
// row first.  With a bf16 kpe (644-byte record, the scale belongs to ckv
// only), the scale multiplies the accumulator after the 512 ckv dimensions
// and before the 64 kpe dimensions are added.
// ---------------------------------------------------------------------------
template <int HB, int KVT, int NB, int NW>
struct StreamShape {
  static constexpr int kWaves = NW;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kHeads = 16 * HB;
  static constexpr int kBufBytes = 18 * 1024;       // one 16-row bf16 group per wave
  static constexpr bool kCache16 = KVT == 0 || KVT == 5;  // bf16 or fp16 cache
  // Q^T: in registers (four waves) with the fp8 580-byte record and the int8
  // 644-byte one; in LDS, [block][chunk][head] x 16 B, otherwise (measured:
  // the fp8 644-byte record runs faster with Q^T in LDS and one buffer)
  static constexpr bool kQRegs = (KVT == 1 || KVT == 2 || KVT == 4) && NW == 4;
  // with Q^T out of LDS, each wave has two group buffers and computes two
  // groups at once (see the kernel)
  static constexpr bool kPipe = kQRegs;
  // Eight waves (two per SIMD, 256 registers each; 580-byte 8-bit record,
  // one group staged per wave): eight group buffers leave LDS room for the
  // Q^T of the 512 ckv dimensions only; the 64 kpe dimensions (QK k-steps 16
  // and 17) stay in registers.
  static constexpr bool kQKpeRegs = NW == 8;
  static constexpr int kQChunks = kQKpeRegs ? 64 : 72;  // 8-dimension chunks of Q^T in LDS
  static constexpr int kQBytes = kQRegs ? 0 : HB * kQChunks * 16 * 16;
  static constexpr int kQOffset = kWaves * kBufBytes * (kPipe ? 2 : 1);
  // end of a segment: eight waves first fold into four (waves 4..7 hand
  // their O^T, reference max and row sums to waves 0..3, lane by lane:
  // [wave & 3][32 column blocks][64 lanes] x 16 B, then 64 maxima, 64 sums),
  // then the four-wave merge (one head block at a time)
  static constexpr int kFoldFloats = 32 * 64 * 4 + 2 * 64;
  static constexpr int kFoldBytes = NW == 8 ? 4 * kFoldFloats * 4 : 0;
  static constexpr int kMergeBytes = merge_bytes<16, 1, NW == 8 ? 4 : NW>();
  static constexpr int kEndBytes = kFoldBytes > kMergeBytes ? kFoldBytes : kMergeBytes;
  static constexpr int kLdsBytes = kQOffset + kQBytes > kEndBytes ? kQOffset + kQBytes
                                                                  : kEndBytes;
  // 16-byte loads per lane per group: bf16 18; 8-bit ckv 8 + kpe 1 (8-bit) or 2 (bf16)
  static constexpr int kLoads = kCache16 ? 18 : (KVT == 3 || KVT == 4 ? 10 : 9);
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

// Cache layouts (KVT): 0 bf16; 1 / 2 fp8 e4m3 / int8 ckv and kpe with one
// scale per token (580 B); 3 / 4 fp8 e4m3 / int8 ckv, bf16 kpe, one scale per
// token for ckv (the 644-byte record).
// 8 codes (two dwords) -> 8 bf16 values, exactly.
template <int KVT>
__device__ __forceinline__ u32x4 codes_to_bf16(unsigned lo, unsigned hi) {
  u32x4 r;
  if constexpr (KVT == 1 || KVT == 3) {  // OCP fp8 e4m3: hardware conversion, scale 1
    r[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, false));
    r[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, true));
    r[2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, false));
    r[3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, true));
  } else {  // int8: |v| <= 128 is exact in bf16
    const unsigned w[2] = {lo, hi};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const unsigned x = w[k >> 1] >> (16 * (k & 1));
      bf16x2 v;
      v[0] = (__bf16)(float)(signed char)(x & 0xFF);
      v[1] = (__bf16)(float)(signed char)((x >> 8) & 0xFF);
      r[k] = __builtin_bit_cast(unsigned, v);
    }
  }
  return r;
}

template <int HB, int KVT, int NB, int NW>
__global__ void __launch_bounds__(64 * NW) mla_decode_stream_kernel(const DecodeArgs a) {
  using S = StreamShape<HB, KVT, NB, NW>;
  static_assert(NW == 4 || (NW == 8 && HB == 1 && NB == 1), "eight waves: one head block, one group each");
  constexpr int H = S::kHeads;
  constexpr bool kC16 = S::kCache16;
  constexpr bool kF16 = KVT == 5;  // fp16 q, cache, P and O
  constexpr int TS = S::kWaves;
  constexpr int NL = S::kLoads;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S::kLdsBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int page_shift = a.page_shift;
  const int page_mask = (1 << page_shift) - 1;
  uint8_t* wbuf = smem + wave * S::kBufBytes * (S::kPipe ? 2 : 1);

  const int ld_r_lo = lane >> 3;
  // QK operand: token row lane & 15, chunk 4 s + (lane >> 4)
  const int qr = lane & 15;
  const int qk_base = (qr >> 3) * kHalfGroupBytes + (qr & 7) * 128;
  const int qk_off_even = ((lane >> 4) ^ swz(qr)) * 16;
  const int qk_off_odd = ((4 + (lane >> 4)) ^ swz(qr)) * 16;
  // PV operand (transpose read), as in the ring kernel
  const int tr_r = 4 * (lane >> 4) + ((lane >> 2) & 3);
  const int tr_q = lane & 3;
  const int tr_base = (tr_r >> 3) * kHalfGroupBytes + (tr_r & 7) * 128 + (tr_q & 1) * 8;
  int tr_off[4];
#pragma unroll
  for (int A = 0; A < 4; ++A) tr_off[A] = tr_base + (((2 * A) | (tr_q >> 1)) ^ swz(tr_r)) * 16;
  // 8-bit layout: load u < 8 covers row (u >> 2) * 8 + lane / 8, bytes
  // (u & 3) * 128 + (lane & 7) * 16 of ckv, i.e. bf16 chunks c, c + 1 with
  // c = (u & 3) * 16 + 2 (lane & 7); load 8 covers row lane / 4, kpe bytes
  // (lane & 3) * 16 (chunks 64 + 2 (lane & 3), + 1).  LDS byte offsets of the
  // two converted chunks, apart from immediates:
  int st8[2][2], st8k[2];
  {
    const int xr = lane >> 3;
    const int base = ((lane >> 2) & 1) * 1024 + xr * 128;
#pragma unroll
    for (int rh = 0; rh < 2; ++rh)
#pragma unroll
      for (int e = 0; e < 2; ++e) st8[rh][e] = base + (((2 * (lane & 3) + e) ^ xr ^ rh) * 16);
    const int rk = lane >> 2;
#pragma unroll
    for (int e = 0; e < 2; ++e)
      st8k[e] = (rk >> 3) * kHalfGroupBytes + 8 * 1024 + ((rk & 7) * 8 + ((2 * (lane & 3) + e) ^ swz(rk))) * 16;
  }

  const int seg_begin = a.one_seg ? (int)blockIdx.x : ld_const(a.worker_ptr + blockIdx.x);
  const int seg_end = a.one_seg ? seg_begin + 1 : ld_const(a.worker_ptr + blockIdx.x + 1);

  for (int si = seg_begin; si < seg_end; ++si) {
    const SegMeta sm = load_seg(a, si);
    const int b = sm.b, t0 = sm.t0, send = sm.send, slot = sm.slot;
    const int kvb = sm.kvb, pbeg = sm.pbeg;
    const int ldev = sm.npg > 0 ? ((sm.npg - 1) << page_shift) + sm.last_len : 0;
    const int t1 = min(send, ldev);
    // score rows at or past tlim[hb] are masked (end of chunk, or causal limit)
    int tlim[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
      tlim[hb] = min(t1, causal_limit<H>(a, b, kvb, hb * 16 + (lane & 15), ldev));
    const int ngroups = t1 > t0 ? (t1 - t0 + 15) >> 4 : 0;
    const int nmine = ngroups > wave ? (ngroups - 1 - wave) / TS + 1 : 0;

    // Q^T of the row block.  16-bit cache: into LDS, item (block, chunk c,
    // head h) at ((block * 72 + c) * 16 + h) * 16.  Its loads go out first,
    // then the loads of this wave's first NB groups (into registers), and only
    // then is Q written to LDS: the group loads are in flight during Q's round
    // trip.  580-byte 8-bit record: in registers, as the QK B operand of
    // k-step s (head 16 hb + (lane & 15), dims 32 s + 8 (lane >> 4) .. + 7),
    // loaded before the groups; this saves each 16-token group 18 KiB of LDS
    // reads.
    constexpr int QC = S::kQChunks;
    constexpr int kQItems = S::kQRegs ? 1 : (HB * QC * 16 + S::kThreads - 1) / S::kThreads;
    u32x4 qv[kQItems];
    bf16x8 qreg[S::kQRegs ? HB : 1][S::kQRegs ? 18 : 1];
    bf16x8 qkpe[S::kQKpeRegs ? HB : 1][2];  // eight waves: k-steps 16, 17 (kpe)
    if constexpr (S::kQRegs) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const int h = hb * 16 + (lane & 15);
#pragma unroll
        for (int s = 0; s < 18; ++s) {
          const int c = 4 * s + (lane >> 4);
          qreg[hb][s] =
              c < 64 ? *reinterpret_cast<const bf16x8*>(a.q_nope + ((size_t)b * H + h) * 512 + c * 8)
                     : *reinterpret_cast<const bf16x8*>(a.q_pe + ((size_t)b * H + h) * 64 + (c - 64) * 8);
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < kQItems; ++k) {
        const int x = min(tid + k * S::kThreads, HB * QC * 16 - 1);
        const int hb = x / (QC * 16);
        const int c = (x >> 4) % QC, h = hb * 16 + (x & 15);
        qv[k] = c < 64 ? *reinterpret_cast<const u32x4*>(a.q_nope + ((size_t)b * H + h) * 512 + c * 8)
                       : *reinterpret_cast<const u32x4*>(a.q_pe + ((size_t)b * H + h) * 64 + (c - 64) * 8);
      }
      if constexpr (S::kQKpeRegs) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
          for (int s = 16; s < 18; ++s)  // chunks 4 s + (lane >> 4) = 64 .. 71: kpe
            qkpe[hb][s - 16] = *reinterpret_cast<const bf16x8*>(
                a.q_pe + ((size_t)b * H + hb * 16 + (lane & 15)) * 64 + (4 * s + (lane >> 4) - 64) * 8);
      }
    }

    // Fetch this wave's j-th group into registers: NL 16-byte loads per lane
    // (+ the four token scales of this lane's score rows for 8-bit caches).
    // Every call issues the same loads, also past the last group (then from a
    // fixed, valid address), so the number of loads in flight is the same on
    // every path and the compiler's vmcnt waits only cover the group consumed.
    const uint8_t* dummy = reinterpret_cast<const uint8_t*>(a.q_nope + (size_t)b * H * 512);
    auto fetch = [&](int j, u32x4 (&st)[NL], f32x4& sc) __attribute__((always_inline)) {
      const bool live = j < nmine;
      const int gs = t0 + 16 * (wave + TS * j);
      const int page = live ? ld_const(a.kv_indices + pbeg + (gs >> page_shift)) : 0;
      const size_t pbase = (size_t)page << page_shift;
      if constexpr (kC16) {
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) {
          const int r = rh * 8 + ld_r_lo;
          const size_t row = pbase + (min(gs + r, t1 - 1) & page_mask);
          const int sw = ((lane & 7) ^ swz(r)) * 16;
          const uint8_t* cbase = live ? a.ckv + row * 1024 + sw : dummy + sw;
          const uint8_t* kbase = live ? a.kpe + row * 128 + sw : dummy + sw;
#pragma unroll
          for (int cb = 0; cb < 8; ++cb)
            st[rh * 9 + cb] = *reinterpret_cast<const u32x4*>(cbase + cb * 128);
          st[rh * 9 + 8] = *reinterpret_cast<const u32x4*>(kbase);
        }
      } else {
#pragma unroll
        for (int rh = 0; rh < 2; ++rh) {
          const int r = rh * 8 + ld_r_lo;
          const size_t row = pbase + (min(gs + r, t1 - 1) & page_mask);
          const uint8_t* cbase = live ? a.ckv + row * 512 + (lane & 7) * 16 : dummy;
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
            st[rh * 4 + cb] = *reinterpret_cast<const u32x4*>(cbase + cb * 128);
        }
        if constexpr (KVT == 3 || KVT == 4) {  // bf16 kpe rows, as in the bf16 layout
#pragma unroll
          for (int rh = 0; rh < 2; ++rh) {
            const int r = rh * 8 + ld_r_lo;
            const size_t row = pbase + (min(gs + r, t1 - 1) & page_mask);
            const int sw = ((lane & 7) ^ swz(r)) * 16;
            st[8 + rh] = *reinterpret_cast<const u32x4*>(live ? a.kpe + row * 128 + sw : dummy + sw);
          }
        } else {
          const size_t rowk = pbase + (min(gs + (lane >> 2), t1 - 1) & page_mask);
          st[8] = *reinterpret_cast<const u32x4*>(live ? a.kpe + rowk * 64 + (lane & 3) * 16 : dummy);
        }
        // scales of score rows 4 (lane >> 4) .. + 3 (16-byte aligned, same page)
        const size_t rows = pbase + ((gs + 4 * (lane >> 4)) & page_mask);
        sc = *reinterpret_cast<const f32x4*>(live ? reinterpret_cast<const uint8_t*>(a.kv_scale + rows)
                                                  : dummy);
      }
    };

    // Consume group j from registers st: LDS write and refill (always, so the
    // memory queue looks the same on every path), then QK, online softmax and
    // PV if the group exists.
    u32x4 st[NB][NL];
    f32x4 sc[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) fetch(u, st[u], sc[u]);

    uint8_t* qlds = smem + S::kQOffset;
    lds_barrier();  // previous segment's merge / combine done with this LDS
    if constexpr (!S::kQRegs) {
      // (computed here, not hoisted out of the segment loop: kept live across
      // the loop, these addresses would be spilled, and a spill reload waits
      // for every load in flight, the group fetches above included)
      int t = tid;
      asm volatile("" : "+v"(t));
      uint8_t* qw = qlds + t * 16;  // item t + k kThreads at qw + k kThreads 16
#pragma unroll
      for (int k = 0; k < kQItems; ++k)
        if ((k + 1) * S::kThreads <= HB * QC * 16 || t + k * S::kThreads < HB * QC * 16)
          *reinterpret_cast<u32x4*>(qw + k * S::kThreads * 16) = qv[k];
      lds_barrier();
    }
    const uint8_t* qbase = qlds + ((lane >> 4) * 16 + qr) * 16;  // + (hb * 72 + s * 4) * 256

    float m_ref[HB], l_run[HB];
    f32x4 acc[HB][32];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      m_ref[hb] = -INFINITY;
      l_run[hb] = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) acc[hb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // The four stages of group j: write (the group, converted, into a wave
    // buffer; then the refill of its registers, NB groups ahead, which is
    // issued also past the last group so that every path keeps the same loads
    // in flight and the compiler's vmcnt waits cover exactly the group
    // consumed), QK, online softmax (with the rescale of O^T) and PV.
    auto stage_write = [&](int j, u32x4 (&st)[NL], f32x4& sc, uint8_t* buf)
        __attribute__((always_inline)) {
      f32x4 sig = sc;
      if constexpr (kC16) {
#pragma unroll
        for (int blk = 0; blk < 18; ++blk)
          *reinterpret_cast<u32x4*>(buf + blk * 1024 + lane * 16) = st[blk];
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int rh = u >> 2, cb = u & 3;
          *reinterpret_cast<u32x4*>(buf + rh * kHalfGroupBytes + cb * 2048 + st8[rh][0]) =
              codes_to_bf16<KVT>(st[u][0], st[u][1]);
          *reinterpret_cast<u32x4*>(buf + rh * kHalfGroupBytes + cb * 2048 + st8[rh][1]) =
              codes_to_bf16<KVT>(st[u][2], st[u][3]);
        }
        if constexpr (KVT == 3 || KVT == 4) {
#pragma unroll
          for (int rh = 0; rh < 2; ++rh)
            *reinterpret_cast<u32x4*>(buf + (rh * 9 + 8) * 1024 + lane * 16) = st[8 + rh];
        } else {
          *reinterpret_cast<u32x4*>(buf + st8k[0]) = codes_to_bf16<KVT>(st[8][0], st[8][1]);
          *reinterpret_cast<u32x4*>(buf + st8k[1]) = codes_to_bf16<KVT>(st[8][2], st[8][3]);
        }
      }
      fetch(j + NB, st, sc);  // registers free again: NB groups ahead in flight
      // scales of rows past the end are zeroed (NaN padding may sit there)
      if constexpr (!kC16) {
        const int row0 = t0 + 16 * (wave + TS * j) + 4 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) sig[i] = (row0 + i < t1) ? sig[i] : 0.f;
      }
      return sig;
    };

    // QK: S^T[16 tokens][16 heads] per head block; K from LDS, Q^T from LDS
    // or registers (kQRegs)
    struct Scores {
      f32x4 v[HB];
    };
    auto stage_qk = [&](const uint8_t* buf, const f32x4& sig) __attribute__((always_inline)) {
      const uint8_t* gbase = buf + qk_base;
      Scores sc;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) sc.v[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s0 = 0; s0 < 18; s0 += 6) {
        bf16x8 kf[6];
#pragma unroll
        for (int u = 0; u < 6; ++u) {
          const int s = s0 + u;
          kf[u] = *reinterpret_cast<const LDS_AS bf16x8*>(
              (const LDS_AS uint8_t*)(gbase + (s >> 1) * 1024 + ((s & 1) ? qk_off_odd : qk_off_even)));
        }
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          bf16x8 qf[6];
#pragma unroll
          for (int u = 0; u < 6; ++u) {
            if constexpr (S::kQRegs)
              qf[u] = qreg[hb][s0 + u];
            else if (S::kQKpeRegs && s0 + u >= 16)
              qf[u] = qkpe[hb][(s0 + u) & 1];
            else
              qf[u] = *reinterpret_cast<const LDS_AS bf16x8*>(
                  (const LDS_AS uint8_t*)(qbase + (hb * QC + (s0 + u) * 4) * 256));
          }
#pragma unroll
          for (int u = 0; u < 6; ++u) {
            // 644-byte record: the scale is ckv's, applied before the kpe steps
            if constexpr (KVT == 3 || KVT == 4)
              if (s0 + u == 16) sc.v[hb] = sc.v[hb] * sig;
            sc.v[hb] = mma_16x16x32<kF16>(kf[u], qf[u], sc.v[hb]);
          }
        }
      }
      return sc;
    };

    // online softmax, log2 domain, lazy rescale; rows past the end masked
    struct Probs {
      s16x4 v[HB];
    };
    auto stage_sm = [&](int j, Scores sacc, const f32x4& sig) __attribute__((always_inline)) {
      const int row0 = t0 + 16 * (wave + TS * j) + 4 * (lane >> 4);
      Probs pv;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float raw = (KVT == 1 || KVT == 2) ? sacc.v[hb][i] * sig[i] : sacc.v[hb][i];
          const float x = (row0 + i < tlim[hb]) ? raw * a.scale_log2 : -INFINITY;
          sacc.v[hb][i] = x;
          tmax = fmaxf(tmax, x);
        }
        tmax = wave_max_16(tmax);
        if (__builtin_amdgcn_ballot_w64(tmax > m_ref[hb] + kRescaleSlack) != 0) {
          const float m_new = fmaxf(m_ref[hb], tmax);
          const float alpha = __builtin_amdgcn_exp2f(m_ref[hb] - m_new);  // 0 when m_ref = -inf
          l_run[hb] *= alpha;
#pragma unroll
          for (int i = 0; i < 32; ++i) acc[hb][i] *= alpha;
          m_ref[hb] = m_new;
        }
        const float m_use = m_ref[hb] == -INFINITY ? 0.f : m_ref[hb];
        float psum = 0.f;
        bf16x4 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(sacc.v[hb][i] - m_use);
          psum += p;
          pb[i] = to16<kF16>(kC16 ? p : p * sig[i]);  // 8-bit: V = scale x codes
        }
        l_run[hb] += psum;
        pv.v[hb] = __builtin_bit_cast(s16x4, pb);
      }
      return pv;
    };

    // PV: O^T[c][h] += V^T[c][t] P^T[t][h]
    auto stage_pv = [&](const uint8_t* buf, const Probs& pv) __attribute__((always_inline)) {
#pragma unroll
      for (int c8 = 0; c8 < 32; c8 += 8) {
        s16x4 vf[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int cb = c8 + u;
          vf[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (LDS_AS s16x4*)((LDS_AS uint8_t*)(buf + (cb >> 2) * 1024 + tr_off[cb & 3])));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int hb = 0; hb < HB; ++hb)
            acc[hb][c8 + u] = mma_16x16x16<kF16>(vf[u], pv.v[hb], acc[hb][c8 + u]);
      }
    };

    if constexpr (S::kPipe) {
      // Two groups in the compute at once: group j + 1 is written to the
      // other buffer, then the QK of group j + 1 and the PV of group j are
      // issued together (independent work: their MFMA chains and LDS
      // latencies overlap), then the softmax of group j + 1.  The arithmetic
      // of every group is the one of the plain sequence.
      static_assert(NB == 2, "pipelined groups alternate two register sets");
      uint8_t* const buf0 = wbuf;
      uint8_t* const buf1 = wbuf + S::kBufBytes;
      Probs pcur;
      {
        const f32x4 sig = stage_write(0, st[0], sc[0], buf0);
        if (nmine > 0) pcur = stage_sm(0, stage_qk(buf0, sig), sig);
      }
      // group j is in `cur`; group j + 1 goes to `nxt` from register set u
      auto step = [&](int j, const uint8_t* cur, uint8_t* nxt, u32x4 (&stn)[NL], f32x4& scn)
          __attribute__((always_inline)) {
        const f32x4 sig = stage_write(j + 1, stn, scn, nxt);
        const Scores sn = stage_qk(nxt, sig);  // past the last group: not used
        stage_pv(cur, pcur);
        if (j + 1 < nmine) pcur = stage_sm(j + 1, sn, sig);
      };
      for (int j = 0; j < nmine; j += 2) {
        step(j, buf0, buf1, st[1], sc[1]);
        if (j + 1 >= nmine) break;
        step(j + 1, buf1, buf0, st[0], sc[0]);
      }
    } else {
      for (int j = 0; j < nmine; j += NB) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const f32x4 sig = stage_write(j + u, st[u], sc[u], wbuf);
          if (j + u < nmine) stage_pv(wbuf, stage_sm(j + u, stage_qk(wbuf, sig), sig));
        }
      }
    }

    lds_barrier();  // every wave is done with its group buffer (the merge area overlaps)
    if constexpr (NW == 8) {
      // fold waves 4..7 into waves 0..3: (m, l, O^T) of the same lane (same
      // head, same columns) combine as M = max(m, m'), O = 2^(m - M) O +
      // 2^(m' - M) O', l likewise, in a fixed order
      float* fold = reinterpret_cast<float*>(smem) + (wave & 3) * S::kFoldFloats;
      if (wave >= 4) {
#pragma unroll
        for (int cb = 0; cb < 32; ++cb)
          *reinterpret_cast<f32x4*>(fold + (cb * 64 + lane) * 4) = acc[0][cb];
        fold[32 * 256 + lane] = m_ref[0];
        fold[32 * 256 + 64 + lane] = l_run[0];
      }
      lds_barrier();
      if (wave < 4) {
        const float mp = fold[32 * 256 + lane], lp = fold[32 * 256 + 64 + lane];
        const float M = fmaxf(m_ref[0], mp);
        const float Mu = M == -INFINITY ? 0.f : M;
        const float wm = __builtin_amdgcn_exp2f(m_ref[0] - Mu);
        const float wp = __builtin_amdgcn_exp2f(mp - Mu);
#pragma unroll
        for (int cb = 0; cb < 32; ++cb)
          acc[0][cb] = acc[0][cb] * wm + *reinterpret_cast<const f32x4*>(fold + (cb * 64 + lane) * 4) * wp;
        l_run[0] = l_run[0] * wm + lp * wp;
        m_ref[0] = M;
      }
      lds_barrier();  // fold area read before the merge overwrites it
      if (wave < 4) {
        write_head_block<H, 1, 4, kF16>(a, acc[0], m_ref[0], l_run[0], b, slot, 0, 0, wave, lane,
                                        smem);
      } else {  // the merge's two barriers
        lds_barrier();
        lds_barrier();
      }
    } else {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
        write_head_block<H, 1, TS, kF16>(a, acc[hb], m_ref[hb], l_run[hb], b, slot, hb, 0, wave,
                                         lane, smem);
    }
  }
}

// ---------------------------------------------------------------------------
// Wide kernel for 128 query heads: 4 waves (one per SIMD, so each may hold up
// to 512 registers), one 32-token tile at a time from an LDS ring.
//   * QK is split across the waves by heads: wave w computes S^T for heads
//     32 w .. 32 w + 31 with v_mfma_f32_32x32x16_bf16 (A = 32 token rows of
//     the tile, B = Q^T of those heads, kept in registers for the segment), runs
//     their online softmax and writes P^T, already in the PV operand layout,
//     plus the heads' rescale factors to LDS;
//   * after a barrier, PV is split by value channels: wave w accumulates O^T
//     for channels 128 w .. 128 w + 127 of all 128 heads (256 accumulator
//     registers) from V^T (transposing reads of the same tile) and every
//     wave's P^T.
// Each LDS byte read for QK feeds 32 heads and each V^T / P^T byte read for
// PV feeds 64 flops, where a wave owning 16 heads and all 512 channels gets
// 16 flops per byte in both, so LDS bandwidth no longer caps the MFMA rate.
//
// Token order inside the MFMA reduction: S^T lane l holds rows
// 8 (r / 4) + 4 (l / 32) + r % 4 of head l % 32 (r = 0..15).  PV step ks
// (16 tokens) takes r = 8 ks .. 8 ks + 7 of that lane as its B operand, i.e.
// k = 8 g + j <-> token 16 ks + 8 (j / 4) + 4 g + j % 4 (g = l / 32); the V^T
// A operand is gathered in the same token order by two transposing reads.
// ---------------------------------------------------------------------------


// Multiply a 16-register MFMA accumulator held in AGPRs by s, in place, through
// one temporary VGPR.  Written as assembly so that the (rarely executed)
// rescale does not make the compiler move the accumulators into VGPRs, which
// costs the registers that hold Q.  The leading s_nops cover the wait states
// between an MFMA writing the AGPRs and v_accvgpr_read, the trailing one those
// before a later MFMA reads them as its accumulator.
__device__ __forceinline__ void scale_agpr16(f32x16& acc, float s) {
  float t;
  asm volatile(
      "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
#define MLA_SCALE_ONE(i)                                                      \
  "v_accvgpr_read_b32 %16, %" #i "\n\tv_mul_f32 %16, %16, %17\n\t"          \
  "v_accvgpr_write_b32 %" #i ", %16\n\t"
      MLA_SCALE_ONE(0) MLA_SCALE_ONE(1) MLA_SCALE_ONE(2) MLA_SCALE_ONE(3)
      MLA_SCALE_ONE(4) MLA_SCALE_ONE(5) MLA_SCALE_ONE(6) MLA_SCALE_ONE(7)
      MLA_SCALE_ONE(8) MLA_SCALE_ONE(9) MLA_SCALE_ONE(10) MLA_SCALE_ONE(11)
      MLA_SCALE_ONE(12) MLA_SCALE_ONE(13) MLA_SCALE_ONE(14) MLA_SCALE_ONE(15)
#undef MLA_SCALE_ONE
      "s_nop 4"
      : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]), "+a"(acc[4]), "+a"(acc[5]),
        "+a"(acc[6]), "+a"(acc[7]), "+a"(acc[8]), "+a"(acc[9]), "+a"(acc[10]), "+a"(acc[11]),
        "+a"(acc[12]), "+a"(acc[13]), "+a"(acc[14]), "+a"(acc[15]), "=&v"(t)
      : "v"(s));
}

// O^T += A B with the accumulator pinned to AGPRs.  As assembly, the
// compiler cannot move the 256 accumulator registers of the wide kernel into
// VGPRs (which then spills the Q operands, and every spill reload waits for
// the whole KV prefetch on vmcnt).  A and B are consumed when the MFMA issues;
// chained MFMAs on the same accumulator need no wait states.  The compiler
// does not know the latency of an MFMA written as assembly, so nothing may
// read or write these accumulators (a v_accvgpr_read, also one the compiler
// adds on its own to copy or spill a block, which it may place on any path
// leaving the tile loop) until enough wait states have passed.  The last MFMA
// of each tile therefore carries 32 wait states in the same statement
// (SETTLE), so no instruction can be placed between it and them; within a
// tile's MFMA sequence the loop stays spill-free, and a CPU test scans every
// path of the compiled kernels for an accumulator access too soon after such
// an MFMA.
template <bool F16 = false, bool SETTLE = false>
__device__ __forceinline__ void mfma_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (F16 && SETTLE)
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc) : "v"(a), "v"(b));
  else if constexpr (F16)
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else if constexpr (SETTLE)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// S (+)= A B with the accumulator in VGPRs, as assembly.  Were the QK MFMA of
// the wide kernel a builtin, the compiler would give its accumulator AGPRs
// (it takes the AGPR form once a kernel uses AGPRs), which O^T fills: every
// tile would then copy an O^T block out to VGPRs and back around QK.  Being
// volatile, these statements also keep the LDS reads written before them
// ahead of them (the scheduler would otherwise sink each operand read down to
// its MFMA, leaving the LDS latency exposed at every k-step).  INIT: C = 0.
// SETTLE: the MFMA is followed, in the same statement, by the wait states
// that must pass before any other instruction reads or writes its result.
#define MLA_SETTLE_NOPS "\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
#define MLA_MFMA_V(OP, TAIL)                                                   \
  if constexpr (INIT)                                                          \
    asm volatile(OP " %0, %1, %2, 0" TAIL : "=&v"(acc) : "v"(a), "v"(b));     \
  else if constexpr (AFTER_VALU)                                               \
    asm volatile("s_nop 4\n\t" OP " %0, %1, %2, %0" TAIL : "+v"(acc) : "v"(a), "v"(b)); \
  else                                                                         \
    asm volatile(OP " %0, %1, %2, %0" TAIL : "+v"(acc) : "v"(a), "v"(b));
// AFTER_VALU: C was last written by a VALU instruction (wait states first).
template <bool F16, bool INIT, bool SETTLE, bool AFTER_VALU = false>
__device__ __forceinline__ void mfma_vgpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (F16 && SETTLE) {
    MLA_MFMA_V("v_mfma_f32_32x32x16_f16", MLA_SETTLE_NOPS)
  } else if constexpr (F16) {
    MLA_MFMA_V("v_mfma_f32_32x32x16_f16", "")
  } else if constexpr (SETTLE) {
    MLA_MFMA_V("v_mfma_f32_32x32x16_bf16", MLA_SETTLE_NOPS)
  } else {
    MLA_MFMA_V("v_mfma_f32_32x32x16_bf16", "")
  }
}
#undef MLA_MFMA_V

// Wait states between the last MFMA writing AGPRs and VALU reads of them.
__device__ __forceinline__ void agpr_settle() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// A 16-register accumulator block read out of its AGPRs (after agpr_settle),
// as assembly, so that the epilogue takes one block at a time and the
// compiler does not move the 256 accumulators around to make room.
__device__ __forceinline__ f32x16 agpr_read16(const f32x16& acc) {
  f32x16 v;
  asm volatile(
#define MLA_READ_ONE(i) "v_accvgpr_read_b32 %" #i ", %" #i "\n\t"
      "v_accvgpr_read_b32 %0, %16\n\tv_accvgpr_read_b32 %1, %17\n\t"
      "v_accvgpr_read_b32 %2, %18\n\tv_accvgpr_read_b32 %3, %19\n\t"
      "v_accvgpr_read_b32 %4, %20\n\tv_accvgpr_read_b32 %5, %21\n\t"
      "v_accvgpr_read_b32 %6, %22\n\tv_accvgpr_read_b32 %7, %23\n\t"
      "v_accvgpr_read_b32 %8, %24\n\tv_accvgpr_read_b32 %9, %25\n\t"
      "v_accvgpr_read_b32 %10, %26\n\tv_accvgpr_read_b32 %11, %27\n\t"
      "v_accvgpr_read_b32 %12, %28\n\tv_accvgpr_read_b32 %13, %29\n\t"
      "v_accvgpr_read_b32 %14, %30\n\tv_accvgpr_read_b32 %15, %31"
#undef MLA_READ_ONE
      : "=v"(v[0]), "=v"(v[1]), "=v"(v[2]), "=v"(v[3]), "=v"(v[4]), "=v"(v[5]), "=v"(v[6]),
        "=v"(v[7]), "=v"(v[8]), "=v"(v[9]), "=v"(v[10]), "=v"(v[11]), "=v"(v[12]), "=v"(v[13]),
        "=v"(v[14]), "=v"(v[15])
      : "a"(acc[0]), "a"(acc[1]), "a"(acc[2]), "a"(acc[3]), "a"(acc[4]), "a"(acc[5]),
        "a"(acc[6]), "a"(acc[7]), "a"(acc[8]), "a"(acc[9]), "a"(acc[10]), "a"(acc[11]),
        "a"(acc[12]), "a"(acc[13]), "a"(acc[14]), "a"(acc[15]));
  return v;
}

// LDS of the wide kernel.  bf16 cache: a ring of kStages bf16 tiles (36 KiB,
// the swizzled 16-row group layout) filled by direct-to-LDS loads.  8-bit
// cache: a ring of kStages code tiles (ckv codes [32][512], kpe codes
// [32][64], the 32 scales; filled by direct-to-LDS loads) and two bf16 tiles:
// the codes of tile k + 1 are converted (exactly) into one of them while tile
// k is computed from the other.  644-byte record (KVT 3 / 4): the code tile
// holds bf16 kpe rows [32][64] (copied, not converted) and only the 128 bytes
// of scales.
template <int KVT>
struct WideShape {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 256;
  static constexpr int kHeads = 128;
  static constexpr int kTile = 32;
  static constexpr bool kCache16 = KVT == 0 || KVT == 5;  // bf16 or fp16 cache
  static constexpr int kStages = kCache16 ? 4 : 3;
  // QK k-steps whose Q^T operands stay in registers (8-bit: the kpe steps live
  // in LDS, to make room for the code conversion)
  static constexpr int kQRegSteps = kCache16 ? 36 : 32;
  static constexpr int kStageBytes = kTile * kRowBytes;              // 36 KiB bf16 tile
  static constexpr bool kKpe16 = KVT == 3 || KVT == 4;  // 644-byte record
  static constexpr int kCodeKpe = kTile * 512;                       // offsets in a code tile
  static constexpr int kCodeScale = kCodeKpe + kTile * 64 * (kKpe16 ? 2 : 1);
  static constexpr int kCodeBytes = kCodeScale + (kKpe16 ? 128 : 1024);  // 19 / 20.1 KiB
  static constexpr int kDmaPerWave = kCache16 ? 9 : (kKpe16 ? 6 : 5);  // loads per tile
  static constexpr int kBf16Offset = kStages * kCodeBytes;           // 8-bit: the two bf16 tiles
  static constexpr int kRingBytes = kCache16 ? kStages * kStageBytes
                                             : kBf16Offset + 2 * kStageBytes;
  static constexpr int kQOffset = kRingBytes;                        // Q^T [wave][step][lane] x 16 B
  static constexpr int kPOffset = kQOffset + 4 * (36 - kQRegSteps) * 1024;  // P^T [wave][ks][lane]
  static constexpr int kAlphaOffset = kPOffset + 4 * 2 * 64 * 16;    // [128] rescale factors
  static constexpr int kFlagOffset = kAlphaOffset + 128 * 4;         // [4] rescale flags
  static constexpr int kStatOffset = kFlagOffset + 16;               // [128] 1 / row sum
  static constexpr int kLimitOffset = kStatOffset + 128 * 4;         // [128] token limit per head
  static constexpr int kLdsBytes = kLimitOffset + 128 * 4;
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

template <int KVT, bool CAUSAL>
__global__ void __launch_bounds__(256) mla_decode_wide_kernel(const DecodeArgs a) {
  using S = WideShape<KVT>;
  constexpr int H = S::kHeads;
  constexpr bool kC16 = S::kCache16;
  constexpr bool kF16 = KVT == 5;  // fp16 q, cache, P and O
  constexpr int T = S::kTile;
  constexpr int NS = S::kStages;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S::kLdsBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int page_shift = a.page_shift;
  const int page_mask = (1 << page_shift) - 1;
  const int ld_r_lo = lane >> 3;

  // QK A operand (ds_read_b128): token l32 of the tile, chunk 2 s + g.
  int qk_off[4];
  {
    const int r = l32 & 15, half = r >> 3, rr = r & 7;
    const int base = (l32 >> 4) * kGroupBytes + half * kHalfGroupBytes + rr * 128;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) qk_off[s4] = base + (((2 * s4 + g) ^ rr ^ half) * 16);
  }
  // PV A operand (ds_read_b64_tr_b16): source lane sl of 16-lane group G reads
  // token 16 ks + 8 half + 4 (G >> 1) + sl / 4, channels
  // 128 w + 32 cb + 16 (G & 1) + 4 (sl % 4) .. + 3.
  int pv_off[2][2];  // [half][cb & 1]
  {
    const int G = lane >> 4, sl = lane & 15;
    const int rr = 4 * (G >> 1) + (sl >> 2);
    const int e = 2 * (G & 1) + ((sl >> 1) & 1);
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int c1 = 0; c1 < 2; ++c1)
        pv_off[half][c1] = half * kHalfGroupBytes + rr * 128 + (((4 * c1 + e) ^ rr ^ half) * 16) +
                           (sl & 1) * 8;
  }
  uint8_t* pbuf = smem + S::kPOffset;
  float* alpha_s = reinterpret_cast<float*>(smem + S::kAlphaOffset);
  int* flags = reinterpret_cast<int*>(smem + S::kFlagOffset);
  float* stat = reinterpret_cast<float*>(smem + S::kStatOffset);
  int* limit_s = reinterpret_cast<int*>(smem + S::kLimitOffset);

  const int seg_begin = a.one_seg ? (int)blockIdx.x : ld_const(a.worker_ptr + blockIdx.x);
  const int seg_end = a.one_seg ? seg_begin + 1 : ld_const(a.worker_ptr + blockIdx.x + 1);

  for (int si = seg_begin; si < seg_end; ++si) {
    // (580-byte 8-bit record: the per-lane offsets of the code loads and of the
    // conversion are formed from these copies, which the compiler cannot take
    // out of the segment loop: formed once at entry and kept across the
    // segments, they were spilled and reloaded at every segment)
    int lane_s = lane, tid_s = tid;
    if constexpr (KVT == 1 || KVT == 2) asm volatile("" : "+v"(lane_s), "+v"(tid_s));
    // (every 8-bit record: the Q^T loads and the epilogue's row, column and
    // lane-half take their lane indices from a per-segment copy too; the
    // 644-byte record gets one of its own for these two places only, since a
    // copy in its tile loop costs spills there)
    int lane_e = lane_s;
    if constexpr (KVT == 3 || KVT == 4) asm volatile("" : "+v"(lane_e));
    const int l32_s = lane_e & 31, g_s = lane_e >> 5;
    const SegMeta sm = load_seg(a, si);
    const int b = sm.b, t0 = sm.t0, send = sm.send, slot = sm.slot;
    const int kvb = sm.kvb, pbeg = sm.pbeg;
    const int ldev = sm.npg > 0 ? ((sm.npg - 1) << page_shift) + sm.last_len : 0;
    const int t1 = min(send, ldev);
    // CAUSAL (several queries per request): score rows of this lane's QK
    // head at or past its causal limit are masked too.  The limit is kept in
    // LDS (each wave reads only its own entries) rather than in a register,
    // which the 8-bit kernel does not have to spare.
    if constexpr (CAUSAL) {
      if (lane < 32)
        limit_s[32 * wave + l32] = min(t1, causal_limit<H>(a, b, kvb, 32 * wave + l32, ldev));
    }
    const int ntiles = t1 > t0 ? (t1 - t0 + T - 1) / T : 0;

    // Page numbers of the two 16-row groups of a tile (a group past the end
    // reuses the group of the last valid token): scalar loads, prefetched one
    // tile ahead.
    const int last_group = t1 > 0 ? ((t1 - 1) >> 4) << 4 : 0;
    int pg_next[2] = {0, 0};
    auto tile_pages = [&](int k) {
      const int kc = min(k, max(ntiles - 1, 0));
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int gs = min(t0 + kc * T + 16 * gi, last_group);
        pg_next[gi] = ld_const(a.kv_indices + pbeg + (gs >> page_shift));
      }
    };

    // Direct-to-LDS loads of tile k into ring slot st.
    //   bf16: wave w loads half group w (group w / 2, rows 8 (w % 2) .. + 7),
    //   9 blocks of 1 KiB in the swizzled layout.
    //   8-bit: wave w issues loads d = 5 w .. 5 w + 4 of 20: ckv code rows 2d,
    //   2d + 1 (d < 16), kpe code rows 16 (d - 16) .. + 15 (d = 16, 17), the 32
    //   scales (d = 18 and again d = 19, so that every wave issues 5 loads).
    //   644-byte record: d = 6 w .. 6 w + 5 of 24: ckv as above, bf16 kpe rows
    //   8 (d - 16) .. + 7 (d = 16 .. 19), the 32 scales by lanes 0..7 (d >= 20).
    //   Past the last tile, the last tile is loaded again (its data lands in
    //   a slot no one reads), which keeps the loads in flight, and so every
    //   vmcnt wait, the same in every iteration.
    // 16-bit cache: source rows and LDS destination of this wave's 9 loads of
    // tile k into slot st (load u < 8: ckv block u, load 8: kpe)
    // (a wave loads 8 rows of one 16-token group, which lies in one page: the
    // page's addresses are wave-uniform, the offsets inside it per lane)
    struct TileDma {
      const uint8_t* cpage;  // ckv / kpe of the group's page
      const uint8_t* kpage;
      uint32_t coff, koff;   // this lane's row and swizzled 16-byte piece in it
      uint32_t dst;
    };
    auto plan_tile = [&](int k, int st) __attribute__((always_inline)) {
      const int pg[2] = {pg_next[0], pg_next[1]};
      tile_pages(k + 1);
      const int kc = min(k, ntiles - 1);
      const int my_group = wave >> 1, my_half = wave & 1;
      const int gs = min(t0 + kc * T + 16 * my_group, last_group);
      const int r = my_half * 8 + ld_r_lo;
      const int tok = min(gs + r, t1 - 1);
      const size_t page_row = (size_t)pg[my_group] << page_shift;
      const uint32_t sw = ((lane & 7) ^ swz(r)) * 16;
      TileDma td;
      td.cpage = a.ckv + page_row * 1024;
      td.kpage = a.kpe + page_row * 128;
      td.coff = (tok & page_mask) * 1024 + sw;
      td.koff = (tok & page_mask) * 128 + sw;
      td.dst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(
          LDS_AS uint8_t*)(smem + st * S::kStageBytes + my_group * kGroupBytes +
                           my_half * kHalfGroupBytes));
      return td;
    };
    // The same in two steps: the page numbers of tile k (scalar loads), and
    // the plan from them (no memory access), so that the loads can be put
    // where a wait covers their latency anyway.
    auto pages_of = [&](int k, int (&pg)[2]) __attribute__((always_inline)) {
      const int kc = min(k, ntiles - 1);
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int gs = min(t0 + kc * T + 16 * gi, last_group);
        pg[gi] = ld_const(a.kv_indices + pbeg + (gs >> page_shift));
      }
    };
    auto plan_from = [&](int k, int st, const int (&pg)[2]) __attribute__((always_inline)) {
      const int kc = min(k, ntiles - 1);
      const int my_group = wave >> 1, my_half = wave & 1;
      const int gs = min(t0 + kc * T + 16 * my_group, last_group);
      const int r = my_half * 8 + ld_r_lo;
      const int tok = min(gs + r, t1 - 1);
      const size_t page_row = (size_t)pg[my_group] << page_shift;
      const uint32_t sw = ((lane & 7) ^ swz(r)) * 16;
      TileDma td;
      td.cpage = a.ckv + page_row * 1024;
      td.kpage = a.kpe + page_row * 128;
      td.coff = (tok & page_mask) * 1024 + sw;
      td.koff = (tok & page_mask) * 128 + sw;
      td.dst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(
          LDS_AS uint8_t*)(smem + st * S::kStageBytes + my_group * kGroupBytes +
                           my_half * kHalfGroupBytes));
      return td;
    };
    auto dma_one = [&](const TileDma& td, int u) __attribute__((always_inline)) {
      if (u < 8)
        dma16_s(td.cpage, td.coff + u * 128, td.dst + u * 1024);
      else
        dma16_s(td.kpage, td.koff, td.dst + 8 * 1024);
    };
    auto issue_tile = [&](int k, int st) {
      if constexpr (kC16) {
        const TileDma td = plan_tile(k, st);
#pragma unroll
        for (int u = 0; u < 9; ++u) dma_one(td, u);
      } else {
        const int pg[2] = {pg_next[0], pg_next[1]};
        tile_pages(k + 1);
        const int kc = min(k, ntiles - 1);
        const int tile0 = t0 + kc * T;
        const uint32_t dst0 = __builtin_amdgcn_readfirstlane(
            (uint32_t)(uintptr_t)(LDS_AS uint8_t*)(smem + st * S::kCodeBytes));
#pragma unroll
        for (int u = 0; u < S::kDmaPerWave; ++u) {
          const int d = S::kDmaPerWave * wave + u;  // wave-uniform
          int t, off;
          uint32_t dst;
          if (d < 16) {
            t = 2 * d + (lane_s >> 5);
            off = (lane_s & 31) * 16;
            dst = dst0 + d * 1024;
          } else if (S::kKpe16 && d < 20) {
            t = 8 * (d - 16) + (lane_s >> 3);
            off = (lane_s & 7) * 16;
            dst = dst0 + S::kCodeKpe + (d - 16) * 1024;
          } else if (!S::kKpe16 && d < 18) {
            t = 16 * (d - 16) + (lane_s >> 2);
            off = (lane_s & 3) * 16;
            dst = dst0 + S::kCodeKpe + (d - 16) * 1024;
          } else {
            t = 4 * min(lane_s, 7);  // lanes 8.. load again what lane 7 loads
            off = 0;
            dst = dst0 + S::kCodeScale;
          }
          const int dscale = S::kKpe16 ? 20 : 18;  // first scale load
          // a 16-byte read of scales covers 4 tokens: keep it inside the page
          const int tok = min(tile0 + t, d < dscale ? t1 - 1 : (t1 - 1) & ~3);
          const int gpage = t < 16 ? pg[0] : pg[1];
          const size_t row = ((size_t)gpage << page_shift) + (tok & page_mask);
          const uint8_t* src =
              d < 16 ? a.ckv + row * 512 + off
                     : (d < dscale ? a.kpe + row * (S::kKpe16 ? 128 : 64) + off
                                   : reinterpret_cast<const uint8_t*>(a.kv_scale + row));
          if (S::kKpe16 && d >= dscale)
            dma16_lanes8(src, __builtin_amdgcn_readfirstlane(dst));  // 128 bytes
          else
            dma16(src, __builtin_amdgcn_readfirstlane(dst));
        }
      }
    };

    // 8-bit: convert the codes of the tile in code slot cs to the bf16 tile
    // layout at dst (exact; the token scales are applied to S and P).
    auto convert_tile = [&](int cs, uint8_t* dst) {
      const uint8_t* cod = smem + cs * S::kCodeBytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // ckv: 1024 pieces of 16 codes
        const int p = i * 256 + tid_s;
        const int t = p >> 5, u = p & 31, r = t & 15;
        const u32x4 c = *reinterpret_cast<const u32x4*>(cod + t * 512 + u * 16);
        uint8_t* row = dst + (t >> 4) * kGroupBytes + (r >> 3) * kHalfGroupBytes + (u >> 2) * 1024 +
                       (r & 7) * 128;
        *reinterpret_cast<u32x4*>(row + ((((2 * u) & 7) ^ swz(r)) * 16)) =
            codes_to_bf16<KVT>(c[0], c[1]);
        *reinterpret_cast<u32x4*>(row + ((((2 * u + 1) & 7) ^ swz(r)) * 16)) =
            codes_to_bf16<KVT>(c[2], c[3]);
      }
      if constexpr (S::kKpe16) {  // bf16 kpe: 256 pieces of 8 values, copied
        const int t = tid_s >> 3, u = tid_s & 7, r = t & 15;
        const u32x4 c = *reinterpret_cast<const u32x4*>(cod + S::kCodeKpe + t * 128 + u * 16);
        uint8_t* row = dst + (t >> 4) * kGroupBytes + (r >> 3) * kHalfGroupBytes + 8 * 1024 +
                       (r & 7) * 128;
        *reinterpret_cast<u32x4*>(row + ((u ^ swz(r)) * 16)) = c;
      } else if (wave < 2) {  // kpe: 128 pieces
        const int t = tid_s >> 2, u = tid_s & 3, r = t & 15;
        const u32x4 c = *reinterpret_cast<const u32x4*>(cod + S::kCodeKpe + t * 64 + u * 16);
        uint8_t* row = dst + (t >> 4) * kGroupBytes + (r >> 3) * kHalfGroupBytes + 8 * 1024 +
                       (r & 7) * 128;
        *reinterpret_cast<u32x4*>(row + (((2 * u) ^ swz(r)) * 16)) = codes_to_bf16<KVT>(c[0], c[1]);
        *reinterpret_cast<u32x4*>(row + (((2 * u + 1) ^ swz(r)) * 16)) =
            codes_to_bf16<KVT>(c[2], c[3]);
      }
    };

    // Q^T of heads 32 w .. 32 w + 31: k-step s holds dims 16 s + 8 g .. + 7.
    constexpr int QR = S::kQRegSteps;
    bf16x8 qf[QR];
    uint8_t* const qlds = smem + S::kQOffset + wave * (36 - QR) * 1024 + lane_e * 16;
    const int qhead = 32 * wave + l32_s;
    const bf16x8* qn = reinterpret_cast<const bf16x8*>(a.q_nope + ((size_t)b * H + qhead) * 512);
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(a.q_pe + ((size_t)b * H + qhead) * 64);
    if constexpr (kC16) {
      // Q first, then the first tiles, and a wait for Q alone (loads complete
      // in issue order): the first QK starts once Q and tile 0 are in, not
      // the whole prologue
#pragma unroll
      for (int s = 0; s < 36; ++s)
        qf[s] = load16_untracked(s < 32 ? qn + 2 * s + g_s : qp + 2 * (s - 32) + g_s);
      // (tiles past the last one load the last tile again, into a ring slot
      // that is not read: every wait below is then the same constant)
      if (ntiles > 0) {
        tile_pages(0);
#pragma unroll
        for (int k = 0; k < NS - 1; ++k) issue_tile(k, k);
        vm_wait_n<9 * (NS - 1)>();
      } else {
        vm_wait_n<0>();  // no tile: nothing may stay in flight
      }
    } else {
      if (ntiles > 0) {
        tile_pages(0);
        for (int k = 0; k < NS - 1; ++k) issue_tile(k, k);
      }
#pragma unroll
      for (int s = 0; s < 36; ++s) {
        const bf16x8 v = s < 32 ? qn[2 * s + g_s] : qp[2 * (s - 32) + g_s];
        if (s < QR)
          qf[s < QR ? s : 0] = v;
        else
          *reinterpret_cast<bf16x8*>(qlds + (s - QR) * 1024) = v;
      }
      vm_wait_n<0>();
    }
    if constexpr (!kC16) {
      if (ntiles > 0) {
        lds_barrier();  // code tile 0 of every wave
        convert_tile(0, smem + S::kBf16Offset);
      }
    }

    f32x16 acc[4][4];  // O^T [channel block cb][head block hb]
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[cb][hb][i] = 0.f;
    float m_ref = -INFINITY;  // head 32 w + l32, log2 domain
    float l_run = 0.f;        // this lane's 16 tokens of that head

    if constexpr (kC16) {
      // ---- 16-bit cache: software-pipelined tile loop ------------------------
      // Iteration it: [tile it + 1 landed; barrier] P^T and the rescale of
      // tile it, kept in registers since its softmax, go to LDS; QK of tile
      // it + 1, with the loads of tile it + 3 issued one per k-step group;
      // [barrier] PV of tile it, with the softmax of tile it + 1 placed
      // between its MFMAs: the VALU work of the softmax issues while the
      // matrix core works instead of between the two contractions.  Tiles it ..
      // it + 3 fill the 4 ring slots (tile it + 3 goes to the slot of tile
      // it - 1, whose PV every wave finished before the first barrier).  The
      // arithmetic of every tile is the one of a loop without the overlap.
      static_assert(NS == 4 && QR == 36, "16-bit pipeline: 4 ring slots, Q^T in registers");
      f32x16 sacc;                  // scores of the tile whose softmax comes next
      bf16x8 pq0 = {}, pq1 = {};    // P^T of the last softmaxed tile (PV B operand)
      float alpha_q = 1.f;          // its rescale factor (1: none)
      unsigned resc_q = 0;          // wave-uniform: its softmax moved the reference max
      float tmax = -INFINITY, psum = 0.f, m_use = 0.f;
      const int tlim = CAUSAL ? limit_s[32 * wave + l32] : t1;
      // LDS addresses of the P^T, rescale-factor and flag areas: one opaque
      // base, so that the accesses take immediate offsets from two per-lane
      // registers instead of a register per address
      uint32_t small_base = (uint32_t)(uintptr_t)(LDS_AS uint8_t*)(smem + S::kPOffset);
      asm volatile("" : "+s"(small_base));
      const uint32_t p_lane = small_base + lane * 16;  // P^T [wave][ks][lane]
      const uint32_t a_lane = small_base + l32 * 4;    // alpha [head]
      constexpr uint32_t kAl = S::kAlphaOffset - S::kPOffset, kFl = S::kFlagOffset - S::kPOffset;
      auto lds_at = [](uint32_t addr) __attribute__((always_inline)) {
        return (LDS_AS uint8_t*)(uintptr_t)addr;
      };

      // QK: S^T[32 tokens][32 heads of this wave] of the tile at `stage`.  The
      // K operands of k-step group g are read two groups ahead (every wave
      // reads the whole tile here, so LDS latency is several MFMA durations);
      // the loads of a later tile go out one per group.  The scheduling
      // barriers keep each group's reads, MFMAs and load where they are put.
      auto qk_tile = [&](const uint8_t* stage, bool dma_on, const TileDma& tdma)
          __attribute__((always_inline)) {
        // qk_off[u] = qk_off[0] ^ 32 u (the swizzle flips bits 5-6 only, and the
        // tile base is a multiple of 1 KiB), so one register per tile serves all 4
        // (computed here, per tile: kept live across the loop, such addresses
        // are spilled, and a spill reload waits for every load in flight)
        uint32_t kbase = (uint32_t)(uintptr_t)(LDS_AS uint8_t*)stage + qk_off[0];
        asm volatile("" : "+v"(kbase));
        auto read_k = [&](int gi, bf16x8 (&kf)[4]) __attribute__((always_inline)) {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            kf[u] = *reinterpret_cast<const LDS_AS bf16x8*>(
                lds_at((kbase ^ (32u * u)) + gi * 1024));
        };
        bf16x8 kq[3][4];
        read_k(0, kq[0]);
        read_k(1, kq[1]);
#pragma unroll
        for (int gi = 0; gi < 9; ++gi) {
          if (gi + 2 < 9) read_k(gi + 2, kq[(gi + 2) % 3]);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int s = 4 * gi + u;
            if (s == 0)
              mfma_vgpr<kF16, true, false>(sacc, kq[gi % 3][u], qf[s]);
            else if (s == 35)
              mfma_vgpr<kF16, false, true>(sacc, kq[gi % 3][u], qf[s]);
            else
              mfma_vgpr<kF16, false, false>(sacc, kq[gi % 3][u], qf[s]);
          }
          if (dma_on) dma_one(tdma, gi);
          __builtin_amdgcn_sched_barrier(0);
        }
      };

      // Online softmax of the scores in sacc (log2 domain, lazy rescale), cut
      // into 32 slots so that PV can issue one slot behind each of its 32
      // MFMAs, while the matrix core is busy with it (a wave's VALU work
      // overlaps its own MFMAs as long as a slot stays within about 4 simple
      // instructions).  sacc holds raw scores here, -inf where masked
      // (mask_tile); the scale s = sm_scale log2 e > 0 commutes with the max,
      // so the row max is taken over raw scores and scaled once, and each
      // probability is exp2(fma(raw, s, -m)).  Slots 0-3: row max over this
      // lane's 16 scores; 4: with the other lane half of the head; 5-7: the
      // rescale decision (alpha = 1 unless the wave moves its reference max; a
      // head with no visible token so far keeps alpha = 1) and the new
      // reference; 8-23: the probabilities, summed in pairs (r, r + 8) in
      // order r = 0..7; 24: the row sum.
      float m_next = 0.f;
      auto sm_slot = [&](int j) __attribute__((always_inline)) {
        if (j < 4) {
          tmax = fmaxf(fmaxf(tmax, sacc[4 * j]), sacc[4 * j + 1]);
          tmax = fmaxf(fmaxf(tmax, sacc[4 * j + 2]), sacc[4 * j + 3]);
        } else if (j == 4) {
          // max with lane l ^ 32 (the same head's other 16 tokens)
          float lo = tmax, hi = tmax;
          asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1"
                       : "+v"(lo), "+v"(hi));
          tmax = fmaxf(lo, hi) * a.scale_log2;
        } else if (j == 5) {
          resc_q = __builtin_amdgcn_ballot_w64(tmax > m_ref + kRescaleSlack) != 0 ? 1u : 0u;
          m_next = resc_q ? fmaxf(m_ref, tmax) : m_ref;
        } else if (j == 6) {
          alpha_q = (resc_q && m_next != -INFINITY) ? __builtin_amdgcn_exp2f(m_ref - m_next) : 1.f;
          m_ref = m_next;
          m_use = m_ref == -INFINITY ? 0.f : -m_ref;  // the negated reference
        } else if (j == 7) {
          l_run *= alpha_q;
          tmax = -INFINITY;
          psum = 0.f;
        } else if (j < 24) {
          const int r = (j - 8) >> 1;
          if (((j - 8) & 1) == 0) {
            sacc[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], a.scale_log2, m_use));
          } else {
            const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[8 + r], a.scale_log2, m_use));
            psum += sacc[r] + e1;
            pq0[r] = to16<kF16>(sacc[r]);
            pq1[r] = to16<kF16>(e1);
          }
        } else if (j == 24) {
          l_run += psum;
        }
      };
      // Scores of tokens past this lane's limit become -inf, in one pass when
      // the tile is not visible to every head of the wave (the last tiles of a
      // segment, or the causal tail), so that the slots need no per-element mask
      auto mask_tile = [&](int tile_start) __attribute__((always_inline)) {
        if (__builtin_amdgcn_ballot_w64(tile_start + T > tlim) != 0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int tok = tile_start + 8 * (r >> 2) + 4 * g + (r & 3);
            sacc[r] = tok < tlim ? sacc[r] : -INFINITY;
          }
        }
      };

      // PV of the tile at `stage` (P^T of every wave and the rescale flags are
      // in LDS); WITH_SM: the softmax slots of the next tile behind its MFMAs.
      auto pv_tile = [&](auto with_sm, const uint8_t* stage)
          __attribute__((always_inline)) {
        constexpr bool kSm = decltype(with_sm)::value;
        // pv_off[h][c1] = (pv_off[0][0] ^ (16 h + 64 c1)) + 9216 h (the swizzle
        // flips bits 4 and 6 only; tile and block bases are multiples of 1 KiB),
        // so the 4 addresses of a tile come from one register, the rest are
        // immediates
        uint32_t vt = (uint32_t)(uintptr_t)(LDS_AS uint8_t*)stage + 2048 * wave + pv_off[0][0];
        asm volatile("" : "+v"(vt));
        uint32_t vx[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int c1 = 0; c1 < 2; ++c1) vx[h][c1] = vt ^ (16u * h + 64u * c1);
        auto read_v = [&](int i) __attribute__((always_inline)) {
          const uint32_t off = (i >> 2) * kGroupBytes + ((i & 3) >> 1) * 1024;
          const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (LDS_AS s16x4*)lds_at(vx[0][i & 1] + off));
          const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (LDS_AS s16x4*)lds_at(vx[1][i & 1] + off + kHalfGroupBytes));
          const bf16x4 a0 = __builtin_bit_cast(bf16x4, v0);
          const bf16x4 a1 = __builtin_bit_cast(bf16x4, v1);
          bf16x8 vf;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            vf[jj] = a0[jj];
            vf[4 + jj] = a1[jj];
          }
          return vf;
        };
        const u32x4 fl = *reinterpret_cast<const LDS_AS u32x4*>(lds_at(small_base + kFl));
        bf16x8 vcur = read_v(0);  // V^T of step i; step i + 1 is read at the start of step i
        // P^T operands of k-step 0; those of k-step 1 into the same registers,
        // each right after the last MFMA that reads its k-step-0 operand
        bf16x8 pb[4];
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          pb[hb] = *reinterpret_cast<const LDS_AS bf16x8*>(lds_at(p_lane + (hb * 2) * 1024));
        {
          const unsigned any = __builtin_amdgcn_readfirstlane(fl[0] | fl[1] | fl[2] | fl[3]);
          if (any != 0) {
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) {
              if (__builtin_amdgcn_readfirstlane(fl[hb]) != 0) {
                const float al = *reinterpret_cast<const LDS_AS float*>(
                    lds_at(a_lane + kAl + 128 * hb));
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) scale_agpr16(acc[cb][hb], al);
              }
            }
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int cb = i & 3;
          const bf16x8 vnext = read_v(i < 7 ? i + 1 : i);
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) {
            if (i == 7 && hb == 3)
              mfma_agpr<kF16, true>(acc[cb][hb], vcur, pb[hb]);
            else
              mfma_agpr<kF16>(acc[cb][hb], vcur, pb[hb]);
            if (i == 3)
              pb[hb] = *reinterpret_cast<const LDS_AS bf16x8*>(lds_at(p_lane + (hb * 2 + 1) * 1024));
            if constexpr (kSm) {
              __builtin_amdgcn_sched_barrier(0);
              sm_slot(4 * i + hb);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          vcur = vnext;
        }
      };

      // The page numbers of tile it + 3 are loaded at the top of iteration
      // it: scalar loads share the lgkm counter with LDS reads and complete
      // out of order, so a wait for any K read issued after them would be a
      // wait for all; issued before the tile wait and the barrier, whose own
      // lgkm wait covers them, their latency is hidden.
      if (ntiles > 0) {
        // tile 0 landed (tiles 1 and 2 may be in flight), QK and softmax of it
        vm_wait_n<18>();
        lds_barrier();
        qk_tile(smem, false, TileDma{});
        mask_tile(t0);
#pragma unroll
        for (int j = 0; j < 32; ++j) sm_slot(j);
      }
      auto iteration = [&](auto with_sm, int it) __attribute__((always_inline)) {
        constexpr bool nxt = decltype(with_sm)::value;  // a tile it + 1 exists
        // tile it + 1 landed: tiles 0 .. it + 2 have been issued (the last
        // ones possibly as reloads of the last tile), so tile it + 2 may still
        // be in flight
        int pg3[2] = {0, 0};
        if constexpr (nxt) {
          pages_of(it + 3, pg3);
          vm_wait_n<9>();
        }
        lds_barrier();  // PV of tile it - 1 done everywhere; tile it + 1 in LDS
        *reinterpret_cast<LDS_AS bf16x8*>(lds_at(p_lane + wave * 2048)) = pq0;
        *reinterpret_cast<LDS_AS bf16x8*>(lds_at(p_lane + wave * 2048 + 1024)) = pq1;
        if (resc_q && lane < 32)
          *reinterpret_cast<LDS_AS float*>(lds_at(a_lane + kAl + 128 * wave)) = alpha_q;
        // (tile 0: the accumulators are still zero, nothing to rescale; a flag
        // rather than a branch on it, so that the loop is not peeled for it)
        if (lane == 0)
          *reinterpret_cast<LDS_AS unsigned*>(lds_at(small_base + kFl + 4 * wave)) =
              it > 0 ? resc_q : 0u;
        if constexpr (nxt) {
          // tile it + 3 into the slot of tile it - 1 (past the end: the last
          // tile again)
          const TileDma tdma = plan_from(it + 3, (it + 3) % NS, pg3);
          qk_tile(smem + ((it + 1) % NS) * S::kStageBytes, true, tdma);
          mask_tile(t0 + (it + 1) * T);
        }
        lds_barrier();  // P^T and the rescale of tile it from every wave
        pv_tile(with_sm, smem + (it % NS) * S::kStageBytes);
      };
      for (int it = 0; it + 1 < ntiles; ++it) iteration(std::true_type{}, it);
      if (ntiles > 0) iteration(std::false_type{}, ntiles - 1);
      vm_wait_n<0>();  // the trailing reloads have landed (their slots are reused)
    }

    // 8-bit cache: one tile per iteration (QK, softmax, PV in turn); the codes
    // of the next tile are converted to bf16 while the current one is computed
    if constexpr (!kC16)
    for (int it = 0; it < ntiles; ++it) {
      // code tile it + 1 landed (tiles it + 2 .. it + NS - 2 may be in
      // flight); bf16 tile `it` converted; iteration it - 1 done everywhere
      vm_wait_n<S::kDmaPerWave * (NS - 3)>();
      lds_barrier();
      issue_tile(it + NS - 1, (it + NS - 1) % NS);
      if (it + 1 < ntiles)
        convert_tile((it + 1) % NS, smem + S::kBf16Offset + ((it + 1) & 1) * S::kStageBytes);
      const uint8_t* stage = smem + S::kBf16Offset + (it & 1) * S::kStageBytes;
      const int tile_start = t0 + it * T;

      // 8-bit: the token scales of this lane's score rows (rows past the end may
      // hold any scale, NaN padding included: zeroed)
      f32x16 sig;
      auto load_sig = [&]() __attribute__((always_inline)) {
        const float* sc = reinterpret_cast<const float*>(smem + (it % NS) * S::kCodeBytes +
                                                         S::kCodeScale);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(sc + 8 * j + 4 * g);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = tile_start + 8 * j + 4 * g + i;
            sig[4 * j + i] = tok < t1 ? v[i] : 0.f;
          }
        }
      };

      // ---- QK: S^T[32 tokens][32 heads of this wave] ------------------------
      // Operands of the 4 k-steps of group g (1 KiB block g of the tile; for
      // the kpe k-steps, whose Q^T lives in LDS, that Q operand too), read
      // just before the group's MFMAs (the registers for a second group are
      // not there).  The chain accumulates in VGPRs; its last MFMA (and, in
      // the 644-byte variant, the last ckv step, which the token scale then
      // multiplies) settles.
      f32x16 sacc;
      auto read_k = [&](int g, bf16x8 (&kf)[4], bf16x8 (&qx)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          kf[u] = *reinterpret_cast<const LDS_AS bf16x8*>(
              (const LDS_AS uint8_t*)(stage + g * 1024 + qk_off[u]));
          if (4 * g + u >= QR)
            qx[u] = *reinterpret_cast<const LDS_AS bf16x8*>(
                (const LDS_AS uint8_t*)(qlds + (4 * g + u - QR) * 1024));
        }
      };
      bf16x8 kcur[4], qcur[4];
#pragma unroll
      for (int s0 = 0; s0 < 36; s0 += 4) {
        if constexpr (S::kKpe16) {
          // 644-byte record: the scale is ckv's, applied before the kpe steps
          if (s0 == 32) {
            load_sig();
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[r] *= sig[r];
          }
        }
        read_k(s0 >> 2, kcur, qcur);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int s = s0 + u;
          const bf16x8 qv = s < QR ? qf[s < QR ? s : 0] : qcur[u];
          if (s == 0)
            mfma_vgpr<kF16, true, false>(sacc, kcur[u], qv);
          else if (S::kKpe16 && s == 32)
            mfma_vgpr<kF16, false, false, true>(sacc, kcur[u], qv);
          else if (s == 35 || (S::kKpe16 && s == 31))
            mfma_vgpr<kF16, false, true>(sacc, kcur[u], qv);
          else
            mfma_vgpr<kF16, false, false>(sacc, kcur[u], qv);
        }
      }

      // ---- online softmax of this wave's heads (log2 domain, lazy rescale) --
      // 8-bit: the token scale multiplies the score (after QK, in fp32) and the
      // probability (before P is rounded to bf16 for PV), the same as
      // dequantising the row first.
      if constexpr (KVT == 1 || KVT == 2) load_sig();
      if constexpr (S::kKpe16) {
        // read the scales again rather than keep them live through the kpe
        // steps (the compiler barrier stops it from reusing the first read)
        asm volatile("" ::: "memory");
        load_sig();
      }
      const int tlim = CAUSAL ? limit_s[32 * wave + l32] : t1;
      float tmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = tile_start + 8 * (r >> 2) + 4 * g + (r & 3);
        const float raw = (KVT == 1 || KVT == 2) ? sacc[r] * sig[r] : sacc[r];
        const float x = tok < tlim ? raw * a.scale_log2 : -INFINITY;
        sacc[r] = x;
        tmax = fmaxf(tmax, x);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      if (__builtin_amdgcn_ballot_w64(tmax > m_ref + kRescaleSlack) != 0) {
        const float m_new = fmaxf(m_ref, tmax);
        // 0 when m_ref = -inf; 1 for a head with no visible token yet (its
        // wave may hold another query's heads that moved the max)
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
        l_run *= alpha;
        m_ref = m_new;
        if (lane < 32) alpha_s[32 * wave + lane] = alpha;
        if (lane == 0) flags[wave] = 1;
      } else if (lane == 0) {
        flags[wave] = 0;
      }
      {
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
        float psum = 0.f;
        bf16x8 p0, p1;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float e0 = __builtin_amdgcn_exp2f(sacc[r] - m_use);
          const float e1 = __builtin_amdgcn_exp2f(sacc[8 + r] - m_use);
          psum += e0 + e1;
          p0[r] = to16<kF16>(e0 * sig[r]);  // V = scale x codes
          p1[r] = to16<kF16>(e1 * sig[8 + r]);
        }
        l_run += psum;
        *reinterpret_cast<bf16x8*>(pbuf + ((wave * 2 + 0) * 64 + lane) * 16) = p0;
        *reinterpret_cast<bf16x8*>(pbuf + ((wave * 2 + 1) * 64 + lane) * 16) = p1;
      }
      lds_barrier();  // P^T and the rescale factors of every wave are in LDS

      // ---- PV: O^T[128 w + c][h] += V^T[c][t] P^T[t][h] ---------------------
      // V^T operand of step i = (ks, cb): two transposing reads
      auto read_v = [&](int i) __attribute__((always_inline)) {
        const uint8_t* vb = stage + (i >> 2) * kGroupBytes + (2 * wave + ((i & 3) >> 1)) * 1024;
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS_AS s16x4*)((LDS_AS uint8_t*)(vb + pv_off[0][i & 1])));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS_AS s16x4*)((LDS_AS uint8_t*)(vb + pv_off[1][i & 1])));
        const bf16x4 a0 = __builtin_bit_cast(bf16x4, v0);
        const bf16x4 a1 = __builtin_bit_cast(bf16x4, v1);
        bf16x8 vf;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vf[j] = a0[j];
          vf[4 + j] = a1[j];
        }
        return vf;
      };
      // every LDS read the rescale does not decide is issued first: the
      // flags, the first V^T operand and the P^T operands of k-step 0
      const u32x4 fl = *reinterpret_cast<const u32x4*>(flags);
      bf16x8 vcur = read_v(0);
      bf16x8 pb[2][4];
      auto read_p = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          pb[ks][hb] = *reinterpret_cast<const LDS_AS bf16x8*>(
              (const LDS_AS uint8_t*)(pbuf + ((hb * 2 + ks) * 64 + lane) * 16));
      };
      read_p(0);
      {
        const unsigned any = __builtin_amdgcn_readfirstlane(fl[0] | fl[1] | fl[2] | fl[3]);
        if (it > 0 && any != 0) {
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) {
            if (__builtin_amdgcn_readfirstlane(fl[hb]) != 0) {
              const float al = alpha_s[32 * hb + l32];
#pragma unroll
              for (int cb = 0; cb < 4; ++cb) scale_agpr16(acc[cb][hb], al);
            }
          }
        }
      }
      // V^T of step i + 1 is read while the MFMAs of step i issue; the P^T
      // operands of k-step 1 at step 4 (no registers to hold both k-steps)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ks = i >> 2, cb = i & 3;
        if (i == 4) read_p(1);
        const bf16x8 vnext = read_v(i < 7 ? i + 1 : i);
#pragma unroll
        for (int hb = 0; hb < 3; ++hb) mfma_agpr<kF16>(acc[cb][hb], vcur, pb[ks][hb]);
        if (i < 7)
          mfma_agpr<kF16>(acc[cb][3], vcur, pb[ks][3]);
        else
          mfma_agpr<kF16, true>(acc[cb][3], vcur, pb[ks][3]);
        vcur = vnext;
      }
    }
    if constexpr (!kC16) vm_wait_n<0>();  // the trailing re-loads have landed
    lds_barrier();  // ring, P^T and flags free
    agpr_settle();

    // ---- epilogue: per-head sums from the QK owners, then O / l ------------
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const bool empty = !(l_tot > 0.f);
    const float lse_v = empty ? -INFINITY : (m_ref + __log2f(l_tot)) * kLn2;
    if (lane_e < 32) stat[32 * wave + lane_e] = empty ? 0.f : 1.f / l_tot;
    lds_barrier();
    float inv[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) inv[hb] = stat[32 * hb + l32_s];
    if (slot < 0) {
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        uint16_t* op = a.o + ((size_t)b * H + 32 * hb + l32_s) * 512 + 128 * wave + 4 * g_s;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const f32x16 x = agpr_read16(acc[cb][hb]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            bf16x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = to16<kF16>(x[4 * q + i] * inv[hb]);
            *reinterpret_cast<bf16x4*>(op + 32 * cb + 8 * q) = v;
          }
        }
      }
      if (lane_e < 32) a.lse[(size_t)b * H + 32 * wave + lane_e] = lse_v;
    } else {
      // Partial of a chunk, merged by the combine kernel after this launch:
      // fp16 with one scale per (head, 128-column block) (scale_exp; half the
      // bytes of fp32: a 64 MB round trip at batch 64 x 4096 tokens becomes
      // 32 MB).  This wave's block of head 32 hb + l32 is spread over lanes
      // l32 and l32 + 32.
      uint16_t* po = reinterpret_cast<uint16_t*>(a.part_o) + (size_t)slot * H * 512;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        f32x16 x[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) x[cb] = agpr_read16(acc[cb][hb]);
        float mx = 0.f;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(x[cb][i]));
        float lo = mx, hi = mx;
        asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(lo), "+v"(hi));
        mx = fmaxf(lo, hi) * inv[hb];
        // mx < 2^e (frexp); the scale 2^(e - 15) maps mx into [2^14, 2^15)
        const int ex = scale_exp(mx);
        const float mult = __builtin_amdgcn_ldexpf(inv[hb], -ex);
        uint16_t* prow = po + (32 * hb + l32_s) * 512 + 128 * wave + 4 * g_s;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f16x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = (_Float16)(x[cb][4 * q + i] * mult);
            *reinterpret_cast<f16x4*>(prow + 32 * cb + 8 * q) = v;
          }
        if (g_s == 0)
          a.part_scale[((size_t)slot * H + 32 * hb + l32_s) * 4 + wave] =
              __builtin_amdgcn_ldexpf(1.f, ex);
      }
      if (lane_e < 32) a.part_lse[(size_t)slot * H + 32 * wave + lane_e] = lse_v;
    }
    lds_barrier();  // stat read by every wave before the next segment rewrites it
  }
}

// ---------------------------------------------------------------------------
// 64-head kernel (16-bit cache).  Split as in the 128-head kernel, only two
// waves would have QK work and PV would fill half of the accumulators.  Here
// the 4 waves (one per SIMD) share each 32-token tile of the same 4-slot LDS
// ring this way:
//   * QK: wave w (head block hw = w & 1, key half kw = w >> 1) runs the
//     k-steps s = 4 gi + 2 kw + v (gi = 0..8, v = 0, 1) of heads
//     32 hw .. 32 hw + 31: 18 of the 36 32x32x16 MFMAs of those heads, with
//     Q^T for its k-steps in 72 VGPRs.  A wave of key half 1 feeds the token
//     rows to the MFMA in the order t ^ 16, so that in both waves of a head
//     block the score registers r = 0..7 of the S^T layout below hold the
//     wave's own token half (tokens 16 kw .. 16 kw + 15) and r = 8..15 the
//     other half;
//   * the two waves of a head block exchange those other halves through LDS
//     and add them: the score of a token is its two key-half partials summed;
//   * a (head, token half) pair is then a "virtual head" with its own online
//     softmax: wave w owns virtual heads 32 w .. 32 w + 31 (heads 32 hw + l,
//     tokens of half kw) and writes their P^T (one 16-token PV k-step) and
//     rescale factors to LDS;
//   * PV by value channels: wave w accumulates O^T for channels 128 w .. + 127
//     of all 128 virtual heads (256 AGPRs; virtual head block vb takes the
//     k-step vb >> 1 only): 16 MFMAs per tile;
//   * the epilogue merges the two virtual heads of every head (the merge of
//     two disjoint token sets, lane by lane, exact up to rounding) into O and
//     LSE, or into the partial of a chunk.
// A tile costs every wave 34 MFMAs.  The loop is the software pipeline of the
// 128-head kernel: QK of tile k + 1 before PV of tile k, the loads of tile
// k + 3 issued one per QK group, and the softmax of tile k + 1 issued
// between PV's MFMAs.
// ---------------------------------------------------------------------------
struct PairShape {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 256;
  static constexpr int kHeads = 64;
  static constexpr int kTile = 32;
  static constexpr int kStages = 4;
  static constexpr int kStageBytes = kTile * kRowBytes;       // 36 KiB bf16 tile
  static constexpr int kPOffset = kStages * kStageBytes;      // P^T [wave][lane] x 16 B
  static constexpr int kXOffset = kPOffset + 4 * 64 * 16;     // score halves [wave][lane] x 32 B
  static constexpr int kAlphaOffset = kXOffset + 4 * 64 * 32;  // [128] rescale factors
  static constexpr int kFlagOffset = kAlphaOffset + 128 * 4;   // [4] rescale flags
  static constexpr int kLdsBytes = kFlagOffset + 16;
  static constexpr int kStatOffset = kXOffset;  // epilogue: (m, l) of the 128 virtual heads
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

template <int KVT, bool CAUSAL>
__global__ void __launch_bounds__(256) mla_decode_pair_kernel(const DecodeArgs a) {
  static_assert(KVT == 0 || KVT == 5, "16-bit caches");
  using S = PairShape;
  constexpr int H = S::kHeads;
  constexpr bool kF16 = KVT == 5;  // fp16 q, cache, P and O
  constexpr int T = S::kTile;
  constexpr int NS = S::kStages;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S::kLdsBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int hw = wave & 1;   // head block: heads 32 hw .. 32 hw + 31
  const int kw = wave >> 1;  // key half of QK, token half after the exchange
  const int page_shift = a.page_shift;
  const int page_mask = (1 << page_shift) - 1;
  const int ld_r_lo = lane >> 3;

  // QK A operand (ds_read_b128): token l32 ^ 16 kw of the tile, k-step
  // s = 4 gi + 2 kw + v, i.e. chunk 2 s + g of the group gi block:
  // qk_w ^ 32 v + 1024 gi from the tile base (the swizzle flips bits 4-6 only)
  uint32_t qk_w;
  {
    const int tr = l32 ^ (16 * kw);
    const int r = tr & 15, half = r >> 3, rr = r & 7;
    const int base = (tr >> 4) * kGroupBytes + half * kHalfGroupBytes + rr * 128;
    qk_w = (uint32_t)(base + (((4 * kw + g) ^ rr ^ half) * 16));
  }
  // PV A operand (ds_read_b64_tr_b16), as in the 128-head kernel
  int pv_off0;
  {
    const int G = lane >> 4, sl = lane & 15;
    const int rr = 4 * (G >> 1) + (sl >> 2);
    const int e = 2 * (G & 1) + ((sl >> 1) & 1);
    pv_off0 = rr * 128 + ((e ^ rr) * 16) + (sl & 1) * 8;
  }

  const int seg_begin = a.one_seg ? (int)blockIdx.x : ld_const(a.worker_ptr + blockIdx.x);
  const int seg_end = a.one_seg ? seg_begin + 1 : ld_const(a.worker_ptr + blockIdx.x + 1);

  for (int si = seg_begin; si < seg_end; ++si) {
    const SegMeta sm = load_seg(a, si);
    const int b = sm.b, t0 = sm.t0, send = sm.send, slot = sm.slot;
    const int kvb = sm.kvb, pbeg = sm.pbeg;
    const int ldev = sm.npg > 0 ? ((sm.npg - 1) << page_shift) + sm.last_len : 0;
    const int t1 = min(send, ldev);
    // scores of this lane's head at or past tlim are masked (end of the
    // chunk; several queries per request: the causal limit of its query)
    const int tlim = CAUSAL ? min(t1, causal_limit<H>(a, b, kvb, 32 * hw + l32, ldev)) : t1;
    const int ntiles = t1 > t0 ? (t1 - t0 + T - 1) / T : 0;

    // Page numbers and direct-to-LDS loads of a tile: wave w loads half group w
    // (group w / 2, rows 8 (w % 2) .. + 7), 9 blocks of 1 KiB; past the last
    // tile the last tile is loaded again, into a slot no one reads, so every
    // vmcnt wait is the same constant.
    const int last_group = t1 > 0 ? ((t1 - 1) >> 4) << 4 : 0;
    struct TileDma {
      const uint8_t* cpage;
      const uint8_t* kpage;
      uint32_t coff, koff;
      uint32_t dst;
    };
    auto pages_of = [&](int k, int (&pg)[2]) __attribute__((always_inline)) {
      const int kc = min(k, ntiles - 1);
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int gs = min(t0 + kc * T + 16 * gi, last_group);
        pg[gi] = ld_const(a.kv_indices + pbeg + (gs >> page_shift));
      }
    };
    auto plan_from = [&](int k, int st, const int (&pg)[2]) __attribute__((always_inline)) {
      const int kc = min(k, ntiles - 1);
      const int my_group = wave >> 1, my_half = wave & 1;
      const int gs = min(t0 + kc * T + 16 * my_group, last_group);
      const int r = my_half * 8 + ld_r_lo;
      const int tok = min(gs + r, t1 - 1);
      const size_t page_row = (size_t)pg[my_group] << page_shift;
      const uint32_t sw = ((lane & 7) ^ swz(r)) * 16;
      TileDma td;
      td.cpage = a.ckv + page_row * 1024;
      td.kpage = a.kpe + page_row * 128;
      td.coff = (tok & page_mask) * 1024 + sw;
      td.koff = (tok & page_mask) * 128 + sw;
      td.dst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(
          LDS_AS uint8_t*)(smem + st * S::kStageBytes + my_group * kGroupBytes +
                           my_half * kHalfGroupBytes));
      return td;
    };
    auto dma_one = [&](const TileDma& td, int u) __attribute__((always_inline)) {
      if (u < 8)
        dma16_s(td.cpage, td.coff + u * 128, td.dst + u * 1024);
      else
        dma16_s(td.kpage, td.koff, td.dst + 8 * 1024);
    };

    // Q^T of heads 32 hw .. 32 hw + 31 for this wave's k-steps: qf[2 gi + v]
    // holds dims 16 s + 8 g .. + 7 of k-step s = 4 gi + 2 kw + v (gi < 8:
    // q_nope, gi = 8: q_pe).  Loaded by assembly before the prologue tiles and
    // waited for alone (loads complete in issue order).
    bf16x8 qf[18];
    {
      const int qhead = 32 * hw + l32;
      const bf16x8* qn =
          reinterpret_cast<const bf16x8*>(a.q_nope + ((size_t)b * H + qhead) * 512) + 4 * kw + g;
      const bf16x8* qp =
          reinterpret_cast<const bf16x8*>(a.q_pe + ((size_t)b * H + qhead) * 64) + 4 * kw + g;
#pragma unroll
      for (int j = 0; j < 18; ++j)
        qf[j] = load16_untracked(j < 16 ? qn + 8 * (j >> 1) + 2 * (j & 1) : qp + 2 * (j & 1));
    }
    if (ntiles > 0) {
      int pg[2];
      pages_of(0, pg);
#pragma unroll
      for (int k = 0; k < NS - 1; ++k) {
        int pn[2];
        pages_of(k + 1, pn);
        const TileDma td = plan_from(k, k, pg);
#pragma unroll
        for (int u = 0; u < 9; ++u) dma_one(td, u);
        pg[0] = pn[0];
        pg[1] = pn[1];
      }
      vm_wait_n<9 * (NS - 1)>();
    } else {
      vm_wait_n<0>();  // no tile: nothing may stay in flight
    }

    f32x16 acc[4][4];  // O^T [channel block cb][virtual head block vb]
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int vb = 0; vb < 4; ++vb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[cb][vb][i] = 0.f;
    float m_ref = -INFINITY;  // virtual head 32 w + l32, log2 domain
    float l_run = 0.f;        // this lane's 8 tokens of it

    f32x16 sacc;           // partial, then (r < 8) full scores of the tile softmaxed next
    bf16x8 pq = {};        // P^T of the last softmaxed tile (PV B operand)
    float alpha_q = 1.f;   // its rescale factor (1: none)
    unsigned resc_q = 0;   // wave-uniform: its softmax moved the reference max
    float tmax = -INFINITY, psum = 0.f, m_use = 0.f, m_next = 0.f;
    f32x4 xin0 = {}, xin1 = {};  // the other key half's partial of this wave's tokens
    int ts_next = t0;            // first token of the tile softmaxed next
    uint32_t small_base = (uint32_t)(uintptr_t)(LDS_AS uint8_t*)(smem + S::kPOffset);
    asm volatile("" : "+s"(small_base));
    constexpr uint32_t kX = S::kXOffset - S::kPOffset, kAl = S::kAlphaOffset - S::kPOffset,
                       kFl = S::kFlagOffset - S::kPOffset;
    const uint32_t p_lane = small_base + lane * 16;       // P^T [wave][lane]
    const uint32_t x_lane = small_base + kX + lane * 32;  // score halves [wave][lane]
    const uint32_t a_lane = small_base + kAl + l32 * 4;   // alpha [virtual head]
    auto lds_at = [](uint32_t addr) __attribute__((always_inline)) {
      return (LDS_AS uint8_t*)(uintptr_t)addr;
    };

    // QK of the tile at `stage`: 9 groups of 2 k-steps, operands read three
    // groups ahead, the loads of a later tile one per group.
    auto qk_tile = [&](const uint8_t* stage, bool dma_on, const TileDma& tdma)
        __attribute__((always_inline)) {
      uint32_t kbase = (uint32_t)(uintptr_t)(LDS_AS uint8_t*)stage + qk_w;
      asm volatile("" : "+v"(kbase));
      auto read_k = [&](int gi, bf16x8 (&kf)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int v = 0; v < 2; ++v)
          kf[v] = *reinterpret_cast<const LDS_AS bf16x8*>(lds_at((kbase ^ (32u * v)) + gi * 1024));
      };
      bf16x8 kq[4][2];
      read_k(0, kq[0]);
      read_k(1, kq[1]);
      read_k(2, kq[2]);
#pragma unroll
      for (int gi = 0; gi < 9; ++gi) {
        if (gi + 3 < 9) read_k(gi + 3, kq[(gi + 3) % 4]);
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          const int j = 2 * gi + v;
          if (j == 0)
            mfma_vgpr<kF16, true, false>(sacc, kq[gi % 4][v], qf[j]);
          else if (j == 17)
            mfma_vgpr<kF16, false, true>(sacc, kq[gi % 4][v], qf[j]);
          else
            mfma_vgpr<kF16, false, false>(sacc, kq[gi % 4][v], qf[j]);
        }
        if (dma_on) dma_one(tdma, gi);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // the other token half of the partial scores, for the other wave of the head block
    auto send_half = [&]() __attribute__((always_inline)) {
      const uint32_t xo = x_lane + 2048u * wave;
      *reinterpret_cast<LDS_AS f32x4*>(lds_at(xo)) = f32x4{sacc[8], sacc[9], sacc[10], sacc[11]};
      *reinterpret_cast<LDS_AS f32x4*>(lds_at(xo + 16)) =
          f32x4{sacc[12], sacc[13], sacc[14], sacc[15]};
    };
    auto recv_half = [&]() __attribute__((always_inline)) {
      const uint32_t xi = x_lane + 2048u * (wave ^ 2);
      xin0 = *reinterpret_cast<const LDS_AS f32x4*>(lds_at(xi));
      xin1 = *reinterpret_cast<const LDS_AS f32x4*>(lds_at(xi + 16));
    };

    // Online softmax of the virtual head's 16 scores (this lane's 8 in sacc[0..7]
    // once the other key half is added; the lane l ^ 32 holds the other 8),
    // in slots issued one behind each of PV's 16 MFMAs.  0: the other key
    // half added; 1: scores past the limit set to -inf; 2-3: the lane's max;
    // 4: with lane l ^ 32, scaled (s = sm_scale log2 e > 0 commutes with the
    // max); 5-7: the rescale decision (alpha = 1 unless the wave moves its
    // reference max; a head with no visible token keeps alpha = 1) and the
    // new reference; 8-11: the probabilities exp2(fma(raw, s, -m)), summed in
    // pairs in order; 12: the row sum.
    auto sm_slot = [&](int j) __attribute__((always_inline)) {
      if (j == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sacc[i] += xin0[i];
          sacc[4 + i] += xin1[i];
        }
      } else if (j == 1) {
        if (__builtin_amdgcn_ballot_w64(ts_next + T > tlim) != 0) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int tok = ts_next + 16 * kw + 8 * (i >> 2) + 4 * g + (i & 3);
            sacc[i] = tok < tlim ? sacc[i] : -INFINITY;
          }
        }
      } else if (j == 2) {
        tmax = fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3]));
      } else if (j == 3) {
        tmax = fmaxf(tmax, fmaxf(fmaxf(sacc[4], sacc[5]), fmaxf(sacc[6], sacc[7])));
      } else if (j == 4) {
        float lo = tmax, hi = tmax;
        asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1"
                     : "+v"(lo), "+v"(hi));
        tmax = fmaxf(lo, hi) * a.scale_log2;
      } else if (j == 5) {
        resc_q = __builtin_amdgcn_ballot_w64(tmax > m_ref + kRescaleSlack) != 0 ? 1u : 0u;
        m_next = resc_q ? fmaxf(m_ref, tmax) : m_ref;
      } else if (j == 6) {
        alpha_q = (resc_q && m_next != -INFINITY) ? __builtin_amdgcn_exp2f(m_ref - m_next) : 1.f;
        m_ref = m_next;
        m_use = m_ref == -INFINITY ? 0.f : -m_ref;
      } else if (j == 7) {
        l_run *= alpha_q;
        psum = 0.f;
      } else if (j < 12) {
        const int k = 2 * (j - 8);
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[k], a.scale_log2, m_use));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[k + 1], a.scale_log2, m_use));
        psum += e0 + e1;
        pq[k] = to16<kF16>(e0);
        pq[k + 1] = to16<kF16>(e1);
      } else if (j == 12) {
        l_run += psum;
      }
    };

    // PV of the tile at `stage` (P^T of every wave and the rescale flags are
    // in LDS); WITH_SM: the softmax slots of the next tile behind its MFMAs.
    auto pv_tile = [&](auto with_sm, const uint8_t* stage) __attribute__((always_inline)) {
      constexpr bool kSm = decltype(with_sm)::value;
      uint32_t vt = (uint32_t)(uintptr_t)(LDS_AS uint8_t*)stage + 2048 * wave + pv_off0;
      asm volatile("" : "+v"(vt));
      uint32_t vx[2][2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c1 = 0; c1 < 2; ++c1) vx[h][c1] = vt ^ (16u * h + 64u * c1);
      // V^T operand of step i = 4 ks + cb: channels 32 cb .. + 31 of this wave's
      // 128, tokens 16 ks .. 16 ks + 15
      auto read_v = [&](int i) __attribute__((always_inline)) {
        const uint32_t off = (i >> 2) * kGroupBytes + ((i & 3) >> 1) * 1024;
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS_AS s16x4*)lds_at(vx[0][i & 1] + off));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS_AS s16x4*)lds_at(vx[1][i & 1] + off + kHalfGroupBytes));
        const bf16x4 a0 = __builtin_bit_cast(bf16x4, v0);
        const bf16x4 a1 = __builtin_bit_cast(bf16x4, v1);
        bf16x8 vf;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          vf[jj] = a0[jj];
          vf[4 + jj] = a1[jj];
        }
        return vf;
      };
      const u32x4 fl = *reinterpret_cast<const LDS_AS u32x4*>(lds_at(small_base + kFl));
      bf16x8 vcur = read_v(0);
      bf16x8 pb[4];
#pragma unroll
      for (int vb = 0; vb < 4; ++vb)
        pb[vb] = *reinterpret_cast<const LDS_AS bf16x8*>(lds_at(p_lane + vb * 1024));
      if constexpr (kSm) recv_half();
      {
        const unsigned any = __builtin_amdgcn_readfirstlane(fl[0] | fl[1] | fl[2] | fl[3]);
        if (any != 0) {
#pragma unroll
          for (int vb = 0; vb < 4; ++vb) {
            if (__builtin_amdgcn_readfirstlane(fl[vb]) != 0) {
              const float al =
                  *reinterpret_cast<const LDS_AS float*>(lds_at(a_lane + 128 * vb));
#pragma unroll
              for (int cb = 0; cb < 4; ++cb) scale_agpr16(acc[cb][vb], al);
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ks = i >> 2, cb = i & 3;
        const bf16x8 vnext = read_v(i < 7 ? i + 1 : i);
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          const int vb = 2 * ks + v;
          if (i == 7 && v == 1)
            mfma_agpr<kF16, true>(acc[cb][vb], vcur, pb[vb]);
          else
            mfma_agpr<kF16>(acc[cb][vb], vcur, pb[vb]);
          if constexpr (kSm) {
            __builtin_amdgcn_sched_barrier(0);
            sm_slot(2 * i + v);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        vcur = vnext;
      }
    };

    if (ntiles > 0) {
      // tile 0 landed (tiles 1 and 2 may be in flight): its QK, the exchange,
      // its softmax
      vm_wait_n<18>();
      lds_barrier();
      qk_tile(smem, false, TileDma{});
      send_half();
      lds_barrier();
      recv_half();
#pragma unroll
      for (int j = 0; j < 16; ++j) sm_slot(j);
    }
    auto iteration = [&](auto with_sm, int it) __attribute__((always_inline)) {
      constexpr bool nxt = decltype(with_sm)::value;  // a tile it + 1 exists
      // tile it + 1 landed (tile it + 2 may be in flight); the page numbers of
      // tile it + 3 are loaded before the waits that cover their latency
      int pg3[2] = {0, 0};
      if constexpr (nxt) {
        pages_of(it + 3, pg3);
        vm_wait_n<9>();
      }
      lds_barrier();  // PV of tile it - 1 and the reads of the exchange done everywhere
      *reinterpret_cast<LDS_AS bf16x8*>(lds_at(p_lane + wave * 1024)) = pq;
      if (resc_q && lane < 32)
        *reinterpret_cast<LDS_AS float*>(lds_at(a_lane + 128 * wave)) = alpha_q;
      // (tile 0: the accumulators are still zero, nothing to rescale)
      if (lane == 0)
        *reinterpret_cast<LDS_AS unsigned*>(lds_at(small_base + kFl + 4 * wave)) =
            it > 0 ? resc_q : 0u;
      if constexpr (nxt) {
        const TileDma tdma = plan_from(it + 3, (it + 3) % NS, pg3);
        qk_tile(smem + ((it + 1) % NS) * S::kStageBytes, true, tdma);
        send_half();
        ts_next = t0 + (it + 1) * T;
      }
      lds_barrier();  // P^T, rescale and score halves of every wave
      pv_tile(with_sm, smem + (it % NS) * S::kStageBytes);
    };
    for (int it = 0; it + 1 < ntiles; ++it) iteration(std::true_type{}, it);
    if (ntiles > 0) iteration(std::false_type{}, ntiles - 1);
    vm_wait_n<0>();  // the trailing reloads have landed (their slots are reused)
    lds_barrier();   // ring, P^T, flags and score halves free
    agpr_settle();

    // ---- epilogue: merge the two token halves of every head ------------------
    // stat[0][v] = m, stat[1][v] = l of virtual head v (log2 domain)
    float* stat = reinterpret_cast<float*>(smem + S::kStatOffset);
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (lane < 32) {
      stat[32 * wave + l32] = m_ref;
      stat[128 + 32 * wave + l32] = l_tot;
    }
    lds_barrier();
    // head 32 hb + l32 = virtual heads hb (tokens of half 0) and hb + 2 (half 1),
    // whose accumulators A0, A1 are unnormalised (sums of 2^(x - m) v):
    // O = (2^(m0 - M) A0 + 2^(m1 - M) A1) / L, L = l0 2^(m0 - M) + l1 2^(m1 - M)
    float c0[2], c1[2], lse_h[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const float m0 = stat[32 * hb + l32], m1 = stat[32 * (hb + 2) + l32];
      const float l0 = stat[128 + 32 * hb + l32], l1 = stat[128 + 32 * (hb + 2) + l32];
      const float M = fmaxf(m0, m1);
      // a half with no visible token has l = 0 (and m = -inf): weight 0
      const float e0 = l0 > 0.f ? __builtin_amdgcn_exp2f(m0 - M) : 0.f;
      const float e1 = l1 > 0.f ? __builtin_amdgcn_exp2f(m1 - M) : 0.f;
      const float L = l0 * e0 + l1 * e1;
      const bool empty = !(L > 0.f);
      const float inv = empty ? 0.f : 1.f / L;
      c0[hb] = e0 * inv;
      c1[hb] = e1 * inv;
      lse_h[hb] = empty ? -INFINITY : (M + __log2f(L)) * kLn2;
    }
    const float lse_v = wave == 0 ? lse_h[0] : lse_h[1];  // waves 0 and 1 write heads 32 w + l32
    if (slot < 0) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        uint16_t* op = a.o + ((size_t)b * H + 32 * hb + l32) * 512 + 128 * wave + 4 * g;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const f32x16 x0 = agpr_read16(acc[cb][hb]), x1 = agpr_read16(acc[cb][hb + 2]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            bf16x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              v[i] = to16<kF16>(x0[4 * q + i] * c0[hb] + x1[4 * q + i] * c1[hb]);
            *reinterpret_cast<bf16x4*>(op + 32 * cb + 8 * q) = v;
          }
        }
      }
      if (wave < 2 && lane < 32) a.lse[(size_t)b * H + 32 * wave + l32] = lse_v;
    } else {
      // partial of a chunk, merged by the combine kernel after this launch:
      // fp16 with one scale per (head, 128-column block) (scale_exp); this
      // wave's block of head 32 hb + l32 is spread over lanes l32, l32 + 32
      uint16_t* po = reinterpret_cast<uint16_t*>(a.part_o) + (size_t)slot * H * 512;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        // the merged values are formed twice (for the block max, then stored)
        // rather than held in 64 more registers; the accumulators are read out
        // of their AGPRs a block at a time (agpr_read16)
        float mx = 0.f;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const f32x16 x0 = agpr_read16(acc[cb][hb]), x1 = agpr_read16(acc[cb][hb + 2]);
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(x0[i] * c0[hb] + x1[i] * c1[hb]));
        }
        float lo = mx, hi = mx;
        asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(lo), "+v"(hi));
        const int ex = scale_exp(fmaxf(lo, hi));
        const float d0 = __builtin_amdgcn_ldexpf(c0[hb], -ex), d1 = __builtin_amdgcn_ldexpf(c1[hb], -ex);
        uint16_t* prow = po + (32 * hb + l32) * 512 + 128 * wave + 4 * g;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const f32x16 x0 = agpr_read16(acc[cb][hb]), x1 = agpr_read16(acc[cb][hb + 2]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f16x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = (_Float16)(x0[4 * q + i] * d0 + x1[4 * q + i] * d1);
            *reinterpret_cast<f16x4*>(prow + 32 * cb + 8 * q) = v;
          }
        }
        if (g == 0)
          a.part_scale[((size_t)slot * H + 32 * hb + l32) * 4 + wave] = __builtin_amdgcn_ldexpf(1.f, ex);
      }
      if (wave < 2 && lane < 32) a.part_lse[(size_t)slot * H + 32 * wave + l32] = lse_v;
    }
    lds_barrier();  // stat read by every wave before the next segment reuses the area
  }
}

// ---------------------------------------------------------------------------
// Merge of split requests (a launch after the decode kernel), for requests cut
// into at most kCombineFewMax chunks (launch_combine sends more to the kernel
// below): one thread per (split request, head, 8 columns), so the merge runs
// on the whole GPU.  The thread issues the loads of all its partials' LSEs and
// O slices at once (one memory round trip), then LSE = M + ln sum_i
// exp(LSE_i - M) and O = sum_i exp(LSE_i - LSE) O_i, summed in chunk order
// i = 0, 1, ...  The 64 threads of a wave share one head, so its partial LSEs
// are one cache line.
// ---------------------------------------------------------------------------
template <int H>
__global__ void __launch_bounds__(256) mla_combine_kernel(const DecodeArgs a) {
  constexpr int kBlocksPerReq = H * 64 / 256;
  constexpr int K = kCombineFewMax;
  const int req = blockIdx.x / kBlocksPerReq;
  const int e = (blockIdx.x % kBlocksPerReq) * 256 + threadIdx.x;
  const int hd = e >> 6;
  const int col = (e & 63) * 8;
  const int* cl = reinterpret_cast<const int*>(a.clist) + req * 4;
  const int b = ld_const(cl + 0);
  const int slot0 = ld_const(cl + 1);
  const int n = min(ld_const(cl + 2), K);
  const float* pl = a.part_lse + (size_t)slot0 * H + hd;
  // fp16 partials and the scale of their 128-column block
  const uint16_t* ph = reinterpret_cast<const uint16_t*>(a.part_o) + ((size_t)slot0 * H + hd) * 512 + col;
  const float* ps = a.part_scale + ((size_t)slot0 * H + hd) * 4 + (col >> 7);
  float lv[K], sv[K];
  f16x8 xh[K];
#pragma unroll
  for (int v = 0; v < K; ++v) {
    const int i = min(v, n - 1);
    lv[v] = pl[(size_t)i * H];
    xh[v] = *reinterpret_cast<const f16x8*>(ph + (size_t)i * H * 512);
    sv[v] = ps[(size_t)i * H * 4];
  }
  float M = -INFINITY;
#pragma unroll
  for (int v = 0; v < K; ++v)
    if (v < n) M = fmaxf(M, lv[v]);
  const float Mu = M == -INFINITY ? 0.f : M;
  float sum = 0.f;
#pragma unroll
  for (int v = 0; v < K; ++v)
    if (v < n) sum += __expf(lv[v] - Mu);
  const bool empty = !(sum > 0.f);
  const float lse_v = empty ? -INFINITY : Mu + __logf(sum);
  float o8[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o8[j] = 0.f;
#pragma unroll
  for (int v = 0; v < K; ++v) {
    if (v < n) {
      const float ws = empty ? 0.f : __expf(lv[v] - lse_v) * sv[v];
#pragma unroll
      for (int j = 0; j < 8; ++j) o8[j] += ws * (float)xh[v][j];
    }
  }
  bf16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = a.o_fp16 ? to16<true>(o8[j]) : to16<false>(o8[j]);
  *reinterpret_cast<bf16x8*>(a.o + ((size_t)b * H + hd) * 512 + col) = v;
  if (col == 0) a.lse[(size_t)b * H + hd] = lse_v;
}

// ---------------------------------------------------------------------------
// Merge of split requests cut into many chunks (more than kCombineFewMax;
// up to 256), as long contexts at small batch are.  One workgroup per (split
// request, head, column chunk), so the n partials of a request are read by
// many workgroups at once rather than by one.  L partial lanes per 8 columns;
// the workgroup covers 8 * 256 / L columns: L = 4 (the whole 512-column row,
// each wave taking every fourth partial) when the (request, head) pairs alone
// give enough workgroups, else L = 16 (128 columns) up to 16 chunks and 32 (64
// columns) beyond.  Thread (q, j) (q = tid % (256 / L), j = tid / (256 / L))
// sums w_i O_i over its 8 columns for partials i = j, j + L, ..., kBatch
// partials' loads in flight and the next batch requested before the current
// one is added.  Its first loads are issued before the LSE reduction, which
// they do not depend on: the workgroup reads the head's n partial LSEs (one
// per thread), reduces them to LSE = M + ln sum_i exp(LSE_i - M) and keeps
// w_i = exp(LSE_i - LSE) in LDS.  The L sums per 8 columns are added by
// xor-shuffles within a wave and then wave by wave.  Every reduction has a
// fixed order, so reruns are bit-identical.
// ---------------------------------------------------------------------------
template <int H, bool F16, int L>
__global__ void __launch_bounds__(256) mla_combine_many_kernel(const DecodeArgs a) {
  constexpr int kItems = 256 / L;           // 8-column items per workgroup
  constexpr int kChunks = 512 / (8 * kItems);
  constexpr int kBatch = L == 4 ? 8 : 4;    // partials in flight per thread
  __shared__ float s_w[256];
  __shared__ float s_red[2][4];
  __shared__ f32x4 s_o[4][kItems][2];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int req = blockIdx.x / (H * kChunks);
  const int hd = (blockIdx.x / kChunks) % H;
  const int ch = blockIdx.x % kChunks;
  const int* cl = reinterpret_cast<const int*>(a.clist) + req * 4;
  const int b = ld_const(cl + 0);
  const int slot0 = ld_const(cl + 1);
  const int n = ld_const(cl + 2);

  const int q = tid % kItems, j = tid / kItems;
  const int col = ch * (8 * kItems) + q * 8;
  // fp16 partials and the scale of their 128-column block
  const uint16_t* ph = reinterpret_cast<const uint16_t*>(a.part_o) + ((size_t)slot0 * H + hd) * 512 + col;
  const float* ps = a.part_scale + ((size_t)slot0 * H + hd) * 4 + (col >> 7);
  // two batches of registers: the next batch is requested before the current
  // one is added
  f16x8 xa[kBatch], xb[kBatch];
  float sa[kBatch], sb[kBatch];
  auto load_batch = [&](int i0, f16x8 (&xh)[kBatch], float (&sv)[kBatch])
      __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = min(i0 + u * L, n - 1);
      xh[u] = *reinterpret_cast<const f16x8*>(ph + (size_t)i * H * 512);
      sv[u] = ps[(size_t)i * H * 4];
    }
  };
  load_batch(j, xa, sa);  // in flight through the LSE reduction

  // ---- LSE over the n partials ---------------------------------------------
  const float* pl = a.part_lse + (size_t)slot0 * H + hd;
  const float v = tid < n ? pl[(size_t)tid * H] : -INFINITY;
  float mx = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) s_red[0][wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
  const float Mu = M == -INFINITY ? 0.f : M;
  float e = tid < n ? __expf(v - Mu) : 0.f;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) e += __shfl_xor(e, o);
  if (lane == 0) s_red[1][wave] = e;
  __syncthreads();
  const float sum = (s_red[1][0] + s_red[1][1]) + (s_red[1][2] + s_red[1][3]);
  const bool empty = !(sum > 0.f);
  const float lse_v = empty ? -INFINITY : Mu + __logf(sum);
  if (tid < n) s_w[tid] = empty ? 0.f : __expf(v - lse_v);
  __syncthreads();

  // ---- O = sum_i w_i O_i over this thread's partials -----------------------
  float o8[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) o8[c] = 0.f;
  auto add_batch = [&](int i0, const f16x8 (&xh)[kBatch], const float (&sv)[kBatch])
      __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + u * L;
      if (i < n) {
        const float ws = s_w[i] * sv[u];
#pragma unroll
        for (int c = 0; c < 8; ++c) o8[c] += ws * (float)xh[u][c];
      }
    }
  };
  constexpr int kStep = kBatch * L;  // partials per batch of the workgroup
  for (int i0 = j; i0 < n; i0 += 2 * kStep) {
    if (i0 + kStep < n) load_batch(i0 + kStep, xb, sb);
    add_batch(i0, xa, sa);
    if (i0 + kStep >= n) break;
    if (i0 + 2 * kStep < n) load_batch(i0 + 2 * kStep, xa, sa);
    add_batch(i0 + kStep, xb, sb);
  }
  // a wave holds lanes j = (64 / kItems) wave + 0 .. 64 / kItems - 1 of every
  // item: lanes that differ in the bits above log2(kItems)
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int o = kItems; o < 64; o <<= 1) o8[c] += __shfl_xor(o8[c], o);
  if (lane < kItems) {
    s_o[wave][lane][0] = f32x4{o8[0], o8[1], o8[2], o8[3]};
    s_o[wave][lane][1] = f32x4{o8[4], o8[5], o8[6], o8[7]};
  }
  __syncthreads();
  if (tid < kItems) {
    bf16x8 out;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const f32x4 r = (s_o[0][tid][h2] + s_o[1][tid][h2]) + (s_o[2][tid][h2] + s_o[3][tid][h2]);
#pragma unroll
      for (int c = 0; c < 4; ++c) out[4 * h2 + c] = to16<F16>(r[c]);
    }
    *reinterpret_cast<bf16x8*>(a.o + ((size_t)b * H + hd) * 512 + ch * (8 * kItems) + tid * 8) =
        out;
  }
  if (tid == 0 && ch == 0) a.lse[(size_t)b * H + hd] = lse_v;
}

// ---------------------------------------------------------------- launchers
template <int HG, int HB, int TS, int MB, int NSTAGE>
static hipError_t launch_decode_cfg(const DecodeArgs& a, int grid, hipStream_t stream,
                                    const LaunchEvents& ev) {
  using S = RingShape<HG, HB, TS, MB, NSTAGE>;
  hipExtLaunchKernelGGL((mla_decode_ring_kernel<HG, HB, TS, MB, NSTAGE>), dim3(grid), dim3(S::kThreads), 0, stream, ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

template <int KVT>
static hipError_t launch_wide(const DecodeArgs& a, int grid, hipStream_t stream,
                              const LaunchEvents& ev) {
  if (a.qo_len > 1)
    hipExtLaunchKernelGGL((mla_decode_wide_kernel<KVT, true>), dim3(grid), dim3(WideShape<KVT>::kThreads), 0, stream, ev.start, ev.stop, 0, a);
  else
    hipExtLaunchKernelGGL((mla_decode_wide_kernel<KVT, false>), dim3(grid), dim3(WideShape<KVT>::kThreads), 0, stream, ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

template <int KVT>
static hipError_t launch_pair(const DecodeArgs& a, int grid, hipStream_t stream,
                              const LaunchEvents& ev) {
  if (a.qo_len > 1)
    hipExtLaunchKernelGGL((mla_decode_pair_kernel<KVT, true>), dim3(grid), dim3(PairShape::kThreads), 0, stream, ev.start, ev.stop, 0, a);
  else
    hipExtLaunchKernelGGL((mla_decode_pair_kernel<KVT, false>), dim3(grid), dim3(PairShape::kThreads), 0, stream, ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

static DecodeConfig pair_config() {
  return DecodeConfig{PairShape::kWaves, PairShape::kTile, PairShape::kLdsBytes};
}

template <int KVT>
static int pair_occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&mla_decode_pair_kernel<KVT, false>),
          PairShape::kThreads, 0) != hipSuccess ||
      n < 1)
    n = 1;
  return n;
}

template <int KVT>
static DecodeConfig wide_config() {
  return DecodeConfig{WideShape<KVT>::kWaves, WideShape<KVT>::kTile, WideShape<KVT>::kLdsBytes};
}

template <int KVT>
static int wide_occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&mla_decode_wide_kernel<KVT, false>),
          WideShape<KVT>::kThreads, 0) != hipSuccess ||
      n < 1)
    n = 1;
  return n;
}

template <int HG, int HB, int TS, int MB, int NSTAGE>
static DecodeConfig config_of() {
  using S = RingShape<HG, HB, TS, MB, NSTAGE>;
  return DecodeConfig{S::kWaves, S::kTile, S::kLdsBytes};
}

template <int HB, int KVT, int NB, int NW>
static hipError_t launch_stream_cfg(const DecodeArgs& a, int grid, hipStream_t stream,
                                    const LaunchEvents& ev) {
  using S = StreamShape<HB, KVT, NB, NW>;
  hipExtLaunchKernelGGL((mla_decode_stream_kernel<HB, KVT, NB, NW>), dim3(grid), dim3(S::kThreads), 0, stream, ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

template <int HB, int KVT, int NB, int NW>
static DecodeConfig stream_config_of() {
  using S = StreamShape<HB, KVT, NB, NW>;
  return DecodeConfig{S::kWaves, 16, S::kLdsBytes};
}

template <int HB, int KVT, int NB, int NW>
static int stream_occupancy_of() {
  using S = StreamShape<HB, KVT, NB, NW>;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&mla_decode_stream_kernel<HB, KVT, NB, NW>), S::kThreads,
          0) != hipSuccess ||
      n < 1)
    n = (160 * 1024) / S::kLdsBytes;
  return n < 1 ? 1 : n;
}

template <int HG, int HB, int TS, int MB, int NSTAGE>
static int occupancy_of() {
  using S = RingShape<HG, HB, TS, MB, NSTAGE>;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&mla_decode_ring_kernel<HG, HB, TS, MB, NSTAGE>),
          S::kThreads, 0) != hipSuccess ||
      n < 1)
    n = (160 * 1024) / S::kLdsBytes;
  return n < 1 ? 1 : n;
}

// One switch describes the kernel chosen for (heads per workgroup, cache
// dtype); `op` is 0 = config, 1 = occupancy, 2 = launch.
static int dispatch(int heads, int kv_dtype, int op, DecodeConfig* cfg, const DecodeArgs* a,
                    int grid, hipStream_t stream, hipError_t* err, const LaunchEvents& ev = {}) {
#define MLA_STREAM(...)                                                     \
  do {                                                                      \
    if (op == 0) *cfg = stream_config_of<__VA_ARGS__>();                    \
    if (op == 1) return stream_occupancy_of<__VA_ARGS__>();                 \
    if (op == 2) *err = launch_stream_cfg<__VA_ARGS__>(*a, grid, stream, ev);   \
    return 1;                                                               \
  } while (0)
#define MLA_WIDE(K)                                                         \
  do {                                                                      \
    if (op == 0) *cfg = wide_config<K>();                                   \
    if (op == 1) return wide_occupancy<K>();                                \
    if (op == 2) *err = launch_wide<K>(*a, grid, stream, ev);                   \
    return 1;                                                               \
  } while (0)
#define MLA_PAIR(K)                                                         \
  do {                                                                      \
    if (op == 0) *cfg = pair_config();                                      \
    if (op == 1) return pair_occupancy<K>();                                \
    if (op == 2) *err = launch_pair<K>(*a, grid, stream, ev);                   \
    return 1;                                                               \
  } while (0)
#define MLA_RING(...)                                                       \
  do {                                                                      \
    if (op == 0) *cfg = config_of<__VA_ARGS__>();                           \
    if (op == 1) return occupancy_of<__VA_ARGS__>();                        \
    if (op == 2) *err = launch_decode_cfg<__VA_ARGS__>(*a, grid, stream, ev);   \
    return 1;                                                               \
  } while (0)
  // ring-kernel shapes: <16-head blocks, blocks per wave, token-split waves,
  // row groups per wave per tile, ring stages>; stream-kernel shapes: <head
  // blocks, cache layout, groups staged in registers per wave, waves> (int8:
  // eight waves, whose second wave per SIMD hides more of the conversion)
  if (kv_dtype == 0) {
    switch (heads) {
      case 16: MLA_STREAM(1, 0, 2, 4);
      case 32: MLA_RING(2, 1, 2, 1, 4);
      case 64: MLA_PAIR(0);
      case 128: MLA_WIDE(0);
      default: return 0;
    }
  }
  if (kv_dtype == 1) {
    switch (heads) {
      case 16: MLA_STREAM(1, 1, 2, 4);
      case 128: MLA_WIDE(1);
      default: return 0;
    }
  }
  if (kv_dtype == 2) {
    switch (heads) {
      case 16: MLA_STREAM(1, 2, 1, 8);
      case 128: MLA_WIDE(2);
      default: return 0;
    }
  }
  if (kv_dtype == 3) {
    switch (heads) {
      case 16: MLA_STREAM(1, 3, 2, 4);
      case 128: MLA_WIDE(3);
      default: return 0;
    }
  }
  if (kv_dtype == 4) {
    switch (heads) {
      case 16: MLA_STREAM(1, 4, 2, 4);
      case 128: MLA_WIDE(4);
      default: return 0;
    }
  }
  if (kv_dtype == 5) {  // fp16: 32- and 64-wide requests run as 16-wide rows
    switch (heads) {
      case 16: MLA_STREAM(1, 5, 2, 4);
      case 64: MLA_PAIR(5);
      case 128: MLA_WIDE(5);
      default: return 0;
    }
  }
  return 0;
#undef MLA_STREAM
#undef MLA_WIDE
#undef MLA_PAIR
#undef MLA_RING
}

template <int H>
static hipError_t launch_combine_h(const DecodeArgs& a, int ncomb, int max_splits,
                                   hipStream_t stream) {
  if (max_splits > kCombineFewMax) {
    // whole rows (4 partial lanes) when the (request, head) pairs fill a
    // device's CUs; else 16 partial lanes (4 column chunks of a head) up to 16
    // chunks, 32 (8) beyond
    if ((long)ncomb * H >= 256) {
      const dim3 grid(ncomb * H);
      if (a.o_fp16)
        hipLaunchKernelGGL((mla_combine_many_kernel<H, true, 4>), grid, dim3(256), 0, stream, a);
      else
        hipLaunchKernelGGL((mla_combine_many_kernel<H, false, 4>), grid, dim3(256), 0, stream, a);
    } else if (max_splits <= 16) {
      const dim3 grid(ncomb * H * 4);
      if (a.o_fp16)
        hipLaunchKernelGGL((mla_combine_many_kernel<H, true, 16>), grid, dim3(256), 0, stream, a);
      else
        hipLaunchKernelGGL((mla_combine_many_kernel<H, false, 16>), grid, dim3(256), 0, stream, a);
    } else {
      const dim3 grid(ncomb * H * 8);
      if (a.o_fp16)
        hipLaunchKernelGGL((mla_combine_many_kernel<H, true, 32>), grid, dim3(256), 0, stream, a);
      else
        hipLaunchKernelGGL((mla_combine_many_kernel<H, false, 32>), grid, dim3(256), 0, stream, a);
    }
  } else {
    hipLaunchKernelGGL(mla_combine_kernel<H>, dim3(ncomb * (H / 4)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_combine(int heads, const DecodeArgs& a, int ncomb, int max_splits,
                          hipStream_t stream) {
  if (ncomb <= 0) return hipSuccess;
  if (max_splits > 256) return hipErrorInvalidValue;
  switch (heads) {
    case 16: return launch_combine_h<16>(a, ncomb, max_splits, stream);
    case 32: return launch_combine_h<32>(a, ncomb, max_splits, stream);
    case 64: return launch_combine_h<64>(a, ncomb, max_splits, stream);
    case 128: return launch_combine_h<128>(a, ncomb, max_splits, stream);
    default: return hipErrorInvalidValue;
  }
}

int decode_config(int heads, int kv_dtype, DecodeConfig* cfg) {
  return dispatch(heads, kv_dtype, 0, cfg, nullptr, 0, nullptr, nullptr) ? 0 : -1;
}

int decode_blocks_per_cu(int heads, int kv_dtype) {
  const int n = dispatch(heads, kv_dtype, 1, nullptr, nullptr, 0, nullptr, nullptr);
  return n < 1 ? 1 : n;
}

hipError_t launch_decode(int heads, int kv_dtype, const DecodeArgs& a, int grid,
                         hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  hipError_t err = hipErrorInvalidValue;
  if (!dispatch(heads, kv_dtype, 2, nullptr, &a, grid, stream, &err, LaunchEvents{start, stop}))
    return hipErrorInvalidValue;
  return err;
}

}  // namespace mla_gpu
