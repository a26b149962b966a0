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
// directly) or a chunk of one (normalised fp32 partial O and its LSE written to
// a partial slot).  The combine kernel merges the chunks of a request in
// chunk order, weighting each by exp(LSE_i - LSE), which is deterministic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace mla_gpu {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

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
template <int ITEMS>
__device__ __forceinline__ void wait_tile(int later) {
  static_assert(3 * ITEMS < 64, "vmcnt range");
  switch (later) {
    case 0: vm_wait_n<0>(); break;
    case 1: vm_wait_n<ITEMS>(); break;
    case 2: vm_wait_n<2 * ITEMS>(); break;
    default: vm_wait_n<3 * ITEMS>(); break;
  }
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

template <int HG, int TS, int MB, int NSTAGE>
struct DecodeShape {
  static constexpr int kPvBatch = HG * TS > 4 ? 2 : 8;  // PV operand reads in flight
  static constexpr int kWaves = HG * TS;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kHeads = 16 * HG;
  static constexpr int kTile = TS * MB * 16;
  static constexpr int kGroups = kTile / 16;
  static constexpr int kItems = kGroups * 18;  // 1 KiB load blocks per tile
  static constexpr int kItemsMin = kItems / kWaves;
  static constexpr int kItemsRem = kItems % kWaves;
  static constexpr int kStageBytes = kTile * kRowBytes;
  static constexpr int kMergeStride = 512 + 4;  // floats per head row in the merge area
  static constexpr int kMergeBytes = TS > 1 ? kWaves * 16 * kMergeStride * 4 + kWaves * 16 * 8 : 0;
  static constexpr int kLdsBytes =
      (NSTAGE * kStageBytes > kMergeBytes) ? NSTAGE * kStageBytes : kMergeBytes;
  static constexpr bool kOneBarrier = NSTAGE >= 3;
  static_assert(MB == 1 || MB % 2 == 0, "MB must be 1 or even");
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

template <int HG, int TS, int MB, int NSTAGE>
__global__ void __launch_bounds__(64 * HG * TS)
    mla_decode_bf16_kernel(const DecodeArgs a) {
  using S = DecodeShape<HG, TS, MB, NSTAGE>;
  constexpr int H = S::kHeads;
  constexpr int T = S::kTile;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S::kLdsBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int lane = tid & 63;
  const int hg = wave % HG;
  const int ts = wave / HG;
  const int my_items = S::kItemsMin + (wave < S::kItemsRem ? 1 : 0);
  const int item0 = wave * S::kItemsMin + (wave < S::kItemsRem ? wave : S::kItemsRem);
  const int page_shift = a.page_shift;
  const int page_mask = (1 << page_shift) - 1;

  // ---- per-lane constant LDS offsets -------------------------------------
  // Loader: lane writes LDS slot `lane` of a block: row r = rh*8 + lane/8,
  // logical chunk = cb*8 + ((lane & 7) ^ swz(r)).
  const int ld_r_lo = lane >> 3;  // row within the half group
  // QK operand: token row r = lane & 15, chunk c = 4*s + (lane >> 4).
  const int qr = lane & 15;
  const int qk_base = (qr >> 3) * kHalfGroupBytes + (qr & 7) * 128;
  const int qk_off_even = (((lane >> 4)) ^ swz(qr)) * 16;       // s even: c & 7 = g
  const int qk_off_odd = ((4 + (lane >> 4)) ^ swz(qr)) * 16;    // s odd:  c & 7 = 4 + g
  // PV operand (transpose read): source lane s = 16G + 4j + q reads row 4G + j,
  // 8 bytes at columns c0 + 4q .. c0 + 4q + 3 of a 16-column block c0.
  const int tr_r = 4 * (lane >> 4) + ((lane >> 2) & 3);
  const int tr_q = lane & 3;
  const int tr_base = (tr_r >> 3) * kHalfGroupBytes + (tr_r & 7) * 128 + (tr_q & 1) * 8;
  int tr_off[4];
#pragma unroll
  for (int A = 0; A < 4; ++A) tr_off[A] = tr_base + (((2 * A) | (tr_q >> 1)) ^ swz(tr_r)) * 16;

  const int seg_begin = ld_const(a.worker_ptr + blockIdx.x);
  const int seg_end = ld_const(a.worker_ptr + blockIdx.x + 1);

  for (int si = seg_begin; si < seg_end; ++si) {
    const int* sgp = reinterpret_cast<const int*>(a.segs + si);
    const int b = ld_const(sgp + 0);
    const int t0 = ld_const(sgp + 1);
    const int send = ld_const(sgp + 2);
    const int slot = ld_const(sgp + 3);
    const int pbeg = ld_const(a.kv_indptr + b);
    const int npg = ld_const(a.kv_indptr + b + 1) - pbeg;
    const int ldev = npg > 0 ? ((npg - 1) << page_shift) + ld_const(a.kv_last_page_len + b) : 0;
    const int t1 = min(send, ldev);
    const int ntiles = t1 > t0 ? (t1 - t0 + T - 1) / T : 0;

    float m_run = -INFINITY;  // running max (log2 domain) of this wave's tokens, head = lane & 15
    float l_run = 0.f;        // this lane's share of the running sum
    f32x4 acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // issue the direct-to-LDS loads of tile k into stage st
    auto issue_tile = [&](int k, int st) {
      const int tile_start = t0 + k * T;
      const int last_group = ((t1 - 1) >> 4) << 4;
      uint8_t* stage = smem + st * S::kStageBytes;
      for (int j = 0; j < my_items; ++j) {
        const int item = item0 + j;
        const int g = item / 18;
        const int blk = item - g * 18;
        const int rh = blk >= 9 ? 1 : 0;
        const int cb = blk - rh * 9;
        const int gs = min(tile_start + 16 * g, last_group);
        const int page = ld_const(a.kv_indices + pbeg + (gs >> page_shift));
        const int r = rh * 8 + ld_r_lo;
        const int tok = min(gs + r, t1 - 1);
        const size_t row = ((size_t)page << page_shift) + (tok & page_mask);
        const int c = cb * 8 + ((lane & 7) ^ swz(r));
        const uint8_t* src = c < 64 ? a.ckv + (row * 512 + c * 8) * 2
                                    : a.kpe + (row * 64 + (c - 64) * 8) * 2;
        const uint32_t dst = __builtin_amdgcn_readfirstlane(
            (uint32_t)(uintptr_t)(LDS_AS uint8_t*)(stage + g * kGroupBytes + blk * 1024));
        dma16(src, dst);
      }
    };

    auto wait_for = [&](int later) {
      if (my_items == S::kItemsMin)
        wait_tile<S::kItemsMin>(later);
      else
        wait_tile<S::kItemsMin + 1>(later);
    };

    for (int k = 0; k < NSTAGE - 1 && k < ntiles; ++k) issue_tile(k, k);

    // ---- Q^T operand for head hg*16 + (lane & 15): 18 x 8 dims -----------
    const int head = hg * 16 + qr;
    bf16x8 qf[18];
    {
      const bf16x8* qn = reinterpret_cast<const bf16x8*>(a.q_nope + ((size_t)b * H + head) * 512);
      const bf16x8* qp = reinterpret_cast<const bf16x8*>(a.q_pe + ((size_t)b * H + head) * 64);
#pragma unroll
      for (int s = 0; s < 18; ++s) {
        const int c = 4 * s + (lane >> 4);
        qf[s] = s < 16 ? qn[c] : qp[c - 64];
      }
    }

    // Q (and the previous segment's stores) complete before the tile loop; the
    // explicit full wait also tells the compiler that no vector load is
    // pending, so it adds no waits inside the loop (where only the LDS DMA,
    // which it does not see, is in flight).
    vm_wait_n<0>();


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

      // ---- QK: S^T for this wave's MB row groups -------------------------
      f32x4 sacc[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int gi = ts * MB + mb;
        const uint8_t* gbase = stage + gi * kGroupBytes + qk_base;
        bf16x8 kf[18];
#pragma unroll
        for (int s = 0; s < 18; ++s) {
          const uint8_t* p = gbase + (s >> 1) * 1024 + ((s & 1) ? qk_off_odd : qk_off_even);
          kf[s] = *reinterpret_cast<const LDS_AS bf16x8*>((const LDS_AS uint8_t*)p);
        }
        f32x4 c4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 18; ++s)
          c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], qf[s], c4, 0, 0, 0);
        sacc[mb] = c4;
      }

      // ---- online softmax (log2 domain) -----------------------------------
      float tmax = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int row0 = tile_start + (ts * MB + mb) * 16 + 4 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = (row0 + i < t1) ? sacc[mb][i] * a.scale_log2 : -INFINITY;
          sacc[mb][i] = x;
          tmax = fmaxf(tmax, x);
        }
      }
      tmax = wave_max_16(tmax);
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float psum = 0.f;
      bf16x4 pb[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(sacc[mb][i] - m_use);
          psum += p;
          pb[mb][i] = (__bf16)p;
        }
      }
      l_run = l_run * alpha + psum;
      if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
#pragma unroll
        for (int i = 0; i < 32; ++i) acc[i] *= alpha;
      }
      m_run = m_new;

      // ---- PV: O^T[c, h] += V^T[c, t] P^T[t, h] ----------------------------
      if constexpr (MB == 1) {
        const uint8_t* gbase = stage + (ts * MB) * kGroupBytes;
        const s16x4 pv = __builtin_bit_cast(s16x4, pb[0]);
#pragma unroll
        for (int c8 = 0; c8 < 32; c8 += S::kPvBatch) {
          s16x4 vf[S::kPvBatch];
#pragma unroll
          for (int u = 0; u < S::kPvBatch; ++u) {
            const int cb = c8 + u;
            const uint8_t* p = gbase + (cb >> 2) * 1024 + tr_off[cb & 3];
            vf[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)((LDS_AS uint8_t*)p));
          }
#pragma unroll
          for (int u = 0; u < S::kPvBatch; ++u)
            acc[c8 + u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf[u], pv, acc[c8 + u], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int mp = 0; mp < MB; mp += 2) {
          const uint8_t* g0 = stage + (ts * MB + mp) * kGroupBytes;
          const uint8_t* g1 = g0 + kGroupBytes;
          bf16x8 pv;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pv[i] = pb[mp][i];
            pv[4 + i] = pb[mp + 1][i];
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
              acc[c8 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[u], pv, acc[c8 + u], 0, 0, 0);
          }
        }
      }
      if constexpr (!S::kOneBarrier) lds_barrier();
    }
    if constexpr (S::kOneBarrier) lds_barrier();  // ring free before the merge / next segment

    // ---- epilogue -----------------------------------------------------------
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
          for (int i = 0; i < 4; ++i) v[i] = (__bf16)(acc[cb][i] * inv);
          *reinterpret_cast<bf16x4*>(op + cb * 16 + 4 * (lane >> 4)) = v;
        }
        if (lane < 16) a.lse[orow] = lse_v;
      } else {
        const size_t prow = (size_t)slot * H + head;
        float* op = a.part_o + prow * 512;
#pragma unroll
        for (int cb = 0; cb < 32; ++cb)
          *reinterpret_cast<f32x4*>(op + cb * 16 + 4 * (lane >> 4)) = acc[cb] * inv;
        if (lane < 16) a.part_lse[prow] = lse_v;
      }
    } else {
      // merge the TS token-split waves of each head group through LDS
      float* mo = reinterpret_cast<float*>(smem);
      float* mstat = mo + S::kWaves * 16 * S::kMergeStride;  // [wave][16][2] (m, l)
      float* mine = mo + wave * 16 * S::kMergeStride;
#pragma unroll
      for (int cb = 0; cb < 32; ++cb)
        *reinterpret_cast<f32x4*>(mine + qr * S::kMergeStride + cb * 16 + 4 * (lane >> 4)) =
            acc[cb];
      if (lane < 16) {
        mstat[(wave * 16 + lane) * 2 + 0] = m_run;
        mstat[(wave * 16 + lane) * 2 + 1] = l_tot;
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
          const float* src = mo + (u * HG + hg) * 16 * S::kMergeStride + hh * S::kMergeStride + col;
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
        const int hd = hg * 16 + hh;
        if (slot < 0) {
          bf16x8 v;
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = (__bf16)(o8[i] * inv);
          *reinterpret_cast<bf16x8*>(a.o + ((size_t)b * H + hd) * 512 + col) = v;
          if (ts == 0 && (e % (kCols / 8)) == 0) a.lse[(size_t)b * H + hd] = lse_v;
        } else {
          float* dst = a.part_o + ((size_t)slot * H + hd) * 512 + col;
          f32x4 y0, y1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            y0[i] = o8[i] * inv;
            y1[i] = o8[4 + i] * inv;
          }
          *reinterpret_cast<f32x4*>(dst) = y0;
          *reinterpret_cast<f32x4*>(dst + 4) = y1;
          if (ts == 0 && (e % (kCols / 8)) == 0) a.part_lse[(size_t)slot * H + hd] = lse_v;
        }
      }
      lds_barrier();  // merge area free before the next segment's loads
    }
  }
}

// One block per (split request, group of 4 heads); thread = (head, 8 columns).
__global__ void __launch_bounds__(256) mla_combine_kernel(const CombineArgs a) {
  const int4 cmb = a.comb[blockIdx.x];
  const int b = cmb.x, slot0 = cmb.y, n = cmb.z;
  const int hd = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int col = (threadIdx.x & 63) * 8;
  const int H = a.num_heads;
  float M = -INFINITY;
  for (int i = 0; i < n; ++i) M = fmaxf(M, a.part_lse[(size_t)(slot0 + i) * H + hd]);
  const float Mu = M == -INFINITY ? 0.f : M;
  float sum = 0.f;
  for (int i = 0; i < n; ++i) sum += __expf(a.part_lse[(size_t)(slot0 + i) * H + hd] - Mu);
  const bool empty = !(sum > 0.f);
  const float lse_v = empty ? -INFINITY : Mu + __logf(sum);
  float o8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o8[i] = 0.f;
  for (int i = 0; i < n; ++i) {
    const float li = a.part_lse[(size_t)(slot0 + i) * H + hd];
    const float w = empty ? 0.f : __expf(li - lse_v);
    const float* src = a.part_o + ((size_t)(slot0 + i) * H + hd) * 512 + col;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o8[j] += w * x0[j];
      o8[4 + j] += w * x1[j];
    }
  }
  bf16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (__bf16)o8[j];
  *reinterpret_cast<bf16x8*>(a.o + ((size_t)b * H + hd) * 512 + col) = v;
  if ((threadIdx.x & 63) == 0) a.lse[(size_t)b * H + hd] = lse_v;
}

// ---------------------------------------------------------------- launchers
template <int HG, int TS, int MB, int NSTAGE>
static hipError_t launch_decode_cfg(const DecodeArgs& a, int grid, hipStream_t stream) {
  using S = DecodeShape<HG, TS, MB, NSTAGE>;
  hipLaunchKernelGGL((mla_decode_bf16_kernel<HG, TS, MB, NSTAGE>), dim3(grid), dim3(S::kThreads),
                     0, stream, a);
  return hipGetLastError();
}

int decode_config(int num_heads, DecodeConfig* cfg) {
  switch (num_heads) {
    case 16: *cfg = DecodeConfig{4, 64}; return 0;
    case 32: *cfg = DecodeConfig{4, 64}; return 0;
    case 64: *cfg = DecodeConfig{4, 32}; return 0;
    case 128: *cfg = DecodeConfig{8, 32}; return 0;
    default: return -1;
  }
}

hipError_t launch_decode(int num_heads, const DecodeArgs& a, int grid, hipStream_t stream) {
  switch (num_heads) {
    case 16: return launch_decode_cfg<1, 4, 1, 2>(a, grid, stream);
    case 32: return launch_decode_cfg<2, 2, 2, 2>(a, grid, stream);
    case 64: return launch_decode_cfg<4, 1, 2, 3>(a, grid, stream);
    case 128: return launch_decode_cfg<8, 1, 2, 3>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_combine(const CombineArgs& a, int num_split_requests, hipStream_t stream) {
  if (num_split_requests <= 0) return hipSuccess;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(num_split_requests, a.num_heads / 4), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace mla_gpu
