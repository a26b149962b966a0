// gfx950 kernel for appending new latent tokens to the paged cache, with
// quantisation on write for 8-bit caches.
//
// FlashMLA PR 233, "What is added": an 8-bit latent cache (FP8 e4m3 or INT8)
// with one fp32 scale per token, written by the layer's prologue.  Per token
// (576 values: 512 ckv, 64 kpe, bf16):
//   amax  = max |x_i|;  scale = amax / 448 (e4m3) or / 127 (int8), binary32,
//           1 for an all-zero token
//   code_i = nearest representable value of x_i / scale (binary32 division),
//           ties to even, saturated at +-448 / +-127
// One wave per token: lane l holds ckv values 8l .. 8l + 7 and kpe value l,
// the max is a wave reduction, and each lane stores its 8 + 1 codes.  The
// 644-byte record (same page: 8-bit ckv, bf16 kpe, one scale per token) takes
// amax over the 512 ckv values only and stores kpe unchanged (KVT 3 / 4).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "append.h"

namespace mla_gpu {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_float(unsigned bits16) {
  return __uint_as_float(bits16 << 16);
}

// e4m3fn code of v (OCP: bias 7, 3 mantissa bits, no infinity, 0x7F NaN,
// largest finite 448): nearest value, ties to even mantissa, saturated.
__device__ __forceinline__ unsigned encode_e4m3fn(float v) {
  const unsigned u = __float_as_uint(v);
  const unsigned sign = (u >> 24) & 0x80u;
  const unsigned mag = u & 0x7FFFFFFFu;
  const float a = __uint_as_float(mag);
  if (!(a < 448.f)) return sign | 0x7Eu;
  if (a < 0.015625f) {  // below 2^-6: the subnormal grid, steps of 2^-9
    return sign | (unsigned)__builtin_rintf(a * 512.f);  // exact scaling; 8 = 2^-6
  }
  unsigned e = (mag >> 23) - 127u + 7u;  // 1 .. 15
  unsigned keep = (mag >> 20) & 7u;      // top 3 mantissa bits
  const unsigned rest = mag & 0xFFFFFu;  // the 20 bits below them
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
  if (keep == 8u) {
    keep = 0u;
    ++e;
  }
  return sign | (e << 3) | keep;  // a < 448 keeps this at or below 0x7E
}

__device__ __forceinline__ unsigned encode_int8(float v) {
  float r = __builtin_rintf(v);
  r = fminf(fmaxf(r, -127.f), 127.f);
  return (unsigned)(int)r & 0xFFu;
}

template <int KVT>
__global__ void __launch_bounds__(256)
    mla_cache_append_kernel(const uint16_t* ckv_new, const uint16_t* kpe_new,
                            const int64_t* slots, int n, uint8_t* ckv, uint8_t* kpe,
                            float* kv_scale) {
  const int j = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (j >= n) return;  // whole wave
  const int64_t slot = slots[j];
  if (slot < 0) return;  // padding token, whole wave
  const u32x4 c = *reinterpret_cast<const u32x4*>(ckv_new + (size_t)j * 512 + lane * 8);
  const unsigned k = kpe_new[(size_t)j * 64 + lane];
  if constexpr (KVT == 0 || KVT == 5) {  // 16-bit cache: copy
    *reinterpret_cast<u32x4*>(ckv + slot * 1024 + lane * 16) = c;
    *reinterpret_cast<uint16_t*>(kpe + slot * 128 + lane * 2) = (uint16_t)k;
  } else {
    float x[9];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_to_float(c[i] & 0xFFFFu);
      x[2 * i + 1] = bf16_to_float(c[i] >> 16);
    }
    constexpr bool kpe16 = KVT == 3 || KVT == 4;  // 644-byte record
    constexpr bool fp8 = KVT == 1 || KVT == 3;
    constexpr int nq = kpe16 ? 8 : 9;  // values of this lane that are quantised
    x[8] = bf16_to_float(k);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < nq; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float qmax = fp8 ? 448.f : 127.f;
    const float scale = amax > 0.f ? amax / qmax : 1.f;  // correctly rounded division
    unsigned codes[9];
#pragma unroll
    for (int i = 0; i < nq; ++i) {
      const float v = x[i] / scale;
      codes[i] = fp8 ? encode_e4m3fn(v) : encode_int8(v);
    }
    u32x2 w;
    w[0] = codes[0] | (codes[1] << 8) | (codes[2] << 16) | (codes[3] << 24);
    w[1] = codes[4] | (codes[5] << 8) | (codes[6] << 16) | (codes[7] << 24);
    *reinterpret_cast<u32x2*>(ckv + slot * 512 + lane * 8) = w;
    if constexpr (kpe16)
      *reinterpret_cast<uint16_t*>(kpe + slot * 128 + lane * 2) = (uint16_t)k;
    else
      kpe[slot * 64 + lane] = (uint8_t)codes[8];
    if (lane == 0) kv_scale[slot] = scale;
  }
}

}  // namespace

hipError_t launch_cache_append(int kv_dtype, const uint16_t* ckv_new, const uint16_t* kpe_new,
                               const int64_t* slots, int n, uint8_t* ckv, uint8_t* kpe,
                               float* kv_scale, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const dim3 grid((n + 3) / 4), block(256);
  switch (kv_dtype) {
    case 0:
      hipLaunchKernelGGL(mla_cache_append_kernel<0>, grid, block, 0, stream, ckv_new, kpe_new,
                         slots, n, ckv, kpe, kv_scale);
      break;
    case 1:
      hipLaunchKernelGGL(mla_cache_append_kernel<1>, grid, block, 0, stream, ckv_new, kpe_new,
                         slots, n, ckv, kpe, kv_scale);
      break;
    case 2:
      hipLaunchKernelGGL(mla_cache_append_kernel<2>, grid, block, 0, stream, ckv_new, kpe_new,
                         slots, n, ckv, kpe, kv_scale);
      break;
    case 3:
      hipLaunchKernelGGL(mla_cache_append_kernel<3>, grid, block, 0, stream, ckv_new, kpe_new,
                         slots, n, ckv, kpe, kv_scale);
      break;
    case 4:
      hipLaunchKernelGGL(mla_cache_append_kernel<4>, grid, block, 0, stream, ckv_new, kpe_new,
                         slots, n, ckv, kpe, kv_scale);
      break;
    case 5:
      hipLaunchKernelGGL(mla_cache_append_kernel<5>, grid, block, 0, stream, ckv_new, kpe_new,
                         slots, n, ckv, kpe, kv_scale);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla_gpu
