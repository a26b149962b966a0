// Measurement kernels for the roofline denominators (not part of the decode
// path): a 16-byte-load stream read over a large buffer and an all-CU bf16
// MFMA loop.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <string>
#include <vector>

#include "../../include/mla_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Each workgroup streams one contiguous slice of the buffer, 8 x 16-byte
// loads in flight per lane (the access pattern that reaches the highest read
// bandwidth on MI355X in our measurements).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kStreamDepth = 8;

__global__ void __launch_bounds__(512) stream_read_kernel(const unsigned char* __restrict__ buf,
                                                          size_t per_wg, size_t bytes,
                                                          uint32_t* __restrict__ sink) {
  const size_t begin = (size_t)blockIdx.x * per_wg;
  const size_t end = begin + per_wg < bytes ? begin + per_wg : bytes;
  const size_t chunk = (size_t)blockDim.x * 16 * kStreamDepth;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t off = begin;
  for (; off + chunk <= end; off += chunk) {
    u32x4 v[kStreamDepth];
#pragma unroll
    for (int d = 0; d < kStreamDepth; ++d)
      v[d] = *reinterpret_cast<const u32x4*>(buf + off + ((size_t)d * blockDim.x + threadIdx.x) * 16);
#pragma unroll
    for (int d = 0; d < kStreamDepth; ++d) acc ^= v[d];
  }
  for (size_t i = off + (size_t)threadIdx.x * 16; i + 16 <= end; i += (size_t)blockDim.x * 16)
    acc ^= *reinterpret_cast<const u32x4*>(buf + i);
  sink[(blockIdx.x * blockDim.x + threadIdx.x) & 0x3FFFF] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

constexpr int kMfmaChains = 8;
constexpr int kMfmaIters = 4096;

__global__ void __launch_bounds__(256) mfma_bf16_kernel(float* __restrict__ sink, float seed) {
  bf16x8 a, b;
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(seed * (threadIdx.x + j));
    b[j] = (__bf16)(seed * (blockIdx.x - j));
  }
  f32x4 c[kMfmaChains];
  for (int k = 0; k < kMfmaChains; ++k) c[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < kMfmaIters; ++it) {
#pragma unroll
    for (int k = 0; k < kMfmaChains; ++k)
      c[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[k], 0, 0, 0);
  }
  float s = 0.f;
  for (int k = 0; k < kMfmaChains; ++k) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
  sink[(blockIdx.x * blockDim.x + threadIdx.x) & 0x3FFFF] = s;
}

template <class Launch>
mla_status time_median(int iters, hipStream_t s, Launch launch, float* ms_out) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  mla_status st = MLA_ERR_HIP;
  std::vector<float> t;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) goto done;
  launch();  // warm-up
  for (int i = 0; i < iters; ++i) {
    float ms = 0.f;
    if (hipEventRecord(e0, s) != hipSuccess) goto done;
    launch();
    if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
        hipEventElapsedTime(&ms, e0, e1) != hipSuccess)
      goto done;
    t.push_back(ms);
  }
  if (hipGetLastError() != hipSuccess) goto done;
  std::sort(t.begin(), t.end());
  *ms_out = t[t.size() / 2];
  st = MLA_OK;
done:
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  return st;
}

}  // namespace

extern "C" {

mla_status mla_peak_stream_read(const void* buf, size_t bytes, void* sink, int32_t iters,
                                float* ms_out, void* stream) {
  if (!buf || !sink || !ms_out || iters <= 0 || bytes < 16 || bytes % 16) return MLA_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MLA_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int grid = cus * 2;  // two 512-thread workgroups per CU, one contiguous slice each
  const size_t per_wg = ((bytes + grid - 1) / grid + 15) & ~(size_t)15;
  return time_median(iters, s, [&] {
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(512), 0, s,
                       static_cast<const unsigned char*>(buf), per_wg, bytes,
                       static_cast<uint32_t*>(sink));
  }, ms_out);
}

mla_status mla_peak_mfma_bf16(void* sink, int32_t iters, float* tflops_out, void* stream) {
  if (!sink || !tflops_out || iters <= 0) return MLA_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MLA_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int grid = cus * 2;  // 8 waves per CU: 2 per SIMD
  float ms = 0.f;
  mla_status st = time_median(iters, s, [&] {
    hipLaunchKernelGGL(mfma_bf16_kernel, dim3(grid), dim3(256), 0, s, static_cast<float*>(sink),
                       1e-3f);
  }, &ms);
  if (st != MLA_OK) return st;
  const double flops = (double)grid * 4 * kMfmaIters * kMfmaChains * 16.0 * 16.0 * 32.0 * 2.0;
  *tflops_out = (float)(flops / (ms * 1e-3) / 1e12);
  return MLA_OK;
}

}  // extern "C"
