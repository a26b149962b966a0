// Launch interface of the cache-append kernel (internal to the library; the
// public C ABI is include/mla_decode.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla_gpu {

// kv_dtype 0 bf16 / 5 fp16 (copy; new tokens of the same type), 1 fp8 e4m3, 2 int8 (quantise ckv and kpe), 3 / 4 fp8 / int8
// ckv with bf16 kpe (quantise ckv, copy kpe); slots[j] < 0 skips token j.
hipError_t launch_cache_append(int kv_dtype, const uint16_t* ckv_new, const uint16_t* kpe_new,
                               const int64_t* slots, int n, uint8_t* ckv, uint8_t* kpe,
                               float* kv_scale, hipStream_t stream);

}  // namespace mla_gpu
