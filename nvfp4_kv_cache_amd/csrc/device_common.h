// Device helpers shared by the gfx950 kernels: bf16 bits, a wave maximum and HIP
// error plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nvfp4kv.h"
#include "nvfp4kv_internal.h"

namespace nvfp4kv {

#define NVFP4KV_HIP_OK(expr) ((expr) == hipSuccess ? NVFP4KV_OK : NVFP4KV_EHIP)

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
  return __uint_as_float(h << 16);
}

template <typename T>
__device__ __forceinline__ T wave_max_u32(T v) {
  for (int off = 32; off >= 1; off >>= 1) {
    const T o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

}  // namespace nvfp4kv
