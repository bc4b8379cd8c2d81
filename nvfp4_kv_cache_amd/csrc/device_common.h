// Device helpers shared by the gfx950 kernels: NVFP4 code arithmetic and HIP
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

// Round v >= 0 (finite) to the nearest E4M3FN value, ties to the even code,
// saturating at 448 (0x7E).  Paper section 2.2 fixes E4M3 with max 448.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
  if (!(v > 0.0f)) return 0u;
  if (v >= 448.0f) return 0x7Eu;
  if (v < 0.015625f) {                       // below 2^-6: subnormal step 2^-9
    return uint32_t(__builtin_rintf(v * 512.0f));   // exact scaling, RNE; 8 -> 0x08
  }
  uint32_t b = __float_as_uint(v);
  b += 0x7FFFFu + ((b >> 20) & 1u);          // keep 3 mantissa bits, ties to even
  const uint32_t code = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
  return code > 0x7Eu ? 0x7Eu : code;
}

// Value of a non-negative E4M3FN byte (0x00..0x7E), exact in fp32.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = c >> 3, m = c & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : float(m) * 0.001953125f;
}

// E2M1 magnitude code of q >= 0: nearest of {0,.5,1,1.5,2,3,4,6}, ties to the
// even code, saturating at 6.  The open/closed interval ends carry the ties.
__device__ __forceinline__ uint32_t e2m1_rne_sat(float q) {
  return uint32_t(q > 0.25f) + uint32_t(q >= 0.75f) + uint32_t(q > 1.25f) +
         uint32_t(q >= 1.75f) + uint32_t(q > 2.5f) + uint32_t(q >= 3.5f) +
         uint32_t(q > 5.0f);
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
