// Copies one resident chunk out of the cache into the codec layout (K and V codes
// [h][token][D/2], scales [h][token][D/block] with block 16 for NVFP4 and 32 for
// MXFP4, and the two fp32 tensor scales, 1 for MXFP4), and
// small device utilities.  V is stored transposed in the cache ([h][d][token/2]),
// so its codes are regathered here nibble by nibble.  Not on the hot path.

#include "device_common.h"

namespace nvfp4kv {

__global__ void export_chunk_kernel(ExportArgs a) {
  const int nb = a.D / a.block;
  const int64_t ntok = int64_t(a.n_frames) * a.T_f;
  const int64_t n_codes = int64_t(a.H) * ntok * (a.D / 2);
  const int64_t n_scales = int64_t(a.H) * ntok * nb;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n_codes; i += stride) {
    const int64_t j = i % (a.D / 2);
    const int64_t t = (i / (a.D / 2)) % ntok;
    const int64_t h = i / ((a.D / 2) * ntok);
    const int64_t stok = int64_t(a.frame_slot[t / a.T_f]) * a.T_f + t % a.T_f;
    a.k_codes_out[i] = a.kcodes[(h * a.rows + stok) * (a.D / 2) + j];
    uint32_t byte = 0;
    for (int e = 0; e < 2; ++e) {
      const int64_t d = 2 * j + e;
      const uint32_t packed = a.vcodes[(h * a.D + d) * (a.rows / 2) + stok / 2];
      byte |= ((packed >> (4 * (stok & 1))) & 0xFu) << (4 * e);
    }
    a.v_codes_out[i] = uint8_t(byte);
  }
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n_scales; i += stride) {
    const int64_t b = i % nb;
    const int64_t t = (i / nb) % ntok;
    const int64_t h = i / (nb * ntok);
    const int64_t stok = int64_t(a.frame_slot[t / a.T_f]) * a.T_f + t % a.T_f;
    a.k_scales_out[i] = a.kscales[(h * a.rows + stok) * nb + b];
    a.v_scales_out[i] = a.vscales[(h * nb + b) * a.rows + stok];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *a.k_scale_out = a.scale_table[2 * a.scale_slot];
    *a.v_scale_out = a.scale_table[2 * a.scale_slot + 1];
  }
}

int launch_export(const ExportArgs &a, void *stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(export_chunk_kernel, dim3(1024), dim3(256), 0, s, a);
  return NVFP4KV_HIP_OK(hipGetLastError());
}

int copy_device_floats(float *dst, const float *src, size_t n, void *stream) {
  if (n == 0) return NVFP4KV_OK;
  return NVFP4KV_HIP_OK(hipMemcpyAsync(dst, src, n * sizeof(float), hipMemcpyDeviceToDevice,
                                       reinterpret_cast<hipStream_t>(stream)));
}

int zero_device_bytes_blocking(void *ptr, size_t bytes) {
  if (bytes == 0) return NVFP4KV_OK;
  return NVFP4KV_HIP_OK(hipMemset(ptr, 0, bytes));
}

}  // namespace nvfp4kv
