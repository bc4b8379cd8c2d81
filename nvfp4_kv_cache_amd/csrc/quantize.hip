// NVFP4 quantization of K/V chunks for gfx950.
//
// Format (paper text section 2.2; reading note section II "The NVFP4
// quantization format"): 16-element blocks along head_dim, one E4M3 scale per
// block, one fp32 scale per tensor, E2M1 elements.  Recipe: s_t = amax/2688,
// bs = (block amax / 6) / s_t -> E4M3 (RNE, saturating), code = E2M1(|x| / (E4M3(bs)
// * s_t)) (RNE, saturating), sign kept; fp32 throughout with IEEE division.
//
// The tensor scale needs the amax of the whole chunk tensor before any block can
// be encoded.  The main kernel does it in ONE read of the input: every workgroup
// loads its tiles into registers and reduces their maxima, all workgroups meet at
// a grid barrier (cooperative launch, so all are co-resident), read the per-
// workgroup partial maxima, and encode from registers.  Inputs too large to sit
// in registers take a two-kernel path (amax pass, then an encode pass that re-reads
// the input).
//
// Work unit: a tile of (256 / (D/16)) token pairs x all D/16 blocks of one head of
// one frame; thread (pair p, block b) owns 2 tokens x 16 elements.  Tiles never
// straddle a frame, so each tile lands in one cache slot.  K (and the standalone
// codec) are written in the codec layout [h][token][D/2]; V in the cache is written
// transposed, [h][d][token/2], via an LDS transpose, so that the attention kernel
// can read 8 consecutive keys of one d with one load.

#include "device_common.h"

namespace nvfp4kv {

namespace {

struct TileInfo {
  int tensor, h, f, ti;
};

__device__ __forceinline__ TileInfo decode_tile(const QuantArgs &a, int tile) {
  const int per_tensor = a.H * a.n_frames * a.tiles_per_frame;
  TileInfo t;
  t.tensor = tile / per_tensor;
  int r = tile - t.tensor * per_tensor;
  const int per_head = a.n_frames * a.tiles_per_frame;
  t.h = r / per_head;
  r -= t.h * per_head;
  t.f = r / a.tiles_per_frame;
  t.ti = r - t.f * a.tiles_per_frame;
  return t;
}

// Loads the 2 x 16 bf16 of (pair tp, block b) of a tile; returns block maxima of
// |x| as bf16 bit patterns packed (token 2tp in the low half).
__device__ __forceinline__ uint32_t load_item(const QuantArgs &a, const TileInfo &t, int tp,
                                              int b, uint32_t (&x)[16]) {
  const int tin = t.ti * a.tile_tokens + 2 * tp;
  const int tok = t.f * a.tokens_per_frame + tin;
  const uint16_t *src =
      a.t[t.tensor].src + (int64_t(t.h) * a.T + tok) * a.D + b * 16;
  uint32_t m0 = 0, m1 = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = 0;
  if (tin < a.tokens_per_frame) {
    const uint4 *p = reinterpret_cast<const uint4 *>(src);
    const uint4 u0 = p[0], u1 = p[1];
    x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w;
    x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
  }
  if (tin + 1 < a.tokens_per_frame) {
    const uint4 *p = reinterpret_cast<const uint4 *>(src + a.D);
    const uint4 u0 = p[0], u1 = p[1];
    x[8] = u0.x; x[9] = u0.y; x[10] = u0.z; x[11] = u0.w;
    x[12] = u1.x; x[13] = u1.y; x[14] = u1.z; x[15] = u1.w;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t w = x[j] & 0x7FFF7FFFu;
    m0 = max(m0, max(w & 0xFFFFu, w >> 16));
    const uint32_t w1 = x[8 + j] & 0x7FFF7FFFu;
    m1 = max(m1, max(w1 & 0xFFFFu, w1 >> 16));
  }
  return m0 | (m1 << 16);
}

// Encodes the 16 elements of one token given the block maximum (bf16 bits) and
// the tensor scale.  Returns the scale byte; codes go to c[0] (elements 0-7) and
// c[1] (8-15), element e in nibble e % 8.
__device__ __forceinline__ uint32_t encode_block(const uint32_t *x8, uint32_t bmax_bits,
                                                 float st, uint32_t (&c)[2]) {
  uint32_t sc = 0;
  float eff = 0.0f;
  if (st > 0.0f) {
    const float bs = (bf16_bits_to_float(bmax_bits) / 6.0f) / st;
    sc = e4m3_rne_sat(bs);
    eff = e4m3_value(sc) * st;
  }
  c[0] = c[1] = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t w = x8[e >> 1];
    const uint32_t hb = (e & 1) ? (w >> 16) : (w & 0xFFFFu);
    uint32_t mag = 0;
    if (eff > 0.0f) mag = e2m1_rne_sat(bf16_bits_to_float(hb & 0x7FFFu) / eff);
    const uint32_t code = mag | ((hb >> 12) & 8u);
    c[e >> 3] |= code << (4 * (e & 7));
  }
  return sc;
}

__device__ __forceinline__ void encode_store_item(const QuantArgs &a, const TileInfo &t, int tp,
                                                  int b, const uint32_t (&x)[16],
                                                  uint32_t bmax, float st, uint8_t *s_tr,
                                                  int TP) {
  const QuantTensor &qt = a.t[t.tensor];
  const int nb = a.D >> 4;
  const int tin = t.ti * a.tile_tokens + 2 * tp;
  const bool v0 = tin < a.tokens_per_frame, v1 = tin + 1 < a.tokens_per_frame;
  const int64_t dtok = int64_t(a.frame_slot[t.f]) * a.tokens_per_frame + tin;
  uint32_t c0[2], c1[2];
  const uint32_t s0 = encode_block(x, bmax & 0xFFFFu, st, c0);
  const uint32_t s1 = encode_block(x + 8, bmax >> 16, st, c1);
  if (!qt.transposed) {
    if (v0) {
      *reinterpret_cast<uint2 *>(qt.codes + (int64_t(t.h) * a.rows + dtok) * (a.D / 2) + b * 8) =
          make_uint2(c0[0], c0[1]);
      qt.scales[(int64_t(t.h) * a.rows + dtok) * nb + b] = uint8_t(s0);
    }
    if (v1) {
      *reinterpret_cast<uint2 *>(qt.codes + (int64_t(t.h) * a.rows + dtok + 1) * (a.D / 2) +
                                 b * 8) = make_uint2(c1[0], c1[1]);
      qt.scales[(int64_t(t.h) * a.rows + dtok + 1) * nb + b] = uint8_t(s1);
    }
  } else {
    // token pair -> one byte per d; staged in LDS as [d][pair]
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t lo = (c0[e >> 3] >> (4 * (e & 7))) & 0xFu;
      const uint32_t hi = (c1[e >> 3] >> (4 * (e & 7))) & 0xFu;
      s_tr[(b * 16 + e) * TP + tp] = uint8_t(lo | (hi << 4));
    }
    if (v0) {
      *reinterpret_cast<uint16_t *>(qt.scales + (int64_t(t.h) * nb + b) * a.rows + dtok) =
          uint16_t(s0 | (s1 << 8));
    }
  }
}

// Writes one LDS-staged transposed tile ([D][TP] bytes) to V's [h][d][rows/2] plane.
__device__ __forceinline__ void store_transposed_tile(const QuantArgs &a, const TileInfo &t,
                                                      const uint8_t *s_tr, int TP) {
  const QuantTensor &qt = a.t[t.tensor];
  const int tid = threadIdx.x;
  const int per_row = TP / 16;              // 16-byte pieces per d row
  const int r = tid / per_row;
  const int col = (tid - r * per_row) * 16;
  if (r >= a.D) return;
  const int tok0 = t.ti * a.tile_tokens;
  int nvalid = a.tokens_per_frame - tok0;
  if (nvalid > a.tile_tokens) nvalid = a.tile_tokens;
  const int nbytes = nvalid / 2;            // multiple of 4 (T_f % 8 == 0)
  const int64_t dst0 = (int64_t(a.frame_slot[t.f]) * a.tokens_per_frame + tok0) / 2;
  uint32_t *dst = reinterpret_cast<uint32_t *>(qt.codes + (int64_t(t.h) * a.D + r) * (a.rows / 2) +
                                               dst0 + col);
  const uint32_t *src = reinterpret_cast<const uint32_t *>(s_tr + r * TP + col);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (col + 4 * j < nbytes) dst[j] = src[j];
}

__device__ __forceinline__ void block_reduce_max2(uint32_t &m0, uint32_t &m1, uint32_t *s_red) {
  m0 = wave_max_u32(m0);
  m1 = wave_max_u32(m1);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) {
    s_red[w] = m0;
    s_red[8 + w] = m1;
  }
  __syncthreads();
  m0 = 0;
  m1 = 0;
#pragma unroll
  for (int i = 0; i < kQuantThreads / 64; ++i) {
    m0 = max(m0, s_red[i]);
    m1 = max(m1, s_red[8 + i]);
  }
  __syncthreads();
}

__device__ __forceinline__ uint32_t atomic_load_relaxed(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Reads the per-workgroup partial maxima of an amax pass of `g` workgroups and
// returns both tensors' scales s_t = amax / 2688 via LDS.
__device__ __forceinline__ void read_tensor_scales(const QuantArgs &a, int g, uint32_t *s_red,
                                                   float *s_st) {
  uint32_t m0 = 0, m1 = 0;
  for (int j = threadIdx.x; j < g; j += kQuantThreads) {
    m0 = max(m0, atomic_load_relaxed(&a.ws->partial[0][j]));
    m1 = max(m1, atomic_load_relaxed(&a.ws->partial[1][j]));
  }
  block_reduce_max2(m0, m1, s_red);
  if (threadIdx.x == 0) {
    s_st[0] = __uint_as_float(m0) / 2688.0f;
    s_st[1] = __uint_as_float(m1) / 2688.0f;
  }
  __syncthreads();
}

}  // namespace

// Single pass: registers hold every tile of the workgroup across the grid barrier.
template <int ITEMS>
__global__ __launch_bounds__(kQuantThreads) void quantize_coop_kernel(QuantArgs a) {
  __shared__ uint32_t s_red[16];
  __shared__ float s_st[2];
  __shared__ uint8_t s_tr[4096];
  const int tid = threadIdx.x;
  const int nb = a.D >> 4;
  const int TP = kQuantThreads / nb;
  const bool act = tid < TP * nb;
  const int b = tid % nb, tp = tid / nb;

  uint32_t x[ITEMS][16];
  uint32_t bmax[ITEMS];
  uint32_t tm[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int tile = blockIdx.x + i * gridDim.x;
    bmax[i] = 0;
    if (tile < a.total_tiles && act) {
      const TileInfo t = decode_tile(a, tile);
      bmax[i] = load_item(a, t, tp, b, x[i]);
      const uint32_t m = max(bmax[i] & 0xFFFFu, bmax[i] >> 16);
      if (t.tensor == 0) tm[0] = max(tm[0], m);
      else tm[1] = max(tm[1], m);
    }
  }
  // workgroup maxima (as fp32 bit patterns) -> partials -> grid barrier
  uint32_t m0 = tm[0] << 16, m1 = tm[1] << 16;
  block_reduce_max2(m0, m1, s_red);
  if (tid == 0) {
    a.ws->partial[0][blockIdx.x] = m0;
    a.ws->partial[1][blockIdx.x] = m1;
    const uint32_t gen = __hip_atomic_load(&a.ws->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t arrived = __hip_atomic_fetch_add(&a.ws->count, 1u, __ATOMIC_ACQ_REL,
                                                    __HIP_MEMORY_SCOPE_AGENT);
    if (arrived == gridDim.x - 1) {
      __hip_atomic_store(&a.ws->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ws->gen, gen + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      // all workgroups are co-resident (cooperative launch); the bound only keeps a
      // corrupted workspace from hanging the device
      uint32_t spins = 0;
      while (__hip_atomic_load(&a.ws->gen, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == gen) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > (1u << 26)) {
          __hip_atomic_store(&a.ws->timeout, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
  }
  __syncthreads();
  read_tensor_scales(a, gridDim.x, s_red, s_st);
  if (blockIdx.x == 0 && tid < a.n_tensors) *a.t[tid].tensor_scale = s_st[tid];

#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int tile = blockIdx.x + i * gridDim.x;
    if (tile >= a.total_tiles) break;   // uniform across the workgroup
    const TileInfo t = decode_tile(a, tile);
    const bool tr = a.t[t.tensor].transposed != 0;
    if (act) encode_store_item(a, t, tp, b, x[i], bmax[i], s_st[t.tensor], s_tr, TP);
    if (tr) {
      __syncthreads();
      store_transposed_tile(a, t, s_tr, TP);
      __syncthreads();
    }
  }
}

// Two-pass fallback, pass 1: per-workgroup maxima over a grid-stride set of tiles.
__global__ __launch_bounds__(kQuantThreads) void quantize_amax_kernel(QuantArgs a) {
  __shared__ uint32_t s_red[16];
  const int tid = threadIdx.x;
  const int nb = a.D >> 4;
  const int TP = kQuantThreads / nb;
  const bool act = tid < TP * nb;
  const int b = tid % nb, tp = tid / nb;
  uint32_t tm[2] = {0u, 0u};
  for (int tile = blockIdx.x; tile < a.total_tiles; tile += gridDim.x) {
    if (!act) continue;
    const TileInfo t = decode_tile(a, tile);
    uint32_t x[16];
    const uint32_t bm = load_item(a, t, tp, b, x);
    const uint32_t m = max(bm & 0xFFFFu, bm >> 16);
    if (t.tensor == 0) tm[0] = max(tm[0], m);
    else tm[1] = max(tm[1], m);
  }
  uint32_t m0 = tm[0] << 16, m1 = tm[1] << 16;
  block_reduce_max2(m0, m1, s_red);
  if (tid == 0) {
    a.ws->partial[0][blockIdx.x] = m0;
    a.ws->partial[1][blockIdx.x] = m1;
  }
}

// Two-pass fallback, pass 2: re-reads the input and encodes.
__global__ __launch_bounds__(kQuantThreads) void quantize_encode_kernel(QuantArgs a, int g_amax) {
  __shared__ uint32_t s_red[16];
  __shared__ float s_st[2];
  __shared__ uint8_t s_tr[4096];
  const int tid = threadIdx.x;
  const int nb = a.D >> 4;
  const int TP = kQuantThreads / nb;
  const bool act = tid < TP * nb;
  const int b = tid % nb, tp = tid / nb;
  read_tensor_scales(a, g_amax, s_red, s_st);
  if (blockIdx.x == 0 && tid < a.n_tensors) *a.t[tid].tensor_scale = s_st[tid];
  for (int tile = blockIdx.x; tile < a.total_tiles; tile += gridDim.x) {
    const TileInfo t = decode_tile(a, tile);
    const bool tr = a.t[t.tensor].transposed != 0;
    if (act) {
      uint32_t x[16];
      const uint32_t bm = load_item(a, t, tp, b, x);
      encode_store_item(a, t, tp, b, x, bm, s_st[t.tensor], s_tr, TP);
    }
    if (tr) {
      __syncthreads();
      store_transposed_tile(a, t, s_tr, TP);
      __syncthreads();
    }
  }
}

namespace {

constexpr int kMaxDevices = 64;
int g_max_grid[kMaxDevices][4];   // per device, per ITEMS in {1,2,4,8}; 0 = unknown
int g_cu_count[kMaxDevices];

int coop_max_grid(int dev, int idx, const void *fn) {
  if (dev < 0 || dev >= kMaxDevices) return 0;
  if (g_max_grid[dev][idx] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kQuantThreads, 0) != hipSuccess)
      return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    g_cu_count[dev] = cus;
    int g = per_cu * cus;
    if (g > kMaxQuantGrid) g = kMaxQuantGrid;
    g_max_grid[dev][idx] = g;
  }
  return g_max_grid[dev][idx];
}

const void *coop_fn(int idx) {
  switch (idx) {
    case 0: return reinterpret_cast<const void *>(&quantize_coop_kernel<1>);
    case 1: return reinterpret_cast<const void *>(&quantize_coop_kernel<2>);
    case 2: return reinterpret_cast<const void *>(&quantize_coop_kernel<4>);
    default: return reinterpret_cast<const void *>(&quantize_coop_kernel<8>);
  }
}

}  // namespace

int quantize_max_grid(int items, int *grid) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4KV_EHIP;
  const int idx = items <= 1 ? 0 : items <= 2 ? 1 : items <= 4 ? 2 : 3;
  *grid = coop_max_grid(dev, idx, coop_fn(idx));
  return *grid > 0 ? NVFP4KV_OK : NVFP4KV_EHIP;
}

int launch_quantize(const QuantArgs &in, void *stream) {
  QuantArgs a = in;
  const int nb = a.D / 16;
  const int TP = kQuantThreads / nb;
  a.tile_tokens = 2 * TP;
  a.tiles_per_frame = (a.tokens_per_frame + a.tile_tokens - 1) / a.tile_tokens;
  const int64_t total = int64_t(a.n_tensors) * a.H * a.n_frames * a.tiles_per_frame;
  if (total >= (int64_t(1) << 31)) return NVFP4KV_EINVAL;
  a.total_tiles = int32_t(total);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4KV_EHIP;

  // smallest register depth whose co-resident grid covers every tile
  for (int idx = 0; idx < 4; ++idx) {
    const int items = 1 << idx;
    const int gmax = coop_max_grid(dev, idx, coop_fn(idx));
    if (gmax <= 0) return NVFP4KV_EHIP;
    const int64_t g = (total + items - 1) / items;
    if (g <= gmax) {
      a.items = items;
      void *args[] = {&a};
      const hipError_t e = hipLaunchCooperativeKernel(coop_fn(idx), dim3(unsigned(g)),
                                                      dim3(kQuantThreads), args, 0, s);
      return e == hipSuccess ? NVFP4KV_OK : NVFP4KV_EHIP;
    }
  }
  // too large for one register-resident pass: amax pass + encode pass
  int cus = g_cu_count[dev] > 0 ? g_cu_count[dev] : 256;
  int g = cus * 4;
  if (g > kMaxQuantGrid) g = kMaxQuantGrid;
  hipLaunchKernelGGL(quantize_amax_kernel, dim3(g), dim3(kQuantThreads), 0, s, a);
  if (hipGetLastError() != hipSuccess) return NVFP4KV_EHIP;
  hipLaunchKernelGGL(quantize_encode_kernel, dim3(g), dim3(kQuantThreads), 0, s, a, g);
  return NVFP4KV_HIP_OK(hipGetLastError());
}

}  // namespace nvfp4kv
