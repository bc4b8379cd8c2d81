// NVFP4 quantization of K/V chunks for gfx950.
//
// Format (paper text section 2.2; reading note section II "The NVFP4
// quantization format"): 16-element blocks along head_dim, one E4M3 scale per
// block, one fp32 scale per tensor, E2M1 elements.  Recipe, in fp32 with correctly
// rounded operations: s_t = amax / 2688; bs = (block amax / 6) / s_t rounded to
// E4M3 (nearest, ties to even, saturating at 448); eff = E4M3(bs) * s_t;
// code = E2M1(|x| / eff) (nearest, ties to even, saturating at 6) with x's sign.
//
// Two kernels.  The tensor scale needs the amax of the whole chunk tensor (all
// heads) before any block can be encoded; a grid-wide barrier inside one kernel
// would need a cooperative launch, which costs far more on this GPU than the whole
// quantization, so:
//   1. quantize_amax_kernel streams K and V once and writes one partial maximum
//      per workgroup (no atomics);
//   2. quantize_encode_kernel reduces the partials, then re-reads its tiles (the
//      chunk, 28.8 MB for the 1.3B shape, is still in the 256 MB Infinity Cache)
//      and writes codes and scales.
//
// Exact encoding without an IEEE division per element.  The gfx950 converts
// v_cvt_scalef32_pk_fp4_f32 / _fp8_f32 (scale 1.0) round to nearest-even and
// saturate exactly like the recipe for every finite fp32 input (fp8 needs a clamp
// at 448, above which it returns NaN), so the code is hw_fp4(RN(x / eff)).  The
// quotient RN(x / b) is obtained from r = RN(1 / b) (one IEEE division per block)
// by Markstein's method: q0 = RN(x r) is within 1.5 ulp of x / b; one correction
// q1 = RN(q0 + (x - q0 b) r) makes it faithful; a second one, with the now exact
// remainder, q2 = RN(q1 + (x - q1 b) r), is the correctly rounded quotient
// (Markstein's theorem: y = RN(1/b) and a faithful q give RN(a/b) in one step).
// Five fp32 operations and no branches per element; the block scale's two
// divisions use the same scheme.  Quotients below 2^-126 fall out of the theorem's
// range but are far below the first E2M1 threshold (0.25), so their code is exact
// regardless; blocks whose eff leaves [2^-120, 2^110] divide each element with
// IEEE division instead.
//
// Work unit: a tile of 2 x (256 / (D/16)) token pairs x all D/16 blocks of one head
// of one frame; thread (pair p, block b) owns token pairs p and p + 256/(D/16), i.e.
// 4 tokens x 16 elements.  Tiles never
// straddle a frame, so each tile lands in one cache slot.  K (and the standalone
// codec) are written in the codec layout [h][token][D/2]; V in the cache is written
// transposed, [h][d][token/2], through LDS, so that the attention kernel can read 8
// consecutive keys of one d with one load; a tile then writes 64 contiguous bytes
// per d row.  For the transposed layout a byte holds tokens (2p, 2p+1) of one d,
// and the fp4 convert is fed exactly that pair.

#include "device_common.h"

namespace nvfp4kv {

constexpr int kAmaxThreads = 1024;

typedef short short2_ __attribute__((ext_vector_type(2)));

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

// max of the 8 |bf16| in a uint4, as two packed 16-bit halves
__device__ __forceinline__ uint32_t vmax4(uint4 u) {
  const uint32_t a = u.x & 0x7FFF7FFFu, b = u.y & 0x7FFF7FFFu;
  const uint32_t c = u.z & 0x7FFF7FFFu, d = u.w & 0x7FFF7FFFu;
  auto pmax = [](uint32_t p, uint32_t q) {
    return max(p & 0xFFFFu, q & 0xFFFFu) | (max(p >> 16, q >> 16) << 16);
  };
  return pmax(pmax(a, b), pmax(c, d));
}

// Loads the 2 x 16 bf16 of tokens (tin, tin+1) of a tile's frame, block b; returns
// block maxima of |x| as bf16 bit patterns packed (token tin in the low half).
__device__ __forceinline__ uint32_t load_item(const QuantArgs &a, const TileInfo &t, int tin,
                                              int b, uint32_t (&x)[16]) {
  const int tok = t.f * a.tokens_per_frame + tin;
  const uint16_t *src = a.t[t.tensor].src + (int64_t(t.h) * a.T + tok) * a.D + b * 16;
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = 0;
  uint4 u0 = make_uint4(0, 0, 0, 0), u1 = u0, u2 = u0, u3 = u0;
  if (tin < a.tokens_per_frame) {
    const uint4 *p = reinterpret_cast<const uint4 *>(src);
    u0 = p[0];
    u1 = p[1];
  }
  if (tin + 1 < a.tokens_per_frame) {
    const uint4 *p = reinterpret_cast<const uint4 *>(src + a.D);
    u2 = p[0];
    u3 = p[1];
  }
  x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w;
  x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
  x[8] = u2.x; x[9] = u2.y; x[10] = u2.z; x[11] = u2.w;
  x[12] = u3.x; x[13] = u3.y; x[14] = u3.z; x[15] = u3.w;
  const uint32_t m01 = vmax4(u0), m23 = vmax4(u2);
  const uint32_t mA = max(vmax4(u1) & 0xFFFFu, m01 & 0xFFFFu);
  const uint32_t mB = max(vmax4(u1) >> 16, m01 >> 16);
  const uint32_t mC = max(vmax4(u3) & 0xFFFFu, m23 & 0xFFFFu);
  const uint32_t mD = max(vmax4(u3) >> 16, m23 >> 16);
  return max(mA, mB) | (max(mC, mD) << 16);
}

// RN(x / b) from r = RN(1 / b): q0 = RN(x r), then two Markstein corrections.
__device__ __forceinline__ float div_rn(float x, float b, float r) {
  float q = x * r;
  float e = __builtin_fmaf(-q, b, x);
  q = __builtin_fmaf(e, r, q);
  e = __builtin_fmaf(-q, b, x);
  return __builtin_fmaf(e, r, q);
}

// Per-tensor constants of the encoder.
struct TensorConsts {
  float st;       // s_t
  float rst;      // RN(1 / s_t)
  bool fast;      // s_t well inside the normal range: Markstein quotients apply
};

__device__ __forceinline__ TensorConsts tensor_consts(float st) {
  TensorConsts c;
  c.st = st;
  c.fast = st >= 0x1p-120f && st <= 0x1p100f;
  c.rst = c.fast ? 1.0f / st : 0.0f;
  return c;
}

// Block scale byte and the per-element divisor of one 16-element block.
struct BlockConsts {
  uint32_t sc;    // E4M3 byte
  float eff;      // E4M3(bs) * s_t
  float r;        // RN(1 / eff); 0 when eff == 0 (codes keep only the signs)
  bool exact;     // eff outside [2^-120, 2^110]: IEEE-divide every element
};

__device__ __forceinline__ BlockConsts block_consts(uint32_t bmax_bits, const TensorConsts &tc) {
  BlockConsts bc;
  const float amax = bf16_bits_to_float(bmax_bits);
  uint32_t sc = 0;
  if (tc.st > 0.0f) {
    float bs;
    if (tc.fast) bs = div_rn(div_rn(amax, 6.0f, 1.0f / 6.0f), tc.st, tc.rst);
    else bs = (amax / 6.0f) / tc.st;
    short2_ p = {0, 0};
    p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, fminf(bs, 448.0f), 0.0f, 1.0f, false);
    sc = uint32_t(uint16_t(p[0])) & 0xFFu;
  }
  bc.sc = sc;
  bc.eff = __builtin_amdgcn_cvt_f32_fp8(sc, 0) * tc.st;
  bc.exact = bc.eff > 0.0f && (bc.eff < 0x1p-120f || bc.eff > 0x1p110f);
  bc.r = (bc.eff > 0.0f && !bc.exact) ? 1.0f / bc.eff : 0.0f;
  return bc;
}

template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// Correctly rounded signed quotient x / eff (0 with x's sign when eff == 0).  The
// corrections of div_rn can turn a zero result into +0 (+0 + -0 = +0), so the sign
// is re-applied from x: a nonzero quotient already carries it.
__device__ __forceinline__ float quot(float x, const BlockConsts &bc) {
  if (!bc.exact) return __builtin_copysignf(div_rn(x, bc.eff, bc.r), x);
  return fminf(fmaxf(x / bc.eff, -1e30f), 1e30f);
}

// Codes of 4 element pairs (xa[i], xb[i]) -> 4 bytes, pair i in byte i (a in the
// low nibble).
__device__ __forceinline__ uint32_t encode4(const float (&xa)[4], const float (&xb)[4],
                                            const BlockConsts &ba, const BlockConsts &bb) {
  uint32_t c = 0;
  c = cvt_fp4<0>(c, quot(xa[0], ba), quot(xb[0], bb));
  c = cvt_fp4<1>(c, quot(xa[1], ba), quot(xb[1], bb));
  c = cvt_fp4<2>(c, quot(xa[2], ba), quot(xb[2], bb));
  c = cvt_fp4<3>(c, quot(xa[3], ba), quot(xb[3], bb));
  return c;
}

__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Encodes and stores one item: token pair p (tokens tin, tin+1 of frame t.f) x block b.
// For the transposed layout the bytes go to s_tr[d][pair column `col`] (row stride
// `pairs` bytes) and are written out per tile by store_transposed_tile.
__device__ __forceinline__ void encode_store_item(const QuantArgs &a, const TileInfo &t, int tin,
                                                  int col, int pairs, int b,
                                                  const uint32_t (&x)[16], uint32_t bmax,
                                                  const TensorConsts &tc, uint8_t *s_tr) {
  const QuantTensor &qt = a.t[t.tensor];
  const int nb = a.D >> 4;
  const bool v0 = tin < a.tokens_per_frame, v1 = tin + 1 < a.tokens_per_frame;
  const int64_t dtok = int64_t(a.frame_slot[t.f]) * a.tokens_per_frame + tin;
  const BlockConsts b0 = block_consts(bmax & 0xFFFFu, tc);
  const BlockConsts b1 = block_consts(bmax >> 16, tc);
  if (!qt.transposed) {
    // token rows: pairs of consecutive elements of the same token
    uint32_t c[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {   // g: token (g >> 1), 8-element half (g & 1)
      const uint32_t *w = x + 4 * g;
      const float xa[4] = {lo_f(w[0]), lo_f(w[1]), lo_f(w[2]), lo_f(w[3])};
      const float xb[4] = {hi_f(w[0]), hi_f(w[1]), hi_f(w[2]), hi_f(w[3])};
      const BlockConsts &bc = (g < 2) ? b0 : b1;
      c[g] = encode4(xa, xb, bc, bc);
    }
    if (v0) {
      *reinterpret_cast<uint2 *>(qt.codes + (int64_t(t.h) * a.rows + dtok) * (a.D / 2) + b * 8) =
          make_uint2(c[0], c[1]);
      qt.scales[(int64_t(t.h) * a.rows + dtok) * nb + b] = uint8_t(b0.sc);
    }
    if (v1) {
      *reinterpret_cast<uint2 *>(qt.codes + (int64_t(t.h) * a.rows + dtok + 1) * (a.D / 2) +
                                 b * 8) = make_uint2(c[2], c[3]);
      qt.scales[(int64_t(t.h) * a.rows + dtok + 1) * nb + b] = uint8_t(b1.sc);
    }
  } else {
    // transposed: one byte per d holds (token tin, token tin+1)
#pragma unroll
    for (int g = 0; g < 4; ++g) {   // d = 4g .. 4g+3 within the block
      const uint32_t w0 = x[2 * g], w1 = x[2 * g + 1], u0 = x[8 + 2 * g], u1 = x[8 + 2 * g + 1];
      const float xa[4] = {lo_f(w0), hi_f(w0), lo_f(w1), hi_f(w1)};
      const float xb[4] = {lo_f(u0), hi_f(u0), lo_f(u1), hi_f(u1)};
      const uint32_t c = encode4(xa, xb, b0, b1);
#pragma unroll
      for (int i = 0; i < 4; ++i) s_tr[(b * 16 + 4 * g + i) * pairs + col] = uint8_t(c >> (8 * i));
    }
    if (v0) {
      *reinterpret_cast<uint16_t *>(qt.scales + (int64_t(t.h) * nb + b) * a.rows + dtok) =
          uint16_t(b0.sc | (b1.sc << 8));
    }
  }
}

// Writes one LDS-staged transposed tile ([D][pairs] bytes, pairs = tile_tokens / 2)
// to V's [h][d][rows/2] plane, 16 bytes per thread-step.
__device__ __forceinline__ void store_transposed_tile(const QuantArgs &a, const TileInfo &t,
                                                      const uint8_t *s_tr, int pairs) {
  const QuantTensor &qt = a.t[t.tensor];
  const int tok0 = t.ti * a.tile_tokens;
  int nvalid = a.tokens_per_frame - tok0;
  if (nvalid > a.tile_tokens) nvalid = a.tile_tokens;
  const int nbytes = nvalid / 2;            // multiple of 4 (T_f % 8 == 0)
  const int64_t dst0 = (int64_t(a.frame_slot[t.f]) * a.tokens_per_frame + tok0) / 2;
  const int per_row = pairs / 16;           // 16-byte pieces per d row
  for (int k = threadIdx.x; k < a.D * per_row; k += kQuantThreads) {
    const int r = k / per_row;
    const int col = (k - r * per_row) * 16;
    uint32_t *dst = reinterpret_cast<uint32_t *>(qt.codes + (int64_t(t.h) * a.D + r) * (a.rows / 2) +
                                                 dst0 + col);
    const uint32_t *src = reinterpret_cast<const uint32_t *>(s_tr + r * pairs + col);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (col + 4 * j < nbytes) dst[j] = src[j];
  }
}

// Reduces the partial maxima of an amax pass of `g` workgroups; s_st[t] = amax_t / 2688.
__device__ __forceinline__ void read_tensor_scales(const QuantArgs &a, int g, uint32_t *s_red,
                                                   float *s_st) {
  uint32_t m0 = 0, m1 = 0;
  for (int j = threadIdx.x; j < g; j += kQuantThreads) {
    m0 = max(m0, a.ws->partial[0][j]);
    m1 = max(m1, a.ws->partial[1][j]);
  }
  m0 = wave_max_u32(m0);
  m1 = wave_max_u32(m1);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_red[w] = m0;
    s_red[8 + w] = m1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r0 = 0, r1 = 0;
    for (int i = 0; i < kQuantThreads / 64; ++i) {
      r0 = max(r0, s_red[i]);
      r1 = max(r1, s_red[8 + i]);
    }
    s_st[0] = __uint_as_float(r0) / 2688.0f;
    s_st[1] = __uint_as_float(r1) / 2688.0f;
  }
  __syncthreads();
}

}  // namespace

// Pass 1: per-workgroup maxima of |x| over the flat K and V tensors (no atomics:
// each workgroup owns one slot of the partials array).  Each thread keeps up to
// 4 vectors of K and 4 of V in flight.
__global__ __launch_bounds__(kAmaxThreads) void quantize_amax_kernel(QuantArgs a) {
  __shared__ uint32_t s_red[2][kAmaxThreads / 64];
  const int64_t n16 = int64_t(a.H) * a.T * a.D / 8;   // uint4 vectors per tensor
  const int64_t stride = int64_t(gridDim.x) * kAmaxThreads;
  const uint4 *pk = reinterpret_cast<const uint4 *>(a.t[0].src);
  const uint4 *pv = reinterpret_cast<const uint4 *>(a.n_tensors > 1 ? a.t[1].src : a.t[0].src);
  const bool two = a.n_tensors > 1;
  uint32_t mk = 0, mv = 0;
  for (int64_t base = int64_t(blockIdx.x) * kAmaxThreads + threadIdx.x; base < n16;
       base += 4 * stride) {
    uint4 uk[4], uv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t i = base + j * stride;
      uk[j] = make_uint4(0, 0, 0, 0);
      uv[j] = make_uint4(0, 0, 0, 0);
      if (i < n16) {
        uk[j] = pk[i];
        if (two) uv[j] = pv[i];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t q = vmax4(uk[j]), w = vmax4(uv[j]);
      mk = max(mk, max(q & 0xFFFFu, q >> 16));
      mv = max(mv, max(w & 0xFFFFu, w >> 16));
    }
  }
  uint32_t m[2] = {wave_max_u32(mk << 16), wave_max_u32(mv << 16)};   // fp32 bit patterns
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_red[0][w] = m[0];
    s_red[1][w] = m[1];
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    uint32_t r = 0;
    for (int i = 0; i < kAmaxThreads / 64; ++i) r = max(r, s_red[threadIdx.x][i]);
    a.ws->partial[threadIdx.x][blockIdx.x] = r;
  }
}

// Pass 2: each workgroup loads a tile (2 x 256 token-pair/block items), reduces the
// pass-1 partials meanwhile, then encodes and stores.
__global__ __launch_bounds__(kQuantThreads) void quantize_encode_kernel(QuantArgs a, int g_amax) {
  __shared__ uint32_t s_red[16];
  __shared__ float s_st[2];
  __shared__ uint8_t s_tr[8192];
  const int tid = threadIdx.x;
  const int nb = a.D >> 4;
  const int TP = kQuantThreads / nb;          // token pairs per item row
  const bool act = tid < TP * nb;
  const int b = tid % nb, tp = tid / nb;
  bool first = true;
  TensorConsts tc0, tc1;
  for (int tile = blockIdx.x; tile < a.total_tiles; tile += gridDim.x) {
    const TileInfo t = decode_tile(a, tile);
    const bool tr = a.t[t.tensor].transposed != 0;
    uint32_t x[2][16];
    uint32_t bm[2] = {0u, 0u};
    const int tin0 = t.ti * a.tile_tokens + 2 * tp;
    if (act) {
      bm[0] = load_item(a, t, tin0, b, x[0]);
      bm[1] = load_item(a, t, tin0 + 2 * TP, b, x[1]);
    }
    if (first) {     // overlaps with the tile loads above
      read_tensor_scales(a, g_amax, s_red, s_st);
      if (blockIdx.x == 0 && tid < a.n_tensors) *a.t[tid].tensor_scale = s_st[tid];
      tc0 = tensor_consts(s_st[0]);
      tc1 = tensor_consts(s_st[1]);
      first = false;
    }
    if (act) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        encode_store_item(a, t, tin0 + 2 * TP * i, tp + TP * i, 2 * TP, b, x[i], bm[i],
                          t.tensor ? tc1 : tc0, s_tr);
    }
    if (tr) {
      __syncthreads();
      store_transposed_tile(a, t, s_tr, 2 * TP);
      __syncthreads();
    }
  }
}

namespace {
constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];

int cu_count(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return 256;
  if (g_cu_count[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      return 256;
    g_cu_count[dev] = cus;
  }
  return g_cu_count[dev];
}
}  // namespace

int launch_quantize(const QuantArgs &in, void *stream) {
  QuantArgs a = in;
  const int nb = a.D / 16;
  const int TP = kQuantThreads / nb;
  a.tile_tokens = 4 * TP;
  a.tiles_per_frame = (a.tokens_per_frame + a.tile_tokens - 1) / a.tile_tokens;
  const int64_t total = int64_t(a.n_tensors) * a.H * a.n_frames * a.tiles_per_frame;
  if (total >= (int64_t(1) << 31)) return NVFP4KV_EINVAL;
  a.total_tiles = int32_t(total);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4KV_EHIP;
  const int cus = cu_count(dev);
  // pass 1: one 1024-thread workgroup per CU (fewer for small inputs)
  const int64_t vecs = int64_t(a.H) * a.T * a.D / 8;
  int64_t g1 = (vecs + kAmaxThreads * 2 - 1) / (kAmaxThreads * 2);
  if (g1 > cus) g1 = cus;
  if (g1 < 1) g1 = 1;
  hipLaunchKernelGGL(quantize_amax_kernel, dim3(unsigned(g1)), dim3(kAmaxThreads), 0, s, a);
  if (hipGetLastError() != hipSuccess) return NVFP4KV_EHIP;
  // pass 2: one workgroup per tile up to 4 per CU, then a grid-stride loop
  int64_t g2 = total;
  if (g2 > int64_t(cus) * 4) g2 = int64_t(cus) * 4;
  hipLaunchKernelGGL(quantize_encode_kernel, dim3(unsigned(g2)), dim3(kQuantThreads), 0, s, a,
                     int(g1));
  return NVFP4KV_HIP_OK(hipGetLastError());
}

}  // namespace nvfp4kv
