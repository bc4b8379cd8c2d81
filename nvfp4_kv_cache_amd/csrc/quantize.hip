// NVFP4 quantization of K/V chunks for gfx950.
//
// Format (paper text section 2.2; reading note section II "The NVFP4
// quantization format"): 16-element blocks along head_dim, one E4M3 scale per
// block, one fp32 scale per tensor, E2M1 elements.  Recipe, in fp32 with correctly
// rounded operations: s_t = amax / 2688; bs = (block amax / 6) / s_t rounded to
// E4M3 (nearest, ties to even, saturating at 448); eff = E4M3(bs) * s_t;
// code = E2M1(|x| / eff) (nearest, ties to even, saturating at 6) with x's sign.
//
// Two schedules.  The tensor scale needs the amax of the whole chunk tensor (all
// heads) before any block can be encoded.
//   * Cache appends (quantize_fused_kernel, one pass): every workgroup of a grid
//     that is resident all at once (the launcher checks the occupancy) loads its
//     tile into registers, publishes its maxima in an epoch-tagged workspace slot,
//     waits (bounded) for every slot of the launch and encodes from the registers,
//     so the chunk is read once.  No cooperative launch is needed.
//   * The standalone codec, and appends with K-smoothing or adaptive V scales,
//     whose workspace cannot carry epochs or which need the channel means first:
//     quantize_amax_kernel streams K and V once and writes one partial maximum per
//     workgroup (no atomics); quantize_encode_kernel reduces the partials, then
//     re-reads its tiles (the chunk, 28.8 MB for the 1.3B shape, is still in the
//     256 MB Infinity Cache) and writes codes and scales.
//
// Exact encoding without an IEEE division per element.  The gfx950 converts
// v_cvt_scalef32_pk_fp4_f32 / _fp8_f32 (scale 1.0) round to nearest-even and
// saturate exactly like the recipe for every finite fp32 input (fp8 needs a clamp
// at 448, above which it returns NaN), so the code is hw_fp4(RN(x / eff)).  The
// quotient RN(x / eff) is obtained from r = RN(1 / eff) (one IEEE division per
// scale code and tensor, in an LDS table) by Markstein's method: q0 = RN(x r), then
// corrections q' = RN(q - (q eff - x) r) with the remainder from one fused
// multiply-add.  For a bf16 x one correction already gives RN(x / eff) whenever the
// remainder is exact (div_rn_bf16: three fp32 operations per element); K minus its
// channel means takes two (div_rn), as do the block scale's two divisions.  Tensors
// whose s_t leaves [2^-80, 2^100] move x and eff by one power of two first, which
// keeps every quotient that can give a nonzero code in that exact range.
//
// Work unit: an item is one octet of consecutive tokens x one 16-element block
// (8 x 32 bytes of bf16), one item per thread; a workgroup tile is 256 / (D/16)
// octets x all D/16 blocks of one head.  Lanes run over blocks fastest, so a
// token's D values are read by neighbouring lanes.  Tiles run over the chunk's
// tokens regardless of frames: the destination row of each octet comes from its
// own frame's cache slot (cache frames hold a multiple of 8 tokens, so an octet
// never straddles two frames).  K (and the standalone codec) are written in the
// codec layout [h][token][D/2]; V in the cache is written transposed,
// [h][d][token/2], so that the attention kernel reads 8 consecutive keys of one d
// with one load: an item then owns one 4-byte word (its 8 tokens) of 16 d rows,
// and each byte holds tokens (2i, 2i+1) of one d, which is exactly the pair the
// fp4 convert is fed.  Tokens are processed pair by pair in load order, so a wave
// starts encoding as soon as its first loads arrive.

#include "device_common.h"

namespace nvfp4kv {

constexpr int kAmaxThreads = 1024;
constexpr int kOctet = 8;           // tokens per item
constexpr int kScaleCodes = 128;    // E4M3 bytes 0x00..0x7F (0x7E is the largest produced)

typedef short short2_ __attribute__((ext_vector_type(2)));

namespace {

// max of the 8 |bf16| in a uint4, as two packed 16-bit halves
__device__ __forceinline__ uint32_t vmax4(uint4 u) {
  const uint32_t a = u.x & 0x7FFF7FFFu, b = u.y & 0x7FFF7FFFu;
  const uint32_t c = u.z & 0x7FFF7FFFu, d = u.w & 0x7FFF7FFFu;
  auto pmax = [](uint32_t p, uint32_t q) {
    return max(p & 0xFFFFu, q & 0xFFFFu) | (max(p >> 16, q >> 16) << 16);
  };
  return pmax(pmax(a, b), pmax(c, d));
}

// RN(x / b) from r = RN(1 / b): q0 = RN(x r), then two Markstein corrections.  The
// remainder is formed negated (q b - x) and subtracted, which leaves every nonzero
// result unchanged and keeps the sign of a zero quotient equal to x's (an added
// remainder would turn -0 into +0).
__device__ __forceinline__ float div_rn(float x, float b, float r) {
  float q = x * r;
  float e = __builtin_fmaf(q, b, -x);
  q = __builtin_fmaf(-e, r, q);
  e = __builtin_fmaf(q, b, -x);
  return __builtin_fmaf(-e, r, q);
}

// The same with ONE correction, for bf16 numerators: then it is already RN(x / b)
// whenever the remainder q0 b - x is computed exactly.  This was checked
// exhaustively: every bf16 significand against every fp32 significand (2^7 x 2^23
// pairs; a power-of-two change of x or b scales every step exactly, so the pairs
// cover every exponent pair with an exact remainder and a normal quotient).  The
// remainder is a multiple of about 2^-47 x, so it is exact for x >= 2^-102; below
// that its rounding can move a quotient that lies next to a rounding boundary.  The
// encoder keeps every quotient that matters in that range (see extreme_rescale).
__device__ __forceinline__ float div_rn_bf16(float x, float b, float r) {
  const float q = x * r;
  const float e = __builtin_fmaf(q, b, -x);
  return __builtin_fmaf(-e, r, q);
}

// Per-tensor constants of the encoder.
struct TensorConsts {
  float st;       // s_t
  float rst;      // RN(1 / s_t), 0 when s_t == 0
  float amin;     // block maxima below this take IEEE divisions for the scale byte
  float xs;       // 2^K applied to x and eff alike when s_t is extreme, else 1
};

// Power of two that brings s_t near 2^-10 when s_t leaves [2^-80, 2^100]: x / eff
// is unchanged when both are scaled by it, and all the scaled operands stay normal.
// Inside the range eff >= 2^-9 s_t >= 2^-89, so every quotient that can round to a
// nonzero code (x / eff > 1/4) has x > 2^-91, where the one-correction quotient is
// exact; a smaller quotient gives code 0 however it is rounded.
__device__ __forceinline__ float extreme_rescale(float st) {
  if (!(st > 0.0f) || (st >= 0x1p-80f && st <= 0x1p100f)) return 1.0f;
  const int e = st < 0x1p-126f ? -127 : int((__float_as_uint(st) >> 23) & 0xFF) - 127;
  return __builtin_ldexpf(1.0f, -10 - e);
}

// Markstein quotients for the scale byte need s_t well inside the normal range and
// amax / 6 far enough above it for the remainders to stay normal.  An all-zero
// tensor (s_t == 0) takes them too: every block maximum is 0 and gives bs = 0.
__device__ __forceinline__ TensorConsts tensor_consts(float st) {
  TensorConsts c;
  c.st = st;
  const bool fast = st >= 0x1p-120f && st <= 0x1p100f;
  c.rst = fast ? 1.0f / st : 0.0f;
  c.amin = fast ? 0x1p-90f : (st == 0.0f ? 0.0f : __builtin_inff());
  c.xs = extreme_rescale(st);
  return c;
}

// E4M3 scale byte of one block: bs = (amax / M) / s_t, nearest-even, saturating;
// M = 6 is the recipe, M = 4 the second candidate of the adaptive block scale.
// Markstein quotients when both are comfortably normal; IEEE division otherwise.
template <int M = 6>
__device__ __forceinline__ uint32_t scale_code(float amax, const TensorConsts &tc) {
  float bs;
  if (amax >= tc.amin) bs = div_rn(div_rn(amax, float(M), 1.0f / float(M)), tc.st, tc.rst);
  else bs = (amax / float(M)) / tc.st;
  short2_ p = {0, 0};
  p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, fminf(bs, 448.0f), 0.0f, 1.0f, false);
  return uint32_t(uint16_t(p[0])) & 0xFFu;
}

// Divisor entry of one scale byte: eff = E4M3(sc) * s_t (rounded as fp32, subnormals
// included), then scaled by xs, and r = RN(1 / eff); r = 0 when eff == 0 (codes keep
// only the signs).
__device__ __forceinline__ float2 divisor_entry(uint32_t sc, float st, float xs) {
  const float eff = (__builtin_amdgcn_cvt_f32_fp8(sc, 0) * st) * xs;
  return make_float2(eff, eff > 0.0f ? 1.0f / eff : 0.0f);
}

// BF16: x is a bf16 value (8 significant bits); otherwise any fp32 (K minus its
// channel means).
template <bool SCALED, bool BF16 = true>
__device__ __forceinline__ float quot(float x, float eff, float r, float xs) {
  if constexpr (BF16) return div_rn_bf16(SCALED ? x * xs : x, eff, r);
  else return div_rn(SCALED ? x * xs : x, eff, r);
}

// One token's 16 bf16 of a block as fp32 (exact), element order.
__device__ __forceinline__ void unpack16(const uint4 (&u)[2], float (&x)[16]) {
  const uint32_t w[8] = {u[0].x, u[0].y, u[0].z, u[0].w, u[1].x, u[1].y, u[1].z, u[1].w};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    x[2 * k] = __uint_as_float(w[k] << 16);
    x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
  }
}

// bf16 bits of max |x| over one token's 16 values (finite inputs: the order of the
// magnitude bits is the order of the values), on packed 16-bit maxima.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t block_max_bits(const uint4 (&u)[2]) {
  auto m = [](uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                   __builtin_bit_cast(u16x2, b)));
  };
  const uint32_t k = 0x7FFF7FFFu;
  const uint32_t r = m(m(m(u[0].x & k, u[0].y & k), m(u[0].z & k, u[0].w & k)),
                       m(m(u[1].x & k, u[1].y & k), m(u[1].z & k, u[1].w & k)));
  return max(r & 0xFFFFu, r >> 16);
}

__device__ __forceinline__ float absmax16(const float (&x)[16]) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i += 2) m = fmaxf(m, fmaxf(fabsf(x[i]), fabsf(x[i + 1])));
  return m;
}

template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// Adaptive block scale (V in the cache): squared error of encoding one token's
// block with scale byte sc, sum over the 16 elements in order of
// (|x| - value * eff)^2 with eff = E4M3(sc) * s_t, every step an fp32 operation
// (no contraction: the choice must match the recipe bit for bit).
template <bool SCALED>
__device__ __forceinline__ float block_sq_error(const float (&x)[16], uint32_t sc, const TensorConsts &tc,
                                                const float2 *tab) {
#pragma clang fp contract(off)
  const float2 dv = tab[sc];
  const float eff = __builtin_amdgcn_cvt_f32_fp8(sc, 0) * tc.st;
  float err = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    const uint32_t c = cvt_fp4<0>(0u, quot<SCALED>(x[i], dv.x, dv.y, tc.xs),
                                  quot<SCALED>(x[i + 1], dv.x, dv.y, tc.xs));
    const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
    const float da = fabsf(x[i]) - fabsf(v[0]) * eff;
    err = err + da * da;
    const float db = fabsf(x[i + 1]) - fabsf(v[1]) * eff;
    err = err + db * db;
  }
  return err;
}

// The 4-candidate wins only with a strictly smaller error (ties keep 6).
template <bool SCALED>
__device__ __forceinline__ uint32_t choose_scale46(const float (&x)[16], float amax, uint32_t sc6,
                                                   const TensorConsts &tc, const float2 *tab) {
  const uint32_t sc4 = scale_code<4>(amax, tc);
  if (sc4 == sc6) return sc6;
  return block_sq_error<SCALED>(x, sc4, tc, tab) < block_sq_error<SCALED>(x, sc6, tc, tab) ? sc4 : sc6;
}

// Codec layout: one token's 16 values -> 8 bytes (element 2k in the low nibble).
template <bool SCALED, bool BF16 = true>
__device__ __forceinline__ uint2 encode_token(const float (&x)[16], float eff, float r, float xs) {
  uint32_t c[2] = {0u, 0u};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float *y = x + 8 * h;
    c[h] = cvt_fp4<0>(c[h], quot<SCALED, BF16>(y[0], eff, r, xs), quot<SCALED, BF16>(y[1], eff, r, xs));
    c[h] = cvt_fp4<1>(c[h], quot<SCALED, BF16>(y[2], eff, r, xs), quot<SCALED, BF16>(y[3], eff, r, xs));
    c[h] = cvt_fp4<2>(c[h], quot<SCALED, BF16>(y[4], eff, r, xs), quot<SCALED, BF16>(y[5], eff, r, xs));
    c[h] = cvt_fp4<3>(c[h], quot<SCALED, BF16>(y[6], eff, r, xs), quot<SCALED, BF16>(y[7], eff, r, xs));
  }
  return make_uint2(c[0], c[1]);
}

// Transposed layout: tokens (2*SEL, 2*SEL+1) of the octet fill byte SEL of each of
// the 16 per-d words.
template <int SEL, bool SCALED>
__device__ __forceinline__ void encode_pair_transposed(const float (&xa)[16], const float (&xb)[16],
                                                       float effa, float ra, float effb, float rb,
                                                       float xs, uint32_t (&out)[16]) {
#pragma unroll
  for (int d = 0; d < 16; ++d)
    out[d] = cvt_fp4<SEL>(out[d], quot<SCALED>(xa[d], effa, ra, xs), quot<SCALED>(xb[d], effb, rb, xs));
}

struct Octet {
  int tensor, h, tok;       // source token of the octet's first token
  int64_t row;              // destination row of that token
  int nvalid;               // tokens of the octet inside the chunk (0..8)
};

// Canonical item: per token, block max -> scale byte -> divisor -> 8 code bytes.
// MEAN: K-smoothing, the block's 16 channel means are subtracted first (fp32).
// bmax (optional): the tokens' block maxima as bf16 bits, taken before s_t was known.
template <bool SCALED, bool MEAN = false>
__device__ __forceinline__ void item_canonical(const QuantArgs &a, const Octet &o, int b,
                                               const uint4 (&u)[kOctet][2],
                                               const TensorConsts &tc, const float2 *tab,
                                               const uint32_t *bmax = nullptr) {
  const QuantTensor &qt = a.t[o.tensor];
  const int nb = a.D >> 4;
  float mu[16];
  if constexpr (MEAN) {
    const float4 *mp = reinterpret_cast<const float4 *>(qt.mean + int64_t(o.h) * a.D + 16 * b);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 m4 = mp[k];
      mu[4 * k] = m4.x;
      mu[4 * k + 1] = m4.y;
      mu[4 * k + 2] = m4.z;
      mu[4 * k + 3] = m4.w;
    }
  }
  // with the maxima at hand, every scale byte and divisor first (their table reads
  // overlap), then the codes
  uint32_t scp[kOctet];
  float2 dvp[kOctet];
  if (bmax) {
#pragma unroll
    for (int j = 0; j < kOctet; ++j) scp[j] = scale_code(__uint_as_float(bmax[j] << 16), tc);
#pragma unroll
    for (int j = 0; j < kOctet; ++j) dvp[j] = tab[scp[j]];
  }
#pragma unroll
  for (int j = 0; j < kOctet; ++j) {
    float x[16];
    unpack16(u[j], x);
    if constexpr (MEAN) {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = x[i] - mu[i];
    }
    const uint32_t sc = bmax ? scp[j] : scale_code(absmax16(x), tc);
    const float2 dv = bmax ? dvp[j] : tab[sc];
    const uint2 c = encode_token<SCALED, !MEAN>(x, dv.x, dv.y, tc.xs);
    if (j < o.nvalid) {
      const int64_t row = int64_t(o.h) * a.rows + o.row + j;
      *reinterpret_cast<uint2 *>(qt.codes + row * (a.D / 2) + b * 8) = c;
      qt.scales[row * nb + b] = uint8_t(sc);
    }
  }
}

// Transposed item (V in the cache; full octets only): 16 words of 8 tokens, one per
// d of the block, and the octet's 8 scale bytes of this block.  Token pairs are
// taken in load order: scale bytes and divisors of a pair right before its codes.
template <bool SCALED, bool ADAPT = false>
__device__ __forceinline__ void item_transposed(const QuantArgs &a, const Octet &o, int b,
                                                const uint4 (&u)[kOctet][2],
                                                const TensorConsts &tc, const float2 *tab,
                                                const uint32_t *bmax = nullptr) {
  const QuantTensor &qt = a.t[o.tensor];
  const int nb = a.D >> 4;
  uint32_t sc[kOctet];
  uint32_t out[16];
#pragma unroll
  for (int d = 0; d < 16; ++d) out[d] = 0u;
  // with the maxima at hand (no adaptive choice), every scale byte and divisor first
  float2 dvp[kOctet];
  const bool pre = bmax && !ADAPT;
  if (pre) {
#pragma unroll
    for (int j = 0; j < kOctet; ++j) sc[j] = scale_code(__uint_as_float(bmax[j] << 16), tc);
#pragma unroll
    for (int j = 0; j < kOctet; ++j) dvp[j] = tab[sc[j]];
  }
#define NVFP4KV_PAIR(SEL)                                                             \
  {                                                                                   \
    float xa[16], xb[16];                                                             \
    unpack16(u[2 * SEL], xa);                                                         \
    unpack16(u[2 * SEL + 1], xb);                                                     \
    float2 da, db;                                                                    \
    if (pre) {                                                                        \
      da = dvp[2 * SEL];                                                              \
      db = dvp[2 * SEL + 1];                                                          \
    } else {                                                                          \
      const float ma = bmax ? __uint_as_float(bmax[2 * SEL] << 16) : absmax16(xa);    \
      const float mb = bmax ? __uint_as_float(bmax[2 * SEL + 1] << 16) : absmax16(xb); \
      sc[2 * SEL] = scale_code(ma, tc);                                               \
      sc[2 * SEL + 1] = scale_code(mb, tc);                                           \
      if constexpr (ADAPT) {                                                          \
        sc[2 * SEL] = choose_scale46<SCALED>(xa, ma, sc[2 * SEL], tc, tab);           \
        sc[2 * SEL + 1] = choose_scale46<SCALED>(xb, mb, sc[2 * SEL + 1], tc, tab);   \
      }                                                                               \
      da = tab[sc[2 * SEL]];                                                          \
      db = tab[sc[2 * SEL + 1]];                                                      \
    }                                                                                 \
    encode_pair_transposed<SEL, SCALED>(xa, xb, da.x, da.y, db.x, db.y, tc.xs, out);  \
  }
  NVFP4KV_PAIR(0)
  NVFP4KV_PAIR(1)
  NVFP4KV_PAIR(2)
  NVFP4KV_PAIR(3)
#undef NVFP4KV_PAIR
  if (o.nvalid == kOctet) {
    uint8_t *dst = qt.codes + (int64_t(o.h) * a.D + 16 * b) * (a.rows / 2) + o.row / 2;
#pragma unroll
    for (int d = 0; d < 16; ++d) *reinterpret_cast<uint32_t *>(dst + d * (a.rows / 2)) = out[d];
    *reinterpret_cast<uint2 *>(qt.scales + (int64_t(o.h) * nb + b) * a.rows + o.row) =
        make_uint2(sc[0] | (sc[1] << 8) | (sc[2] << 16) | (sc[3] << 24),
                   sc[4] | (sc[5] << 8) | (sc[6] << 16) | (sc[7] << 24));
  }
}

__device__ __forceinline__ Octet locate_octet(const QuantArgs &a, int tile, int o) {
  Octet r;
  r.tensor = tile / (a.H * a.tiles_per_head);
  const int rem = tile - r.tensor * a.H * a.tiles_per_head;
  r.h = rem / a.tiles_per_head;
  r.tok = (rem - r.h * a.tiles_per_head) * a.tile_tokens + kOctet * o;
  r.nvalid = min(max(a.T - r.tok, 0), kOctet);
  const int f = min(r.tok / a.tokens_per_frame, a.n_frames - 1);
  r.row = int64_t(a.frame_slot[f]) * a.tokens_per_frame + (r.tok - f * a.tokens_per_frame);
  return r;
}

// Loads the octet's 8 x 16 values; tokens past the chunk end re-read its last
// token (their results are not stored), so every load is unconditional.
__device__ __forceinline__ void load_octet(const QuantArgs &a, const Octet &o, int b,
                                           uint4 (&u)[kOctet][2]) {
  const uint4 *src = reinterpret_cast<const uint4 *>(a.t[o.tensor].src + int64_t(o.h) * a.T * a.D +
                                                     16 * b);
  const int stride = a.D / 8;    // uint4 per token
#pragma unroll
  for (int j = 0; j < kOctet; ++j) {
    const int64_t tok = min(o.tok + j, a.T - 1);
    u[j][0] = src[tok * stride];
    u[j][1] = src[tok * stride + 1];
  }
}

}  // namespace

// Pass 1: per-workgroup maxima of |x| over the flat K and V tensors (no atomics:
// each workgroup owns one slot of the partials array), as fp32 bit patterns.  Each
// thread keeps up to 4 vectors of K and 4 of V in flight.  With K-smoothing the K
// maximum is taken over x - mean (fp32), the mean of each element's channel.
__global__ __launch_bounds__(kAmaxThreads) void quantize_amax_kernel(QuantArgs a) {
  __shared__ uint32_t s_red[2][kAmaxThreads / 64];
  const int64_t n16 = int64_t(a.H) * a.T * a.D / 8;   // uint4 vectors per tensor
  const int64_t stride = int64_t(gridDim.x) * kAmaxThreads;
  const uint4 *pk = reinterpret_cast<const uint4 *>(a.t[0].src);
  const uint4 *pv = reinterpret_cast<const uint4 *>(a.n_tensors > 1 ? a.t[1].src : a.t[0].src);
  const bool two = a.n_tensors > 1;
  const float *kmean = a.t[0].mean;
  const int64_t head_vecs = int64_t(a.T) * a.D / 8;
  uint32_t mk = 0, mv = 0;   // fp32 bit patterns of |x|
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
      const int64_t i = base + j * stride;
      if (kmean) {
        if (i < n16) {
          const int64_t hh = i / head_vecs;
          const int d0 = int((i - hh * head_vecs) % (a.D / 8)) * 8;
          const float4 *mp = reinterpret_cast<const float4 *>(kmean + hh * a.D + d0);
          const float4 m0 = mp[0], m1 = mp[1];
          const float mu[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
          const uint32_t w[4] = {uk[j].x, uk[j].y, uk[j].z, uk[j].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = __uint_as_float(e & 1 ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
            mk = max(mk, __float_as_uint(x - mu[e]) & 0x7FFFFFFFu);
          }
        }
      } else {
        const uint32_t q = vmax4(uk[j]);
        mk = max(mk, max(q & 0xFFFFu, q >> 16) << 16);
      }
      const uint32_t w = vmax4(uv[j]);
      mv = max(mv, max(w & 0xFFFFu, w >> 16) << 16);
    }
  }
  uint32_t m[2] = {wave_max_u32(mk), wave_max_u32(mv)};
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

// Pass 2: every workgroup loads the pass-1 partials first, then its first tile; it
// reduces the partials to s_t and fills a per-tensor table of divisors (eff, 1/eff
// for each of the 128 scale bytes) while the tile is in flight, then encodes.
__global__ __launch_bounds__(kQuantThreads) void quantize_encode_kernel(QuantArgs a, int g_amax) {
  __shared__ uint32_t s_red[2][kQuantThreads / 64];
  __shared__ float s_st[2];
  __shared__ float2 s_tab[2][kScaleCodes];
  const int tid = threadIdx.x;
  const int nb = a.D >> 4;
  const int opt = kQuantThreads / nb;         // octets per tile
  const bool act = tid < opt * nb;
  const int b = tid % nb, o = tid / nb;

  // g_amax <= kQuantThreads: one partial per thread, duplicates are harmless
  const int pj = min(tid, g_amax - 1);
  uint32_t m0 = a.ws->partial[0][pj];
  uint32_t m1 = a.ws->partial[1][pj];
  int tile = blockIdx.x;
  uint4 u[kOctet][2];
  Octet oc = locate_octet(a, min(tile, a.total_tiles - 1), min(o, opt - 1));
  load_octet(a, oc, b, u);

  m0 = wave_max_u32(m0);
  m1 = wave_max_u32(m1);
  if ((tid & 63) == 0) {
    s_red[0][tid >> 6] = m0;
    s_red[1][tid >> 6] = m1;
  }
  __syncthreads();
  if (tid < 2) {
    uint32_t r = 0;
    for (int i = 0; i < kQuantThreads / 64; ++i) r = max(r, s_red[tid][i]);
    s_st[tid] = __uint_as_float(r) / 2688.0f;
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid < a.n_tensors) *a.t[tid].tensor_scale = s_st[tid];
  const TensorConsts tc0 = tensor_consts(s_st[0]), tc1 = tensor_consts(s_st[1]);
  for (int e = tid; e < 2 * kScaleCodes; e += kQuantThreads) {
    const int t = e / kScaleCodes;
    s_tab[t][e % kScaleCodes] = divisor_entry(e % kScaleCodes, s_st[t], t ? tc1.xs : tc0.xs);
  }
  __syncthreads();

  while (tile < a.total_tiles) {
    if (act) {
      const TensorConsts &tc = oc.tensor ? tc1 : tc0;
      const float2 *tab = s_tab[oc.tensor];
      const QuantTensor &qt = a.t[oc.tensor];
      const bool tr = qt.transposed != 0;
      if (tc.xs == 1.0f) {
        if (tr) {
          if (qt.adaptive) item_transposed<false, true>(a, oc, b, u, tc, tab);
          else item_transposed<false>(a, oc, b, u, tc, tab);
        } else {
          if (qt.mean) item_canonical<false, true>(a, oc, b, u, tc, tab);
          else item_canonical<false>(a, oc, b, u, tc, tab);
        }
      } else {
        if (tr) {
          if (qt.adaptive) item_transposed<true, true>(a, oc, b, u, tc, tab);
          else item_transposed<true>(a, oc, b, u, tc, tab);
        } else {
          if (qt.mean) item_canonical<true, true>(a, oc, b, u, tc, tab);
          else item_canonical<true>(a, oc, b, u, tc, tab);
        }
      }
    }
    tile += gridDim.x;
    if (tile < a.total_tiles) {
      oc = locate_octet(a, tile, min(o, opt - 1));
      load_octet(a, oc, b, u);
    }
  }
}

// Single pass (cache appends): every workgroup loads its tile into registers,
// publishes its maxima of |x| in its workspace slot tagged with the launch's epoch,
// waits until every workgroup's slot carries that epoch, and encodes from the
// registers, so the chunk is read once.  All workgroups of the grid must be
// resident at the same time (the launcher checks the grid against the occupancy).
// The wait is bounded (a.spin_limit polls): a workgroup that gives up scans the whole
// tensors for their maxima itself, which gives the same result, so no workgroup can
// wait forever.

__device__ __forceinline__ void tensor_max_scan(const QuantArgs &a, uint32_t &mk, uint32_t &mv) {
  const int64_t n16 = int64_t(a.H) * a.T * a.D / 8;
  const uint4 *pk = reinterpret_cast<const uint4 *>(a.t[0].src);
  const uint4 *pv = reinterpret_cast<const uint4 *>(a.n_tensors > 1 ? a.t[1].src : a.t[0].src);
  for (int64_t i = threadIdx.x; i < n16; i += kQuantThreads) {
    const uint32_t q = vmax4(pk[i]), w = vmax4(pv[i]);
    mk = max(mk, max(q & 0xFFFFu, q >> 16));
    mv = max(mv, max(w & 0xFFFFu, w >> 16));
  }
}

__global__ __launch_bounds__(kQuantThreads) void quantize_fused_kernel(QuantArgs a) {
  __shared__ uint32_t s_red[2][kQuantThreads / 64];
  __shared__ int s_ok[kQuantThreads / 64];
  __shared__ float s_st[2];
  __shared__ float2 s_tab[2][kScaleCodes];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nb = a.D >> 4;
  const int opt = kQuantThreads / nb;         // octets per tile
  const bool act = tid < opt * nb;
  const int b = tid % nb, o = tid / nb;

  // the tile (tokens past the end re-read the last token: part of the tensor)
  uint4 u[kOctet][2];
  const Octet oc = locate_octet(a, blockIdx.x, min(o, opt - 1));
  load_octet(a, oc, b, u);
  // the tokens' block maxima (needed by the encode, known before s_t)
  uint32_t bm[kOctet], mx = 0;
#pragma unroll
  for (int j = 0; j < kOctet; ++j) {
    bm[j] = block_max_bits(u[j]);
    mx = max(mx, bm[j]);
  }
  uint32_t mk = wave_max_u32(oc.tensor == 0 ? mx : 0u);
  uint32_t mv = wave_max_u32(oc.tensor == 1 ? mx : 0u);
  if (lane == 0) {
    s_red[0][wv] = mk;
    s_red[1][wv] = mv;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t rk = 0, rv = 0;
    for (int i = 0; i < kQuantThreads / 64; ++i) {
      rk = max(rk, s_red[0][i]);
      rv = max(rv, s_red[1][i]);
    }
    const uint64_t word = (a.epoch << 30) | (uint64_t(rk) << 15) | uint64_t(rv);
    __hip_atomic_store(&a.ws->slot[blockIdx.x], word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();

  // wait for the slots of every workgroup of this launch
  uint32_t gk = 0, gv = 0;
  for (int spin = 0;; ++spin) {
    bool ok = true;
    uint32_t k = 0, v = 0;
    for (int j = tid; j < int(gridDim.x); j += kQuantThreads) {
      const uint64_t w = __hip_atomic_load(&a.ws->slot[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ok = ok && (w >> 30) == a.epoch;
      k = max(k, uint32_t(w >> 15) & 0x7FFFu);
      v = max(v, uint32_t(w) & 0x7FFFu);
    }
    const int wave_ok = __all(ok);
    k = wave_max_u32(k);
    v = wave_max_u32(v);
    if (lane == 0) {
      s_ok[wv] = wave_ok;
      s_red[0][wv] = k;
      s_red[1][wv] = v;
    }
    __syncthreads();
    bool all_ok = true;
    gk = gv = 0;
    for (int i = 0; i < kQuantThreads / 64; ++i) {
      all_ok = all_ok && s_ok[i];
      gk = max(gk, s_red[0][i]);
      gv = max(gv, s_red[1][i]);
    }
    __syncthreads();
    if (all_ok) break;
    if (spin >= a.spin_limit) {   // give up waiting: scan the tensors
      uint32_t fk = 0, fv = 0;
      tensor_max_scan(a, fk, fv);
      fk = wave_max_u32(fk);
      fv = wave_max_u32(fv);
      if (lane == 0) {
        s_red[0][wv] = fk;
        s_red[1][wv] = fv;
      }
      __syncthreads();
      gk = gv = 0;
      for (int i = 0; i < kQuantThreads / 64; ++i) {
        gk = max(gk, s_red[0][i]);
        gv = max(gv, s_red[1][i]);
      }
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }

  const float st0 = bf16_bits_to_float(gk) / 2688.0f, st1 = bf16_bits_to_float(gv) / 2688.0f;
  if (blockIdx.x == 0 && tid == 0) {
    *a.t[0].tensor_scale = st0;
    if (a.n_tensors > 1) *a.t[1].tensor_scale = st1;
  }
  const TensorConsts tc0 = tensor_consts(st0), tc1 = tensor_consts(st1);
  for (int e = tid; e < 2 * kScaleCodes; e += kQuantThreads) {
    const int t = e / kScaleCodes;
    s_tab[t][e % kScaleCodes] = divisor_entry(e % kScaleCodes, t ? st1 : st0, t ? tc1.xs : tc0.xs);
  }
  __syncthreads();
  if (act) {
    const TensorConsts &tc = oc.tensor ? tc1 : tc0;
    const float2 *tab = s_tab[oc.tensor];
    const bool tr = a.t[oc.tensor].transposed != 0;
    if (tc.xs == 1.0f) {
      if (tr) item_transposed<false>(a, oc, b, u, tc, tab, bm);
      else item_canonical<false>(a, oc, b, u, tc, tab, bm);
    } else {
      if (tr) item_transposed<true>(a, oc, b, u, tc, tab, bm);
      else item_canonical<true>(a, oc, b, u, tc, tab, bm);
    }
  }
}

// MXFP4 (paper text, appendix A.2 "FP4 Quantization", and the OCP Microscaling
// Formats (MX) specification v1.0 it cites): blocks of 32 along head_dim, each with a
// power-of-two scale 2^E stored as the E8M0 byte E + 127, E = floor(log2(block max))
// - 2 clamped to [-127, 127] (-127 for an all-zero block); element code =
// E2M1(x * 2^-E) nearest-even, saturating at 6.  No tensor scale: every block is
// encoded on its own, so one pass reads the chunk once with no grid-wide step.
//
// The items are those of the NVFP4 kernels (an octet of tokens x one 16-element
// half of an MX block); the two halves of a block are neighbouring lanes (lanes run
// over 16-element blocks fastest and D/16 is even), which exchange their maxima with
// one DPP move.  The scaling by 2^-E is exact (2^-E is a normal fp32 and the product
// can only lose bits far below the first E2M1 threshold 0.25), and the convert
// rounds to nearest-even and saturates like the recipe.

// E8M0 exponent E of a block whose largest |x| has the bf16 bit pattern m (sign
// cleared): floor(log2) from the exponent field, or from the mantissa's leading bit
// for a subnormal; -2; clamped.
__device__ __forceinline__ int mx_exponent(uint32_t m) {
  const int ef = int(m >> 7);
  const int fl = ef > 0 ? ef - 127 : -133 + (31 - __builtin_clz(m | 1u));
  return m == 0 ? -127 : max(-127, min(127, fl - 2));
}

// the largest |x| bits of the lane's 16 values of token j, combined with the other
// half of the block (lane ^ 1)
__device__ __forceinline__ uint32_t mx_block_max(const uint4 (&u)[2]) {
  const uint32_t p = vmax4(u[0]), q = vmax4(u[1]);
  const uint32_t m = max(max(p & 0xFFFFu, p >> 16), max(q & 0xFFFFu, q >> 16));
  // quad_perm [1, 0, 3, 2]: the neighbouring lane's value
  const uint32_t o = uint32_t(__builtin_amdgcn_mov_dpp(int(m), 0xB1, 0xF, 0xF, false));
  return max(m, o);
}

__device__ __forceinline__ float pow2_neg(int e) { return __uint_as_float(uint32_t(127 - e) << 23); }

__global__ __launch_bounds__(kQuantThreads) void quantize_mx_kernel(QuantArgs a) {
  const int tid = threadIdx.x;
  const int nb = a.D >> 4;
  const int opt = kQuantThreads / nb;
  const int b = tid % nb, o = tid / nb;
  for (int tile = blockIdx.x; tile < a.total_tiles; tile += gridDim.x) {
    // threads past the tile's octets (when D/16 does not divide the workgroup) redo
    // its last octet, without storing: every lane takes part in the maxima exchange
    const Octet oc = locate_octet(a, tile, min(o, opt - 1));
    uint4 u[kOctet][2];
    load_octet(a, oc, b, u);
    const QuantTensor &qt = a.t[oc.tensor];
    const int nmx = a.D >> 5;                 // MX blocks per token
    const bool lead = (b & 1) == 0;           // writes the block's scale byte(s)
    if (qt.transposed) {
      // V in the cache: 16 words of 8 tokens (one per d of this half block) and, from
      // the lead lane, the octet's 8 scale bytes of the MX block
      uint32_t out[16];
      uint32_t sb[kOctet];
#pragma unroll
      for (int d = 0; d < 16; ++d) out[d] = 0u;
#define NVFP4KV_MX_PAIR(SEL)                                                           \
  {                                                                                    \
    const int ea = mx_exponent(mx_block_max(u[2 * SEL]));                              \
    const int eb = mx_exponent(mx_block_max(u[2 * SEL + 1]));                          \
    sb[2 * SEL] = uint32_t(ea + 127);                                                  \
    sb[2 * SEL + 1] = uint32_t(eb + 127);                                              \
    float xa[16], xb[16];                                                              \
    unpack16(u[2 * SEL], xa);                                                          \
    unpack16(u[2 * SEL + 1], xb);                                                      \
    const float ia = pow2_neg(ea), ib = pow2_neg(eb);                                  \
    _Pragma("unroll") for (int d = 0; d < 16; ++d) out[d] = cvt_fp4<SEL>(out[d], xa[d] * ia, xb[d] * ib); \
  }
      NVFP4KV_MX_PAIR(0)
      NVFP4KV_MX_PAIR(1)
      NVFP4KV_MX_PAIR(2)
      NVFP4KV_MX_PAIR(3)
#undef NVFP4KV_MX_PAIR
      if (o < opt && oc.nvalid == kOctet) {
        uint8_t *dst = qt.codes + (int64_t(oc.h) * a.D + 16 * b) * (a.rows / 2) + oc.row / 2;
#pragma unroll
        for (int d = 0; d < 16; ++d) *reinterpret_cast<uint32_t *>(dst + d * (a.rows / 2)) = out[d];
        if (lead)
          *reinterpret_cast<uint2 *>(qt.scales + (int64_t(oc.h) * nmx + (b >> 1)) * a.rows + oc.row) =
              make_uint2(sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24),
                         sb[4] | (sb[5] << 8) | (sb[6] << 16) | (sb[7] << 24));
      }
    } else {
      // codec layout: per token, 8 code bytes and (lead lane) the block's scale byte
#pragma unroll
      for (int j = 0; j < kOctet; ++j) {
        const int e = mx_exponent(mx_block_max(u[j]));
        float x[16];
        unpack16(u[j], x);
        const float inv = pow2_neg(e);
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] *= inv;
        uint32_t c[2] = {0u, 0u};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float *y = x + 8 * hh;
          c[hh] = cvt_fp4<0>(c[hh], y[0], y[1]);
          c[hh] = cvt_fp4<1>(c[hh], y[2], y[3]);
          c[hh] = cvt_fp4<2>(c[hh], y[4], y[5]);
          c[hh] = cvt_fp4<3>(c[hh], y[6], y[7]);
        }
        if (o < opt && j < oc.nvalid) {
          const int64_t row = int64_t(oc.h) * a.rows + oc.row + j;
          *reinterpret_cast<uint2 *>(qt.codes + row * (a.D / 2) + b * 8) = make_uint2(c[0], c[1]);
          if (lead) qt.scales[row * nmx + (b >> 1)] = uint8_t(e + 127);
        }
      }
    }
  }
  // no tensor scale: the chunk's scale-table entries read 1
  if (blockIdx.x == 0 && tid < a.n_tensors && a.t[tid].tensor_scale) *a.t[tid].tensor_scale = 1.0f;
}

// K-smoothing channel sums, one level of the pairwise tree (reading note, "The
// inference infrastructure": K-smoothing inside each frame chunk).  A workgroup
// reduces `group` consecutive leaves of one head for all D channels: each of its
// waves sums R = group / active-waves consecutive leaves per channel pair in
// registers, pairwise (v[i] = v[2i] + v[2i+1], level by level), then the waves'
// results are combined pairwise through LDS.  Leaf order and pairing are those of
// the full tree over the padded token count, so the result is the same fp32 value
// as that tree, whatever the number of levels and workgroups.
template <int R>
__global__ __launch_bounds__(1024) void channel_sum_kernel(MeanLevel a) {
  __shared__ float2 s_part[16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nodes = a.n_in / a.group;
  const int h = blockIdx.x / nodes, node = blockIdx.x - h * nodes;
  const int waves = a.group / R;           // a power of two, at most 16
  const bool col = 2 * lane < a.D;         // lane = channel pair (2 lane, 2 lane + 1)
  if (w < waves && col) {
    float2 v[R];
    const int leaf0 = node * a.group + w * R;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int leaf = leaf0 + i;
      if (a.src16) {
        v[i] = make_float2(0.0f, 0.0f);   // padding leaves are +0.0
        if (leaf < a.T) {
          const uint32_t x =
              *reinterpret_cast<const uint32_t *>(a.src16 + (int64_t(h) * a.T + leaf) * a.D + 2 * lane);
          v[i] = make_float2(__uint_as_float(x << 16), __uint_as_float(x & 0xFFFF0000u));
        }
      } else {
        v[i] = *reinterpret_cast<const float2 *>(a.src32 + (int64_t(h) * a.n_in + leaf) * a.D + 2 * lane);
      }
    }
#pragma unroll
    for (int width = R; width > 1; width >>= 1)
#pragma unroll
      for (int i = 0; i < width / 2; ++i) v[i] = make_float2(v[2 * i].x + v[2 * i + 1].x, v[2 * i].y + v[2 * i + 1].y);
    s_part[w][lane] = v[0];
  }
  __syncthreads();
  for (int width = waves; width > 1; width >>= 1) {
    float2 r = make_float2(0.0f, 0.0f);
    if (w < width / 2 && col) {
      const float2 p = s_part[2 * w][lane], q = s_part[2 * w + 1][lane];
      r = make_float2(p.x + q.x, p.y + q.y);
    }
    __syncthreads();
    if (w < width / 2 && col) s_part[w][lane] = r;
    __syncthreads();
  }
  if (w == 0 && col) {
    float2 r = s_part[0][lane];
    if (a.last) {
      const float t = float(a.T);
      *reinterpret_cast<float2 *>(a.dst + int64_t(h) * a.D + 2 * lane) = make_float2(r.x / t, r.y / t);
    } else {
      *reinterpret_cast<float2 *>(a.dst + (int64_t(h) * nodes + node) * a.D + 2 * lane) = r;
    }
  }
}

namespace {
constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];
int g_fused_per_cu[kMaxDevices];   // co-resident workgroups of the single-pass kernel per CU

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

namespace {
int64_t pow2_at_least(int64_t n) {
  int64_t p = 1;
  while (p < n) p *= 2;
  return p;
}
}  // namespace

int launch_channel_mean(const uint16_t *k, int H, int T, int D, float *mean, float *ws, void *stream) {
  if (H < 1 || T < 1 || D < 2 || D > 128 || D % 2) return NVFP4KV_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  MeanLevel a;
  a.src16 = k;
  a.src32 = nullptr;
  a.H = H;
  a.D = D;
  a.T = T;
  a.n_in = int32_t(pow2_at_least(T));
  const size_t half = channel_mean_ws_floats(H, T, D) / 2;
  int pingpong = 0;
  while (true) {
    a.group = a.n_in < kMeanGroup ? a.n_in : kMeanGroup;
    const int nodes = a.n_in / a.group;
    a.last = nodes == 1;
    a.dst = a.last ? mean : ws + pingpong * half;
    const int r = a.group >= 16 ? a.group / 16 : 1;
    const dim3 grid(unsigned(int64_t(H) * nodes)), block(1024);
    switch (r) {
      case 1: hipLaunchKernelGGL(channel_sum_kernel<1>, grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL(channel_sum_kernel<2>, grid, block, 0, s, a); break;
      case 4: hipLaunchKernelGGL(channel_sum_kernel<4>, grid, block, 0, s, a); break;
      case 8: hipLaunchKernelGGL(channel_sum_kernel<8>, grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL(channel_sum_kernel<16>, grid, block, 0, s, a); break;
    }
    if (hipGetLastError() != hipSuccess) return NVFP4KV_EHIP;
    if (a.last) return NVFP4KV_OK;
    a.src16 = nullptr;
    a.src32 = a.dst;
    a.n_in = nodes;
    pingpong ^= 1;
  }
}

int launch_quantize_mx(const QuantArgs &in, void *stream) {
  QuantArgs a = in;
  const int nb = a.D / 16;
  if (a.D % 32 != 0 || nb > kQuantThreads || a.tokens_per_frame < 1 || a.n_frames < 1)
    return NVFP4KV_EINVAL;
  a.tile_tokens = kOctet * (kQuantThreads / nb);
  a.tiles_per_head = int32_t((int64_t(a.T) + a.tile_tokens - 1) / a.tile_tokens);
  const int64_t total = int64_t(a.n_tensors) * a.H * a.tiles_per_head;
  if (total >= (int64_t(1) << 31)) return NVFP4KV_EINVAL;
  a.total_tiles = int32_t(total);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4KV_EHIP;
  // one workgroup per tile, up to 16 per CU, then a grid-stride loop
  int64_t g = total;
  if (g > int64_t(cu_count(dev)) * 16) g = int64_t(cu_count(dev)) * 16;
  hipLaunchKernelGGL(quantize_mx_kernel, dim3(unsigned(g)), dim3(kQuantThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), a);
  return NVFP4KV_HIP_OK(hipGetLastError());
}

int launch_quantize(const QuantArgs &in, void *stream) {
  QuantArgs a = in;
  const int nb = a.D / 16;
  if (nb < 1 || nb > kQuantThreads || a.tokens_per_frame < 1 || a.n_frames < 1) return NVFP4KV_EINVAL;
  a.tile_tokens = kOctet * (kQuantThreads / nb);
  a.tiles_per_head = int32_t((int64_t(a.T) + a.tile_tokens - 1) / a.tile_tokens);
  const int64_t total = int64_t(a.n_tensors) * a.H * a.tiles_per_head;
  if (total >= (int64_t(1) << 31)) return NVFP4KV_EINVAL;
  a.total_tiles = int32_t(total);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4KV_EHIP;
  const int cus = cu_count(dev);
  if (a.epoch > 0 && a.total_tiles <= kMaxQuantGrid && dev >= 0 && dev < kMaxDevices) {
    if (g_fused_per_cu[dev] == 0) {
      int per = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, quantize_fused_kernel, kQuantThreads, 0) !=
          hipSuccess)
        return NVFP4KV_EHIP;
      g_fused_per_cu[dev] = per > 0 ? per : -1;
    }
    if (g_fused_per_cu[dev] > 0 && a.total_tiles <= int64_t(cus) * g_fused_per_cu[dev]) {
      hipLaunchKernelGGL(quantize_fused_kernel, dim3(unsigned(a.total_tiles)), dim3(kQuantThreads), 0, s,
                         a);
      return NVFP4KV_HIP_OK(hipGetLastError());
    }
  }
  // pass 1: one 1024-thread workgroup per CU (fewer for small inputs)
  const int64_t vecs = int64_t(a.H) * a.T * a.D / 8;
  int64_t g1 = (vecs + kAmaxThreads * 2 - 1) / (kAmaxThreads * 2);
  if (g1 > cus) g1 = cus;
  if (g1 > kMaxQuantGrid) g1 = kMaxQuantGrid;
  if (g1 < 1) g1 = 1;
  hipLaunchKernelGGL(quantize_amax_kernel, dim3(unsigned(g1)), dim3(kAmaxThreads), 0, s, a);
  if (hipGetLastError() != hipSuccess) return NVFP4KV_EHIP;
  // pass 2: one workgroup per tile, up to 16 per CU, then a grid-stride loop
  int64_t g2 = total;
  if (g2 > int64_t(cus) * 16) g2 = int64_t(cus) * 16;
  hipLaunchKernelGGL(quantize_encode_kernel, dim3(unsigned(g2)), dim3(kQuantThreads), 0, s, a,
                     int(g1));
  return NVFP4KV_HIP_OK(hipGetLastError());
}

}  // namespace nvfp4kv
