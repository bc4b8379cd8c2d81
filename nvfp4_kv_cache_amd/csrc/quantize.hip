// NVFP4 quantization of K/V chunks for gfx950.
//
// Format (paper text section 2.2; reading note section II "The NVFP4
// quantization format"): 16-element blocks along head_dim, one E4M3 scale per
// block, one fp32 scale per tensor, E2M1 elements.  Recipe, in fp32 with correctly
// rounded operations: s_t = amax / 2688; bs = (block amax / 6) / s_t rounded to
// E4M3 (nearest, ties to even, saturating at 448); eff = E4M3(bs) * s_t;
// code = E2M1(|x| / eff) (nearest, ties to even, saturating at 6) with x's sign.
//
// Schedules.  The tensor scale needs the amax of the whole chunk tensor (all
// heads) before any block can be encoded.
//   * Cache appends (quantize_fused_kernel, one pass): every workgroup of a grid
//     that is resident all at once (the launcher checks the occupancy) loads its
//     tile into registers, publishes its maxima in an epoch-tagged workspace slot,
//     waits (bounded, then helping) for every slot of its tensor (K or V) and
//     encodes from the registers, so the chunk is read once.  While it waits it
//     already holds its values as fp32 and each scale byte's first quotient, so
//     only the s_t-dependent steps follow the wait.  No cooperative launch.
//   * Cache appends with K-smoothing and/or adaptive V scales take their own
//     single-pass kernel (quantize_options_kernel, below), with further exchanges
//     for the channel means and the heads' maxima of K minus its means.
//   * The standalone codec (its workspace cannot carry epochs), and appends whose
//     grid would not be resident at once: quantize_amax_kernel streams K and V once
//     and writes one partial maximum per workgroup (no atomics);
//     quantize_encode_kernel reduces the partials, then re-reads its tiles (the
//     chunk, 28.8 MB for the 1.3B shape, is still in the 256 MB Infinity Cache)
//     and writes codes and scales.
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

#include <atomic>

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

// The same from a6 = RN(amax / 6) taken beforehand (amax_bits: the block maximum as
// bf16 bits): the first quotient of either branch above is that correctly rounded one.
__device__ __forceinline__ uint32_t scale_code_pre(uint32_t amax_bits, float a6, const TensorConsts &tc) {
  const float bs = __uint_as_float(amax_bits << 16) >= tc.amin ? div_rn(a6, tc.st, tc.rst) : a6 / tc.st;
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

// The same for a token already held as fp32.
__device__ __forceinline__ void unpack16(const float (&xf)[16], float (&x)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = xf[i];
}

// Element i (0..15) of one token's block as fp32 (exact), extracted where it is used.
__device__ __forceinline__ float elem16(const uint4 (&u)[2], int i) {
  const uint4 q = u[i >> 3];
  const int c = (i >> 1) & 3;
  const uint32_t w = c == 0 ? q.x : c == 1 ? q.y : c == 2 ? q.z : q.w;
  return __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
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

// Adaptive block scale (V in the cache), token by token: squared error of encoding one
// token's block with scale byte sc, summed over its 16 elements in order of
// (|x| - value * eff)^2 with eff = E4M3(sc) * s_t, every step an fp32 operation (no
// contraction: the choice must match the recipe bit for bit).
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

// The same choice, one token pair (2*SEL, 2*SEL+1) of an octet at a time, keeping the
// codes: both candidates' codes go straight into byte SEL of their own set of the 16
// transposed words (o6, o4), each token's two errors are summed exactly as above
// (element order, no contraction), and keep4 collects the nibbles of the tokens whose
// 4-candidate won.
template <int SEL, bool SCALED>
__device__ __forceinline__ void adaptive_pair(const float (&xa)[16], const float (&xb)[16], float ma, float mb,
                                              const TensorConsts &tc, const float2 *tab, uint32_t (&o6)[16],
                                              uint32_t (&o4)[16], uint32_t &keep4, uint32_t &sca,
                                              uint32_t &scb) {
#pragma clang fp contract(off)
  const uint32_t a6 = scale_code(ma, tc), b6 = scale_code(mb, tc);
  const uint32_t a4 = scale_code<4>(ma, tc), b4 = scale_code<4>(mb, tc);
  const float2 da6 = tab[a6], db6 = tab[b6], da4 = tab[a4], db4 = tab[b4];
  const float ea6 = __builtin_amdgcn_cvt_f32_fp8(a6, 0) * tc.st, eb6 = __builtin_amdgcn_cvt_f32_fp8(b6, 0) * tc.st;
  const float ea4 = __builtin_amdgcn_cvt_f32_fp8(a4, 0) * tc.st, eb4 = __builtin_amdgcn_cvt_f32_fp8(b4, 0) * tc.st;
  float ra6 = 0.0f, rb6 = 0.0f, ra4 = 0.0f, rb4 = 0.0f;
#pragma unroll
  for (int d = 0; d < 16; ++d) {
    o6[d] = cvt_fp4<SEL>(o6[d], quot<SCALED>(xa[d], da6.x, da6.y, tc.xs), quot<SCALED>(xb[d], db6.x, db6.y, tc.xs));
    const auto v6 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(o6[d], 1.0f, SEL);
    const float pa6 = fabsf(xa[d]) - fabsf(v6[0]) * ea6;
    ra6 = ra6 + pa6 * pa6;
    const float pb6 = fabsf(xb[d]) - fabsf(v6[1]) * eb6;
    rb6 = rb6 + pb6 * pb6;
    o4[d] = cvt_fp4<SEL>(o4[d], quot<SCALED>(xa[d], da4.x, da4.y, tc.xs), quot<SCALED>(xb[d], db4.x, db4.y, tc.xs));
    const auto v4 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(o4[d], 1.0f, SEL);
    const float pa4 = fabsf(xa[d]) - fabsf(v4[0]) * ea4;
    ra4 = ra4 + pa4 * pa4;
    const float pb4 = fabsf(xb[d]) - fabsf(v4[1]) * eb4;
    rb4 = rb4 + pb4 * pb4;
  }
  const bool wa = ra4 < ra6, wb = rb4 < rb6;
  sca = wa ? a4 : a6;
  scb = wb ? b4 : b6;
  keep4 |= ((wa ? 0x0Fu : 0u) | (wb ? 0xF0u : 0u)) << (8 * SEL);
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
template <bool SCALED, bool MEAN = false, typename U>
__device__ __forceinline__ void item_canonical(const QuantArgs &a, const Octet &o, int b, const U &u,
                                               const TensorConsts &tc, const float2 *tab,
                                               const uint32_t *bmax = nullptr, const float *pre6 = nullptr) {
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
    for (int j = 0; j < kOctet; ++j)
      scp[j] = pre6 ? scale_code_pre(bmax[j], pre6[j], tc) : scale_code(__uint_as_float(bmax[j] << 16), tc);
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
// ADAPT (adaptive block scales): KEEP takes each token's codes from its winning
// candidate's error pass (about a fifth fewer VALU operations, 32 words live instead
// of 16); without it every token's scale byte is chosen first and the octet is then
// encoded once more with the winners, for kernels that would spill the extra words.
template <bool SCALED, bool ADAPT = false, bool KEEP = true, typename U>
__device__ __forceinline__ void item_transposed(const QuantArgs &a, const Octet &o, int b, const U &u,
                                                const TensorConsts &tc, const float2 *tab,
                                                const uint32_t *bmax = nullptr, const float *pre6 = nullptr) {
  const QuantTensor &qt = a.t[o.tensor];
  const int nb = a.D >> 4;
  uint32_t sc[kOctet];
  uint32_t out[16];
#pragma unroll
  for (int d = 0; d < 16; ++d) out[d] = 0u;
  if constexpr (ADAPT && KEEP) {
    uint32_t o4[16], keep4 = 0u;
#pragma unroll
    for (int d = 0; d < 16; ++d) o4[d] = 0u;
#define NVFP4KV_APAIR(SEL)                                                                               \
    {                                                                                                    \
      float xa[16], xb[16];                                                                              \
      unpack16(u[2 * SEL], xa);                                                                          \
      unpack16(u[2 * SEL + 1], xb);                                                                      \
      const float ma = bmax ? __uint_as_float(bmax[2 * SEL] << 16) : absmax16(xa);                       \
      const float mb = bmax ? __uint_as_float(bmax[2 * SEL + 1] << 16) : absmax16(xb);                   \
      adaptive_pair<SEL, SCALED>(xa, xb, ma, mb, tc, tab, out, o4, keep4, sc[2 * SEL], sc[2 * SEL + 1]); \
    }
    NVFP4KV_APAIR(0)
    NVFP4KV_APAIR(1)
    NVFP4KV_APAIR(2)
    NVFP4KV_APAIR(3)
#undef NVFP4KV_APAIR
#pragma unroll
    for (int d = 0; d < 16; ++d) out[d] = (o4[d] & keep4) | (out[d] & ~keep4);
  } else {
    // every scale byte and divisor first when the maxima are at hand, or (adaptive
    // scales) after choosing each token's byte on its own, one token at a time
    float2 dvp[kOctet];
    const bool pre = bmax || ADAPT;
    if (ADAPT) {
#pragma unroll
      for (int j = 0; j < kOctet; ++j) {
        float x[16];
        unpack16(u[j], x);
        const float m = bmax ? __uint_as_float(bmax[j] << 16) : absmax16(x);
        sc[j] = choose_scale46<SCALED>(x, m, scale_code(m, tc), tc, tab);
      }
#pragma unroll
      for (int j = 0; j < kOctet; ++j) dvp[j] = tab[sc[j]];
    } else if (bmax) {
#pragma unroll
      for (int j = 0; j < kOctet; ++j)
        sc[j] = pre6 ? scale_code_pre(bmax[j], pre6[j], tc) : scale_code(__uint_as_float(bmax[j] << 16), tc);
#pragma unroll
      for (int j = 0; j < kOctet; ++j) dvp[j] = tab[sc[j]];
    }
#define NVFP4KV_PAIR(SEL)                                                              \
    {                                                                                  \
      float xa[16], xb[16];                                                            \
      unpack16(u[2 * SEL], xa);                                                        \
      unpack16(u[2 * SEL + 1], xb);                                                    \
      float2 da, db;                                                                   \
      if (pre) {                                                                       \
        da = dvp[2 * SEL];                                                             \
        db = dvp[2 * SEL + 1];                                                         \
      } else {                                                                         \
        sc[2 * SEL] = scale_code(absmax16(xa), tc);                                    \
        sc[2 * SEL + 1] = scale_code(absmax16(xb), tc);                                \
        da = tab[sc[2 * SEL]];                                                         \
        db = tab[sc[2 * SEL + 1]];                                                     \
      }                                                                                \
      encode_pair_transposed<SEL, SCALED>(xa, xb, da.x, da.y, db.x, db.y, tc.xs, out); \
    }
    NVFP4KV_PAIR(0)
    NVFP4KV_PAIR(1)
    NVFP4KV_PAIR(2)
    NVFP4KV_PAIR(3)
#undef NVFP4KV_PAIR
  }
  if (o.nvalid == kOctet) {
    uint8_t *dst = qt.codes + (int64_t(o.h) * a.D + 16 * b) * (a.rows / 2) + o.row / 2;
#pragma unroll
    for (int d = 0; d < 16; ++d) *reinterpret_cast<uint32_t *>(dst + d * (a.rows / 2)) = out[d];
    *reinterpret_cast<uint2 *>(qt.scales + (int64_t(o.h) * nb + b) * a.rows + o.row) =
        make_uint2(sc[0] | (sc[1] << 8) | (sc[2] << 16) | (sc[3] << 24),
                   sc[4] | (sc[5] << 8) | (sc[6] << 16) | (sc[7] << 24));
  }
}

// The octet's source only (tensor, head, first token, tokens inside the chunk): what a
// helper needs, without the destination rows' frame table.
__device__ __forceinline__ Octet locate_source(const QuantArgs &a, int tile, int o) {
  Octet r;
  r.tensor = tile / (a.H * a.tiles_per_head);
  const int rem = tile - r.tensor * a.H * a.tiles_per_head;
  r.h = rem / a.tiles_per_head;
  r.tok = (rem - r.h * a.tiles_per_head) * a.tile_tokens + kOctet * o;
  r.nvalid = min(max(a.T - r.tok, 0), kOctet);
  r.row = 0;
  return r;
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
// OPT: the tensors may carry K-smoothing means or adaptive V scales (their items need
// more registers; the plain codec keeps its own instance).
template <bool OPT>
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
          if (OPT && qt.adaptive) item_transposed<false, OPT, false>(a, oc, b, u, tc, tab);
          else item_transposed<false>(a, oc, b, u, tc, tab);
        } else {
          if (OPT && qt.mean) item_canonical<false, OPT>(a, oc, b, u, tc, tab);
          else item_canonical<false>(a, oc, b, u, tc, tab);
        }
      } else {
        if (tr) {
          if (OPT && qt.adaptive) item_transposed<true, OPT, false>(a, oc, b, u, tc, tab);
          else item_transposed<true>(a, oc, b, u, tc, tab);
        } else {
          if (OPT && qt.mean) item_canonical<true, OPT>(a, oc, b, u, tc, tab);
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
// waits until the slot of every workgroup of its tensor carries that epoch (K and V
// do not wait for each other), and encodes from the registers, so the chunk is read
// once.  The launcher only takes this path when the
// grid fits on the GPU at once (occupancy), but co-residency is not guaranteed (other
// streams' kernels may hold CUs), so the wait is bounded (a.spin_limit polls): past
// it, a waiting workgroup helps instead of waiting.  Each polling round it takes one
// tile whose slot is still missing (the k-th missing one, k from its own number, so
// that helpers spread over the missing tiles), computes that tile's maxima exactly
// as its owner would, and publishes them in the owner's slot (the owner, when it
// runs, writes the same word).  A helper thus reads one tile per round; all helpers
// together read each missing tile about once (at most one extra read of the chunk),
// and every slot is filled even if its owner never becomes resident first.

// Packed maxima word of one tile: |bf16| bits of K in bits 15-29, of V in bits 0-14
// (a tile belongs to one tensor; the other field is 0).
__device__ __forceinline__ void tile_maxima(const QuantArgs &a, int tile, uint32_t &mk, uint32_t &mv) {
  const int nb = a.D >> 4;
  const int opt = kQuantThreads / nb;
  const int b = threadIdx.x % nb, o = threadIdx.x / nb;
  const Octet oc = locate_source(a, tile, min(o, opt - 1));
  const uint4 *src = reinterpret_cast<const uint4 *>(a.t[oc.tensor].src + int64_t(oc.h) * a.T * a.D + 16 * b);
  uint32_t mx = 0;
  for (int j = 0; j < kOctet; ++j) {
    const int64_t tok = min(oc.tok + j, a.T - 1);
    const uint4 u[2] = {src[tok * (a.D / 8)], src[tok * (a.D / 8) + 1]};
    mx = max(mx, block_max_bits(u));
  }
  mk = oc.tensor == 0 ? mx : 0u;
  mv = oc.tensor == 1 ? mx : 0u;
}

__global__ __launch_bounds__(kQuantThreads) void quantize_fused_kernel(QuantArgs a) {
  __shared__ uint32_t s_red[2][kQuantThreads / 64];
  __shared__ int s_ok[kQuantThreads / 64];
  __shared__ int s_help;
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
  // work that does not need s_t, done while the exchange is pending: the tokens as
  // fp32 and the first quotient amax / 6 of each scale byte (kept in registers: the
  // empty asm statements keep the compiler from moving them after the wait)
  float xf[kOctet][16], a6[kOctet];
#pragma unroll
  for (int j = 0; j < kOctet; ++j) {
    unpack16(u[j], xf[j]);
    a6[j] = __uint_as_float(bm[j] << 16) / 6.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(xf[j][i]));
    asm volatile("" : "+v"(a6[j]));
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

  // wait for the slots of every workgroup of this tensor (bounded; then help): the
  // K tiles come first, [0, nk), then the V tiles
  constexpr int kSlotsPerThread = kMaxQuantGrid / kQuantThreads;
  const int nk = a.H * a.tiles_per_head;
  const bool is_k = int(blockIdx.x) < nk;
  const int lo = is_k ? 0 : nk, hi = is_k ? nk : int(gridDim.x);
  uint32_t gk = 0, gv = 0;
  for (int spin = 0;; ++spin) {
    uint32_t k = 0, v = 0, miss = 0;
#pragma unroll
    for (int i = 0; i < kSlotsPerThread; ++i) {
      const int j = lo + tid + i * kQuantThreads;
      if (j < hi) {
        const uint64_t w = __hip_atomic_load(&a.ws->slot[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((w >> 30) != a.epoch) miss |= 1u << i;
        k = max(k, uint32_t(w >> 15) & 0x7FFFu);
        v = max(v, uint32_t(w) & 0x7FFFu);
      }
    }
    // missing slots: per-thread counts, scanned over the workgroup
    const int cnt = __builtin_popcount(miss);
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    k = wave_max_u32(k);
    v = wave_max_u32(v);
    if (lane == 63) s_ok[wv] = incl;
    if (lane == 0) {
      s_red[0][wv] = k;
      s_red[1][wv] = v;
    }
    __syncthreads();
    int n_miss = 0, before = 0;
    gk = gv = 0;
    for (int i = 0; i < kQuantThreads / 64; ++i) {
      n_miss += s_ok[i];
      before += i < wv ? s_ok[i] : 0;
      gk = max(gk, s_red[0][i]);
      gv = max(gv, s_red[1][i]);
    }
    if (n_miss == 0) break;
    if (spin >= a.spin_limit) {
      // help: the k-th missing slot of this round, k from this workgroup's number
      const int kth = int((blockIdx.x + uint32_t(spin - a.spin_limit)) % uint32_t(n_miss));
      const int excl = before + incl - cnt;
      if (kth >= excl && kth < excl + cnt) {
        uint32_t m = miss;
        for (int r = kth - excl; r > 0; --r) m &= m - 1;   // drop the lower set bits
        s_help = lo + tid + (__builtin_ctz(m)) * kQuantThreads;
      }
      __syncthreads();
      const int tile = s_help;
      uint32_t hk, hv;
      tile_maxima(a, tile, hk, hv);
      hk = wave_max_u32(hk);
      hv = wave_max_u32(hv);
      if (lane == 0) {
        s_red[0][wv] = hk;
        s_red[1][wv] = hv;
      }
      __syncthreads();
      if (tid == 0) {
        uint32_t rk = 0, rv = 0;
        for (int i = 0; i < kQuantThreads / 64; ++i) {
          rk = max(rk, s_red[0][i]);
          rv = max(rv, s_red[1][i]);
        }
        const uint64_t word = (a.epoch << 30) | (uint64_t(rk) << 15) | uint64_t(rv);
        __hip_atomic_store(&a.ws->slot[tile], word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      __builtin_amdgcn_s_sleep(2);
    }
    __syncthreads();
  }

  // this tensor's scale (the other field of its slots is 0): written by its first tile
  const float st0 = bf16_bits_to_float(gk) / 2688.0f, st1 = bf16_bits_to_float(gv) / 2688.0f;
  if ((int(blockIdx.x) == 0 || int(blockIdx.x) == nk) && tid == 0) *a.t[is_k ? 0 : 1].tensor_scale = is_k ? st0 : st1;
  const TensorConsts tc0 = tensor_consts(st0), tc1 = tensor_consts(st1);
  for (int e = tid; e < kScaleCodes; e += kQuantThreads)
    s_tab[oc.tensor][e] = divisor_entry(e, oc.tensor ? st1 : st0, oc.tensor ? tc1.xs : tc0.xs);
  __syncthreads();
  if (act) {
    const TensorConsts &tc = oc.tensor ? tc1 : tc0;
    const float2 *tab = s_tab[oc.tensor];
    const bool tr = a.t[oc.tensor].transposed != 0;
    if (tc.xs == 1.0f) {
      if (tr) item_transposed<false>(a, oc, b, xf, tc, tab, bm, a6);
      else item_canonical<false>(a, oc, b, xf, tc, tab, bm, a6);
    } else {
      if (tr) item_transposed<true>(a, oc, b, xf, tc, tab, bm, a6);
      else item_canonical<true>(a, oc, b, xf, tc, tab, bm, a6);
    }
  }
}

// ---- single pass with the cache options (K-smoothing, adaptive V block scales)
// Its own kernel with its own occupancy check, so that the plain single pass keeps
// its registers.  The structure is the plain single pass's, with the options' extra
// exchanges:
//  * V workgroups (and K workgroups without smoothing) publish their tile maxima and
//    wait for the slots of their own tensor only, then encode (V with the adaptive
//    block scale when asked).
//  * K workgroups with smoothing need the channel means before the tensor maximum.
//    The means' pairwise tree runs over the +0.0-padded power-of-two token count
//    n_in; a tile of tile_tokens tokens starting at a multiple of tile_tokens is one
//    aligned subtree of it (all of it when n_in < tile_tokens: the chunk is then one
//    tile).  Each workgroup publishes, per channel, its tile's node sum and the
//    largest and smallest value of its tokens; waits for the nodes of its head;
//    finishes the top of the tree (nodes past the last tile are +0.0) and divides by
//    T: the same fp32 operations as the tree taken level by level.  Rounding is
//    monotone, so over a channel's values x the largest |RN(x - mean)| is that of its
//    largest or of its smallest value: the head's max |K - mean| follows from the
//    published extremes, exactly.  Every workgroup of the head publishes that head
//    word (all alike), waits for every head's word, and encodes K - mean from its
//    registers.
// The exchanged words carry the low half of the launch's epoch in their upper half,
// so a reader that sees the tag sees the value (no fences).  Every wait is bounded:
// past a.spin_limit polls a workgroup helps, one missing tile or head per round (the
// k-th missing one, k from its own number), computing exactly what its owner would
// publish; a missing head word is computed from that head's published tiles (helping
// with them first if some are missing).
namespace {

struct OptShared {
  uint32_t red[2][kQuantThreads / 64];
  int cnt[kQuantThreads / 64];
  int pick;
  uint32_t mask;
  float2 tab[kScaleCodes];
  float mu[128];
  float mu_help[128];
  float part[kQuantThreads * 16];      // [octets per tile][D]: each octet's channel sums
  uint32_t ext[kQuantThreads * 16];    // [octets per tile][D]: its largest | smallest value (bf16 bits)
};

__device__ __forceinline__ uint64_t tagged(const QuantArgs &a, uint32_t bits) {
  return (uint64_t(uint32_t(a.epoch)) << 32) | bits;
}
__device__ __forceinline__ bool tag_ok(const QuantArgs &a, uint64_t w) {
  return uint32_t(w >> 32) == uint32_t(a.epoch);
}

// Leaves of the means tree under one node: min(n_in, tile_tokens), n_in the power of
// two >= T; and the nodes of the tree's top.
__device__ __forceinline__ int node_leaves(const QuantArgs &a) {
  const int n_in = a.T <= 1 ? 1 : 1 << (32 - __builtin_clz(uint32_t(a.T - 1)));
  return min(n_in, a.tile_tokens);
}
__device__ __forceinline__ int top_nodes(const QuantArgs &a) {
  const int n_in = a.T <= 1 ? 1 : 1 << (32 - __builtin_clz(uint32_t(a.T - 1)));
  return n_in / node_leaves(a);
}

// Pairwise sum of v[0..n), n a power of two <= 32: neighbours first, level by level.
__device__ __forceinline__ float tree32(const float (&v)[32], int n) {
  float l1[16], l2[8], l3[4], l4[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) l1[i] = v[2 * i] + v[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 8; ++i) l2[i] = l1[2 * i] + l1[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) l3[i] = l2[2 * i] + l2[2 * i + 1];
  l4[0] = l3[0] + l3[1];
  l4[1] = l3[2] + l3[3];
  const float l5 = l4[0] + l4[1];
  return n >= 32 ? l5 : n == 16 ? l4[0] : n == 8 ? l3[0] : n == 4 ? l2[0] : n == 2 ? l1[0] : v[0];
}

// Pairwise sum in push order: after 2^m pushes of aligned subtree sums, st[m] holds
// their pairwise sum (a pushed value meets its left neighbours level by level).
template <int N>
__device__ __forceinline__ void pairwise_push(float (&st)[N], int i, float v) {
#pragma unroll
  for (int k = 0; k < N; ++k) {
    if ((i >> k) & 1) {
      v = st[k] + v;
    } else {
      st[k] = v;
      return;
    }
  }
}
template <int N>
__device__ __forceinline__ float pairwise_total(const float (&st)[N], int levels) {
  float r = st[0];
#pragma unroll
  for (int k = 1; k < N; ++k) r = k == levels ? st[k] : r;
  return r;
}

// Word of tile statistic (head h, channel c, tile of the head `node`): channels in
// groups of 64, the tiles of a head consecutive within a group, so that a wave's 64
// channels of one node are one 512-byte run and the nodes of a channel are 512 bytes
// apart (immediate offsets from one address).
__device__ __forceinline__ int64_t stat_index(const QuantArgs &a, int h, int c, int node) {
  return ((int64_t(h) * (a.D >> 6) + (c >> 6)) * a.tiles_per_head + node) * 64 + (c & 63);
}

// Packed extremes of bf16 values: largest value's bits << 16 | smallest value's bits.
__device__ __forceinline__ uint32_t ext_pack(float hi, float lo) {
  return (__float_as_uint(hi) & 0xFFFF0000u) | (__float_as_uint(lo) >> 16);
}
__device__ __forceinline__ float ext_hi(uint32_t e) { return __uint_as_float(e & 0xFFFF0000u); }
__device__ __forceinline__ float ext_lo(uint32_t e) { return __uint_as_float(e << 16); }

// Workgroup-wide count of missing slots (bit i of `miss`: slot tid + i * kQuantThreads
// of the polled range) and maxima of k, v.  With `help` and some missing, the k-th
// missing slot (k = seed mod the count) is left in sh.pick.  Every thread calls it;
// it ends with a barrier.
__device__ int poll_reduce(uint32_t miss, uint32_t &k, uint32_t &v, bool help, uint32_t seed,
                           OptShared &sh) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int cnt = __builtin_popcount(miss);
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  k = wave_max_u32(k);
  v = wave_max_u32(v);
  if (lane == 63) sh.cnt[wv] = incl;
  if (lane == 0) {
    sh.red[0][wv] = k;
    sh.red[1][wv] = v;
  }
  __syncthreads();
  int n = 0, before = 0;
  k = v = 0;
  for (int i = 0; i < kQuantThreads / 64; ++i) {
    n += sh.cnt[i];
    before += i < wv ? sh.cnt[i] : 0;
    k = max(k, sh.red[0][i]);
    v = max(v, sh.red[1][i]);
  }
  if (help && n > 0) {
    const int kth = int(seed % uint32_t(n));
    const int excl = before + incl - cnt;
    if (kth >= excl && kth < excl + cnt) {
      uint32_t m = miss;
      for (int r = kth - excl; r > 0; --r) m &= m - 1;   // drop the lower set bits
      sh.pick = tid + __builtin_ctz(m) * kQuantThreads;
    }
  }
  __syncthreads();
  return n;
}

// Bounded wait for the maxima slots [lo, hi) (helping past the limit); K and V maxima
// over them.
__device__ void wait_maxima(const QuantArgs &a, int lo, int hi, uint32_t &gk, uint32_t &gv, OptShared &sh) {
  constexpr int kSlotsPerThread = kMaxQuantGrid / kQuantThreads;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int spin = 0;; ++spin) {
    uint32_t k = 0, v = 0, miss = 0;
#pragma unroll
    for (int i = 0; i < kSlotsPerThread; ++i) {
      const int j = lo + tid + i * kQuantThreads;
      if (j < hi) {
        const uint64_t w = __hip_atomic_load(&a.ws->slot[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((w >> 30) != a.epoch) miss |= 1u << i;
        k = max(k, uint32_t(w >> 15) & 0x7FFFu);
        v = max(v, uint32_t(w) & 0x7FFFu);
      }
    }
    const bool help = spin >= a.spin_limit;
    const int n = poll_reduce(miss, k, v, help, blockIdx.x + uint32_t(spin), sh);
    if (n == 0) {
      gk = k;
      gv = v;
      return;
    }
    if (help) {
      const int tile = lo + sh.pick;
      uint32_t hk, hv;
      tile_maxima(a, tile, hk, hv);
      hk = wave_max_u32(hk);
      hv = wave_max_u32(hv);
      if (lane == 0) {
        sh.red[0][wv] = hk;
        sh.red[1][wv] = hv;
      }
      __syncthreads();
      if (tid == 0) {
        uint32_t rk = 0, rv = 0;
        for (int i = 0; i < kQuantThreads / 64; ++i) {
          rk = max(rk, sh.red[0][i]);
          rv = max(rv, sh.red[1][i]);
        }
        const uint64_t word = (a.epoch << 30) | (uint64_t(rk) << 15) | uint64_t(rv);
        __hip_atomic_store(&a.ws->slot[tile], word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
    } else {
      __builtin_amdgcn_s_sleep(2);
    }
  }
}

// Order-preserving 16-bit keys of two packed bf16 values (negative values have all
// bits flipped, others only the sign), so that unsigned 16-bit maxima and minima of
// keys are those of the values; key_to_bf16 undoes it.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_keys(uint32_t w) {
  const uint32_t neg = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2_t, w) >> (i16x2_t){15, 15});
  return w ^ (neg | 0x80008000u);
}
__device__ __forceinline__ uint32_t keys_to_bf16(uint32_t k) {
  // a key with the top bit clear came from a negative value
  const uint32_t pos = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2_t, k) >> (i16x2_t){15, 15});
  return k ^ (~pos | 0x80008000u);
}
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t x, uint32_t y) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, x), __builtin_bit_cast(u16x2_t, y)));
}
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t x, uint32_t y) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2_t, x), __builtin_bit_cast(u16x2_t, y)));
}

// One half (8 channels) of the thread's octet into the LDS tables: the channel sums
// of its 8 leaves, pairwise (tokens past T are +0.0; a node of fewer than 8 leaves,
// L < 8, i.e. T <= 4, is the left part of octet 0), and the channel extremes (tokens
// past T re-read the last token, a value of the channel), as bf16 bits.
__device__ __forceinline__ void octet_half(const uint4 (&uh)[kOctet], int nvalid, int L, float *sums,
                                           uint32_t *ext) {
  // extremes: per word (two channels) the packed key maxima / minima over the tokens
  uint32_t kmax[4], kmin[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t k = bf16_keys(c == 0 ? uh[0].x : c == 1 ? uh[0].y : c == 2 ? uh[0].z : uh[0].w);
    kmax[c] = kmin[c] = k;
#pragma unroll
    for (int j = 1; j < kOctet; ++j) {
      k = bf16_keys(c == 0 ? uh[j].x : c == 1 ? uh[j].y : c == 2 ? uh[j].z : uh[j].w);
      kmax[c] = pk_max_u16(kmax[c], k);
      kmin[c] = pk_min_u16(kmin[c], k);
    }
    kmax[c] = keys_to_bf16(kmax[c]);
    kmin[c] = keys_to_bf16(kmin[c]);
  }
  uint32_t e[8];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    e[2 * c] = (kmax[c] << 16) | (kmin[c] & 0xFFFFu);
    e[2 * c + 1] = (kmax[c] & 0xFFFF0000u) | (kmin[c] >> 16);
  }
  // sums
  float s[8];
  const bool full = nvalid == kOctet;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float x[kOctet];
#pragma unroll
    for (int j = 0; j < kOctet; ++j) {
      const uint4 q = uh[j];
      const int c = i >> 1;
      const uint32_t w = c == 0 ? q.x : c == 1 ? q.y : c == 2 ? q.z : q.w;
      x[j] = __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
      if (!full) x[j] = j < nvalid ? x[j] : 0.0f;
    }
    const float p0 = x[0] + x[1], p1 = x[2] + x[3], p2 = x[4] + x[5], p3 = x[6] + x[7];
    const float q0 = p0 + p1, q1 = p2 + p3;
    s[i] = L >= 8 ? q0 + q1 : L == 4 ? q0 : L == 2 ? p0 : x[0];
  }
  float4 *s4 = reinterpret_cast<float4 *>(sums);
  s4[0] = make_float4(s[0], s[1], s[2], s[3]);
  s4[1] = make_float4(s[4], s[5], s[6], s[7]);
  uint4 *e4 = reinterpret_cast<uint4 *>(ext);
  e4[0] = make_uint4(e[0], e[1], e[2], e[3]);
  e4[1] = make_uint4(e[4], e[5], e[6], e[7]);
}

// The octets' tables -> the tile's node sum and extremes per channel, published as
// tagged words sums[h][tile of the head][c] and ext[h][tile of the head][c] (ext after
// the H x tiles_per_head x D sums).  Threads [0, D) take the sums, threads [D, 2D) the
// extremes.  Every thread calls it.
__device__ void publish_tile_stats(const QuantArgs &a, int tile, int h, OptShared &sh) {
  __syncthreads();
  const int tid = threadIdx.x;
  const int L = node_leaves(a);
  const int n_oct = L >= 8 ? L / 8 : 1;                 // octets under the node (at most 64)
  const int n_all = kQuantThreads / (a.D >> 4);         // octets of the tile
  const int64_t n_sums = int64_t(a.H) * a.tiles_per_head * a.D;
  if (tid < a.D) {
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = i < n_oct ? sh.part[i * a.D + tid] : 0.0f;
    float node = tree32(v, min(n_oct, 32));
    if (n_oct > 32) {   // two aligned halves of 32 octets
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = sh.part[(32 + i) * a.D + tid];
      node = node + tree32(v, 32);
    }
    __hip_atomic_store(a.sum_slots + stat_index(a, h, tid, tile % a.tiles_per_head),
                       tagged(a, __float_as_uint(node)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (tid < 2 * a.D) {
    const int c = tid - a.D;
    float hi = -__builtin_inff(), lo = __builtin_inff();
    for (int i0 = 0; i0 < n_all; i0 += 32) {   // 32 or 64 octets: independent reads
      uint32_t e[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) e[i] = sh.ext[(i0 + i) * a.D + c];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        hi = fmaxf(hi, ext_hi(e[i]));
        lo = fminf(lo, ext_lo(e[i]));
      }
    }
    __hip_atomic_store(a.sum_slots + n_sums + stat_index(a, h, c, tile % a.tiles_per_head),
                       tagged(a, ext_pack(hi, lo)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
}

// The owner: its tile's statistics from the registers.
__device__ void own_tile_stats(const QuantArgs &a, int tile, const Octet &oc, int o, int b,
                               const uint4 (&u)[kOctet][2], OptShared &sh) {
  const int L = node_leaves(a);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    uint4 uh[kOctet];
#pragma unroll
    for (int j = 0; j < kOctet; ++j) uh[j] = u[j][hh];
    octet_half(uh, oc.nvalid, L, sh.part + o * a.D + 16 * b + 8 * hh, sh.ext + o * a.D + 16 * b + 8 * hh);
  }
  publish_tile_stats(a, tile, oc.h, sh);
}

// A helper: loads K tile `tile` half a block at a time and publishes its statistics.
__device__ void help_tile_stats(const QuantArgs &a, int tile, OptShared &sh) {
  const int nb = a.D >> 4;
  const int opt = kQuantThreads / nb;
  const int b = threadIdx.x % nb, o = threadIdx.x / nb;
  const Octet oc = locate_source(a, tile, min(o, opt - 1));
  const int L = node_leaves(a);
  const uint4 *src = reinterpret_cast<const uint4 *>(a.t[0].src + int64_t(oc.h) * a.T * a.D + 16 * b);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    uint4 uh[kOctet];
#pragma unroll
    for (int j = 0; j < kOctet; ++j) uh[j] = src[int64_t(min(oc.tok + j, a.T - 1)) * (a.D / 8) + hh];
    octet_half(uh, oc.nvalid, L, sh.part + o * a.D + 16 * b + 8 * hh, sh.ext + o * a.D + 16 * b + 8 * hh);
  }
  publish_tile_stats(a, tile, oc.h, sh);
}

// Means of head h into mu[0..D) and the head's max |K - mean| (fp32 bits, returned to
// every thread): waits until every tile of the head has published its statistics
// (bounded; then helps), finishes the top of the means tree with the nodes past the
// last tile as +0.0 and divides by T; per channel max(|RN(hi - mean)|, |RN(lo - mean)|)
// over the head's extremes.  The nodes go in batches of 32 (aligned subtrees when
// there are more); P = 256 / D threads share a channel, each taking 32 / P consecutive
// nodes of the batch.  Every thread calls it.
__device__ uint32_t head_stats(const QuantArgs &a, int h, float *mu, OptShared &sh) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int tph = a.tiles_per_head;
  const int n_top = top_nodes(a);           // a power of two, >= tph, <= 2^11
  const int P = kQuantThreads / a.D;        // 2 (D = 128) or 4 (D = 64)
  const int npp = 32 / P;                   // nodes per thread and batch: 16 or 8
  const int c = tid % a.D, part = tid / a.D;
  const int n_batch = min(n_top, 32);       // nodes per batch (all batches alike)
  const int n_parts = max(1, n_batch / npp);   // parts holding nodes of a batch
  const int n_mine = min(npp, n_batch);     // nodes per part
  const int64_t n_sums = int64_t(a.H) * tph * a.D;
  float st[7];                              // pairwise stack over the batches
  float hi = -__builtin_inff(), lo = __builtin_inff();
  // First a light wait on one word per tile of the head (its channel-0 extremes), so
  // that the full statistics are normally read once; the full read below still checks
  // every word's tag (another lane's words may become visible later) and polls again.
  for (int spin = 0;; ++spin) {
    uint32_t miss = 0, k = 0, v = 0;
    for (int i = 0; i < (tph + kQuantThreads - 1) / kQuantThreads; ++i) {
      const int node = tid + i * kQuantThreads;
      if (node < tph && !tag_ok(a, __hip_atomic_load(a.sum_slots + n_sums + stat_index(a, h, 0, node),
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)))
        miss |= 1u << i;
    }
    const bool help = spin >= a.spin_limit;
    if (poll_reduce(miss, k, v, help, blockIdx.x + uint32_t(spin), sh) == 0) break;
    if (help) help_tile_stats(a, h * tph + sh.pick, sh);   // barriers inside
    else __builtin_amdgcn_s_sleep(2);
  }
  if (tid == 0) sh.mask = 0u;
  __syncthreads();
  for (int base = 0, spin = 0; base < n_top; base += 32) {
    float half = 0.0f;
    while (true) {
      uint32_t miss = 0;
      float bh = -__builtin_inff(), bl = __builtin_inff();
      if (part < n_parts) {
        uint64_t w[16], x[16];
        const int first = base + part * npp;
        // unconditional loads from one address: nodes past the head's last tile (at
        // most max(tiles_per_head, 16) of them) read the next rows' words or the slack
        // after the arrays, and are not used
        const uint64_t *ps = a.sum_slots + stat_index(a, h, c, first), *px = ps + n_sums;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          w[i] = __hip_atomic_load(ps + 64 * i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          x[i] = __hip_atomic_load(px + 64 * i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        float v[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          v[i] = 0.0f;
          if (i < 16) {
            const bool real = i < n_mine && first + i < tph;   // past the last tile: +0.0
            if (real && !(tag_ok(a, w[i]) && tag_ok(a, x[i]))) miss |= 1u << (part * npp + i);
            v[i] = real ? __uint_as_float(uint32_t(w[i])) : 0.0f;
            if (real) {
              bh = fmaxf(bh, ext_hi(uint32_t(x[i])));
              bl = fminf(bl, ext_lo(uint32_t(x[i])));
            }
          }
        }
        half = tree32(v, n_mine);
      }
      if (miss) atomicOr(&sh.mask, miss);
      __syncthreads();
      const uint32_t all = sh.mask;
      if (all == 0u) {
        if (part > 0 && part < n_parts) sh.part[part * a.D + c] = half;
        hi = fmaxf(hi, bh);
        lo = fminf(lo, bl);
        __syncthreads();
        break;
      }
      __syncthreads();
      if (tid == 0) sh.mask = 0u;   // everyone has read it; the next writes follow a barrier
      if (spin >= a.spin_limit) {
        uint32_t m = all;
        for (int r = int((blockIdx.x + uint32_t(spin)) % uint32_t(__builtin_popcount(all))); r > 0; --r) m &= m - 1;
        help_tile_stats(a, h * tph + base + __builtin_ctz(m), sh);   // barriers inside
      } else {
        __builtin_amdgcn_s_sleep(2);
        __syncthreads();
      }
      ++spin;
    }
    if (part == 0) {
      float sub = half;   // the batch's subtree: its parts pairwise (1, 2 or 4 of them)
      if (n_parts == 2) sub = half + sh.part[a.D + c];
      if (n_parts == 4) sub = (half + sh.part[a.D + c]) + (sh.part[2 * a.D + c] + sh.part[3 * a.D + c]);
      pairwise_push(st, base / 32, sub);
    }
    __syncthreads();   // sh.part is read before the next batch or a helper writes it
  }
  // the parts' extremes of each channel meet in LDS; then the channel's maximum
  if (part > 0) {
    sh.ext[part * a.D + c] = ext_pack(hi, lo);
  }
  __syncthreads();
  uint32_t m = 0;
  if (part == 0) {
    for (int p = 1; p < P; ++p) {
      hi = fmaxf(hi, ext_hi(sh.ext[p * a.D + c]));
      lo = fminf(lo, ext_lo(sh.ext[p * a.D + c]));
    }
    const int levels = n_top > 32 ? __builtin_ctz(uint32_t(n_top / 32)) : 0;
    const float mean = pairwise_total(st, levels) / float(a.T);
    mu[c] = mean;
    m = max(__float_as_uint(hi - mean) & 0x7FFFFFFFu, __float_as_uint(lo - mean) & 0x7FFFFFFFu);
  }
  m = wave_max_u32(m);
  if (lane == 0) sh.red[0][wv] = m;
  __syncthreads();
  uint32_t r = 0;
  for (int i = 0; i < kQuantThreads / 64; ++i) r = max(r, sh.red[0][i]);
  __syncthreads();
  return r;
}

// One poll of the H head words: returns the number missing (the k-th missing one,
// k = seed mod the count, left in sh.pick when `help`) and their maximum in kmax.
__device__ int poll_heads(const QuantArgs &a, bool help, uint32_t seed, uint32_t &kmax, OptShared &sh) {
  constexpr int kSlotsPerThread = kMaxQuantGrid / kQuantThreads;
  const int tid = threadIdx.x;
  uint32_t k = 0, v = 0, miss = 0;
#pragma unroll
  for (int i = 0; i < kSlotsPerThread; ++i) {
    const int j = tid + i * kQuantThreads;
    if (j < a.H) {
      const uint64_t w = __hip_atomic_load(a.cmax_slots + 16 * j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (!tag_ok(a, w)) miss |= 1u << i;
      k = max(k, uint32_t(w));
    }
  }
  const int n = poll_reduce(miss, k, v, help, seed, sh);
  kmax = k;
  return n;
}

// max |x - mu| (fp32 bits) of the thread's 8 tokens of one block, per token.
__device__ __forceinline__ void centered_maxima(const uint4 (&u)[kOctet][2], const float (&mu)[16],
                                                uint32_t (&bmf)[kOctet]) {
#pragma unroll
  for (int j = 0; j < kOctet; ++j) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = max(m, __float_as_uint(elem16(u[j], i) - mu[i]) & 0x7FFFFFFFu);
    bmf[j] = m;
  }
}

// K - mean in the codec layout: per token the block's scale byte from its max
// |x - mean| (taken before s_t was known), then the codes with two-correction
// quotients (x - mean is not a bf16 value).
template <bool SCALED>
__device__ __forceinline__ void item_centered(const QuantArgs &a, const Octet &o, int b,
                                              const uint4 (&u)[kOctet][2], const float (&mu)[16],
                                              const uint32_t (&bmf)[kOctet], const TensorConsts &tc,
                                              const float2 *tab) {
  const QuantTensor &qt = a.t[o.tensor];
  const int nb = a.D >> 4;
  uint32_t scp[kOctet];
  float2 dvp[kOctet];
#pragma unroll
  for (int j = 0; j < kOctet; ++j) scp[j] = scale_code(__uint_as_float(bmf[j]), tc);
#pragma unroll
  for (int j = 0; j < kOctet; ++j) dvp[j] = tab[scp[j]];
#pragma unroll
  for (int j = 0; j < kOctet; ++j) {
    float x[16];
    unpack16(u[j], x);
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = x[i] - mu[i];
    const uint2 c = encode_token<SCALED, false>(x, dvp[j].x, dvp[j].y, tc.xs);
    if (j < o.nvalid) {
      const int64_t row = int64_t(o.h) * a.rows + o.row + j;
      *reinterpret_cast<uint2 *>(qt.codes + row * (a.D / 2) + b * 8) = c;
      qt.scales[row * nb + b] = uint8_t(scp[j]);
    }
  }
}

}  // namespace

template <bool KS, bool VA>
__global__ __launch_bounds__(kQuantThreads, 2) void quantize_options_kernel(QuantArgs a) {
  __shared__ OptShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nb = a.D >> 4;
  const int opt = kQuantThreads / nb;         // octets per tile
  const int b = tid % nb, o = tid / nb;
  const int nk = a.H * a.tiles_per_head;      // K tiles come first
  const int tile = blockIdx.x;
  const bool is_k = tile < nk;

  uint4 u[kOctet][2];
  const Octet oc = locate_octet(a, tile, min(o, opt - 1));
  load_octet(a, oc, b, u);

  float st;
  float mu[16];
  uint32_t bm[kOctet];    // per token: the block's max |x| (bf16 bits) or max |x - mean| (fp32 bits)
  if (KS && is_k) {
    own_tile_stats(a, tile, oc, o, b, u, sh);
    // The tile is read again for the encode (from the caches) once the tensor maximum
    // is known: holding it in registers through the statistics exchange would spill.
    // First the own head's statistics; then, while head words are missing, wait or
    // (past the limit) compute a missing head's word (one call site of head_stats).
    int head = oc.h;
    uint32_t kmax = 0;
    for (int spin = -1;; ++spin) {
      if (head >= 0) {
        const uint32_t m = head_stats(a, head, spin < 0 ? sh.mu : sh.mu_help, sh);
        if (tid == 0) __hip_atomic_store(a.cmax_slots + 16 * head, tagged(a, m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (spin < 0 && tile % a.tiles_per_head == 0 && tid < a.D) a.k_mean_out[int64_t(oc.h) * a.D + tid] = sh.mu[tid];
      const bool help = spin >= a.spin_limit;
      if (poll_heads(a, help, blockIdx.x + uint32_t(spin), kmax, sh) == 0) break;
      head = help ? sh.pick : -1;
      if (!help) __builtin_amdgcn_s_sleep(2);
    }
    st = __uint_as_float(kmax) / 2688.0f;
    load_octet(a, oc, b, u);
#pragma unroll
    for (int i = 0; i < 16; ++i) mu[i] = sh.mu[16 * b + i];
    centered_maxima(u, mu, bm);
  } else {
    uint32_t mx = 0;
#pragma unroll
    for (int j = 0; j < kOctet; ++j) {
      bm[j] = block_max_bits(u[j]);
      mx = max(mx, bm[j]);
    }
    const uint32_t mk = wave_max_u32(is_k ? mx : 0u), mv = wave_max_u32(is_k ? 0u : mx);
    if (lane == 0) {
      sh.red[0][wv] = mk;
      sh.red[1][wv] = mv;
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t rk = 0, rv = 0;
      for (int i = 0; i < kQuantThreads / 64; ++i) {
        rk = max(rk, sh.red[0][i]);
        rv = max(rv, sh.red[1][i]);
      }
      const uint64_t word = (a.epoch << 30) | (uint64_t(rk) << 15) | uint64_t(rv);
      __hip_atomic_store(&a.ws->slot[tile], word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    uint32_t gk, gv;
    wait_maxima(a, is_k ? 0 : nk, is_k ? nk : 2 * nk, gk, gv, sh);
    st = bf16_bits_to_float(is_k ? gk : gv) / 2688.0f;
  }

  if ((tile == 0 || tile == nk) && tid == 0) *a.t[is_k ? 0 : 1].tensor_scale = st;
  const TensorConsts tc = tensor_consts(st);
  for (int e = tid; e < kScaleCodes; e += kQuantThreads) sh.tab[e] = divisor_entry(e, st, tc.xs);
  __syncthreads();
  if (is_k) {
    if constexpr (KS) {
      if (tc.xs == 1.0f) item_centered<false>(a, oc, b, u, mu, bm, tc, sh.tab);
      else item_centered<true>(a, oc, b, u, mu, bm, tc, sh.tab);
    } else {
      if (tc.xs == 1.0f) item_canonical<false>(a, oc, b, u, tc, sh.tab, bm);
      else item_canonical<true>(a, oc, b, u, tc, sh.tab, bm);
    }
  } else {
    // with K-smoothing the kernel holds more registers elsewhere: kept codes would spill
    if (tc.xs == 1.0f) item_transposed<false, VA, !KS>(a, oc, b, u, tc, sh.tab, bm);
    else item_transposed<true, VA, !KS>(a, oc, b, u, tc, sh.tab, bm);
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

namespace {
// Tile shape of the quantize kernels (sets a.tile_tokens, tiles_per_head, total_tiles).
int quantize_tiles(QuantArgs &a) {
  const int nb = a.D / 16;
  if (nb < 1 || nb > kQuantThreads || a.tokens_per_frame < 1 || a.n_frames < 1) return NVFP4KV_EINVAL;
  a.tile_tokens = kOctet * (kQuantThreads / nb);
  a.tiles_per_head = int32_t((int64_t(a.T) + a.tile_tokens - 1) / a.tile_tokens);
  const int64_t total = int64_t(a.n_tensors) * a.H * a.tiles_per_head;
  if (total >= (int64_t(1) << 31)) return NVFP4KV_EINVAL;
  a.total_tiles = int32_t(total);
  return NVFP4KV_OK;
}

// 1 when the single-pass kernel takes this launch: an epoch is given and the grid (one
// workgroup per tile) fits on the current device at once by the occupancy API.
int fused_fits(const QuantArgs &a, int dev) {
  if (a.epoch == 0 || a.total_tiles > kMaxQuantGrid || dev < 0 || dev >= kMaxDevices) return 0;
  if (g_fused_per_cu[dev] == 0) {
    int per = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, quantize_fused_kernel, kQuantThreads, 0) != hipSuccess)
      return NVFP4KV_EHIP;
    g_fused_per_cu[dev] = per > 0 ? per : -1;
  }
  return g_fused_per_cu[dev] > 0 && a.total_tiles <= int64_t(cu_count(dev)) * g_fused_per_cu[dev] ? 1 : 0;
}
}  // namespace

int quantize_single_pass(const QuantArgs &in) {
  QuantArgs a = in;
  if (int rc = quantize_tiles(a)) return rc;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4KV_EHIP;
  return fused_fits(a, dev);
}

int launch_quantize(const QuantArgs &in, void *stream) {
  QuantArgs a = in;
  if (int rc = quantize_tiles(a)) return rc;
  const int64_t total = a.total_tiles;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4KV_EHIP;
  const int cus = cu_count(dev);
  const int fits = fused_fits(a, dev);
  if (fits < 0) return fits;
  if (fits) {
    hipLaunchKernelGGL(quantize_fused_kernel, dim3(unsigned(a.total_tiles)), dim3(kQuantThreads), 0, s, a);
    return NVFP4KV_HIP_OK(hipGetLastError());
  }
  // pass 1: one 1024-thread workgroup per CU (fewer for small inputs)
  const int64_t vecs = int64_t(a.H) * a.T * a.D / 8;
  int64_t g1 = (vecs + kAmaxThreads * 2 - 1) / (kAmaxThreads * 2);
  if (g1 > cus) g1 = cus;
  // the encode kernel reduces one partial per thread of its workgroup
  static_assert(kQuantThreads <= kMaxQuantGrid, "partials array holds every amax workgroup");
  if (g1 > kQuantThreads) g1 = kQuantThreads;
  if (g1 < 1) g1 = 1;
  hipLaunchKernelGGL(quantize_amax_kernel, dim3(unsigned(g1)), dim3(kAmaxThreads), 0, s, a);
  if (hipGetLastError() != hipSuccess) return NVFP4KV_EHIP;
  // pass 2: one workgroup per tile, up to 16 per CU, then a grid-stride loop
  int64_t g2 = total;
  if (g2 > int64_t(cus) * 16) g2 = int64_t(cus) * 16;
  const bool opt = a.t[0].mean != nullptr || (a.n_tensors > 1 && a.t[1].adaptive);
  if (opt)
    hipLaunchKernelGGL(quantize_encode_kernel<true>, dim3(unsigned(g2)), dim3(kQuantThreads), 0, s, a, int(g1));
  else
    hipLaunchKernelGGL(quantize_encode_kernel<false>, dim3(unsigned(g2)), dim3(kQuantThreads), 0, s, a, int(g1));
  return NVFP4KV_HIP_OK(hipGetLastError());
}

namespace {
// Co-resident workgroups per CU of each options instantiation (0: not yet asked, -1: none).
int g_opt_per_cu[kMaxDevices][3];

template <bool KS, bool VA>
int options_per_cu(int dev) {
  int &slot = g_opt_per_cu[dev][(KS ? 1 : 0) + (VA ? 2 : 0) - 1];
  if (slot == 0) {
    int per = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, quantize_options_kernel<KS, VA>, kQuantThreads, 0) !=
        hipSuccess)
      return NVFP4KV_EHIP;
    slot = per > 0 ? per : -1;
  }
  return slot;
}

// 1 when the options single pass takes this launch (a.tile_tokens etc. already set).
int options_fits(const QuantArgs &a, bool ks, bool va, int dev) {
  if (!ks && !va) return 0;
  if (a.epoch == 0 || uint32_t(a.epoch) == 0 || a.n_tensors != 2 || a.total_tiles > kMaxQuantGrid) return 0;
  if (dev < 0 || dev >= kMaxDevices) return 0;
  if (ks) {
    if (!a.sum_slots || !a.cmax_slots || !a.k_mean_out || a.D > 128) return 0;
    // the top of the means tree: at most 2^11 nodes per head
    int64_t n_in = 1;
    while (n_in < a.T) n_in *= 2;
    const int64_t leaves = n_in < a.tile_tokens ? n_in : a.tile_tokens;
    if (n_in / leaves > 2048) return 0;
  }
  const int per = ks ? (va ? options_per_cu<true, true>(dev) : options_per_cu<true, false>(dev))
                     : options_per_cu<false, true>(dev);
  if (per < 0 && per != -1) return per;
  return per > 0 && a.total_tiles <= int64_t(cu_count(dev)) * per ? 1 : 0;
}
}  // namespace

int quantize_options_single_pass(const QuantArgs &in, bool k_smooth, bool v_adaptive) {
  QuantArgs a = in;
  if (int rc = quantize_tiles(a)) return rc;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4KV_EHIP;
  // the cache gives the slots to every K-smoothing append; stand-ins for the check
  static uint64_t probe;
  static float probe_mean;
  if (k_smooth) {
    a.sum_slots = a.cmax_slots = &probe;
    a.k_mean_out = &probe_mean;
  }
  return options_fits(a, k_smooth, v_adaptive, dev);
}

int launch_quantize_options(const QuantArgs &in, float *k_mean, float *kmean_ws, void *stream) {
  QuantArgs a = in;
  if (int rc = quantize_tiles(a)) return rc;
  const bool ks = k_mean != nullptr, va = a.n_tensors > 1 && a.t[1].adaptive != 0;
  a.k_mean_out = k_mean;
  a.t[0].mean = k_mean;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4KV_EHIP;
  const int fits = options_fits(a, ks, va, dev);
  if (fits < 0) return fits;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (fits) {
    const dim3 grid(unsigned(a.total_tiles)), block(kQuantThreads);
    if (ks && va) hipLaunchKernelGGL((quantize_options_kernel<true, true>), grid, block, 0, s, a);
    else if (ks) hipLaunchKernelGGL((quantize_options_kernel<true, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((quantize_options_kernel<false, true>), grid, block, 0, s, a);
    return NVFP4KV_HIP_OK(hipGetLastError());
  }
  // the two passes, after the channel means
  if (ks) {
    const int rm = launch_channel_mean(a.t[0].src, a.H, a.T, a.D, k_mean, kmean_ws, stream);
    if (rm != NVFP4KV_OK) return rm;
  }
  a.epoch = 0;
  return launch_quantize(a, stream);
}

// ---- same-size streaming reference (a measurement hook, not part of the method)
// Reads two bf16 tensors of n elements and writes, per tensor, n/2 code bytes and
// n/16 scale bytes in the codec layout, with the quantizer's tiling (one octet of
// tokens x one 16-element block per thread, one 256-token x D tile per workgroup, one
// workgroup per tile) and a trivial per-element operation: the same bytes moved with
// no exchange between workgroups and almost no arithmetic, i.e. the time this
// transfer size allows.
__global__ __launch_bounds__(kQuantThreads) void stream_reference_kernel(QuantArgs a) {
  const int tid = threadIdx.x;
  const int nb = a.D >> 4;
  const int opt = kQuantThreads / nb;
  const int b = tid % nb, o = tid / nb;
  const Octet oc = locate_octet(a, blockIdx.x, min(o, opt - 1));
  uint4 u[kOctet][2];
  load_octet(a, oc, b, u);
  if (o >= opt) return;
  const QuantTensor &qt = a.t[oc.tensor];
#pragma unroll
  for (int j = 0; j < kOctet; ++j) {
    // code nibble = the top 4 bits of each bf16 (sign and 3 exponent bits); scale
    // byte = the block's largest exponent byte
    uint32_t c[2] = {0u, 0u}, e = 0u;
    const uint32_t w[8] = {u[j][0].x, u[j][0].y, u[j][0].z, u[j][0].w, u[j][1].x, u[j][1].y, u[j][1].z, u[j][1].w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      c[k >> 2] |= (((w[k] >> 12) & 0xFu) | ((w[k] >> 24) & 0xF0u)) << (8 * (k & 3));
      e = max(e, (w[k] >> 7) & 0xFFu);
    }
    if (j < oc.nvalid) {
      const int64_t row = int64_t(oc.h) * a.rows + oc.row + j;
      *reinterpret_cast<uint2 *>(qt.codes + row * (a.D / 2) + b * 8) = make_uint2(c[0], c[1]);
      qt.scales[row * nb + b] = uint8_t(e);
    }
  }
}

int launch_stream_reference(const QuantArgs &in, void *stream) {
  QuantArgs a = in;
  if (int rc = quantize_tiles(a)) return rc;
  hipLaunchKernelGGL(stream_reference_kernel, dim3(unsigned(a.total_tiles)), dim3(kQuantThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), a);
  return NVFP4KV_HIP_OK(hipGetLastError());
}

// ---- the codec without a caller workspace
// File-scope device array standing in for the workspace: one copy per GPU, at its
// own address on each, resolved once per device with hipGetSymbolAddress (in host
// code the array's name is only a host-side stand-in, never a device address).  The
// two-pass codec writes every partial maximum it reads within the same call, so
// nothing in it has to start zeroed; calls that overlap on one GPU share it and race.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
std::atomic<void *> g_scratch_ptr[kMaxDevices];

void *scratch_for_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}
}  // namespace

int launch_quantize_noalloc(const QuantArgs &in, void *stream) {
  // the codec's workspace need does not grow with the input (one partial maximum per
  // workgroup of the first pass, at most kQuantThreads of them), so the fixed array
  // always suffices; the check keeps that true if the launch shape ever changes
  static_assert(sizeof(QuantWorkspace) <= kNoAllocScratchBytes, "codec workspace fits the scratch array");
  if (in.epoch != 0) return NVFP4KV_EINVAL;   // the single-pass append needs zeroed epoch slots
  void *p = scratch_for_current_device();
  if (!p) return NVFP4KV_EHIP;
  QuantArgs a = in;
  a.ws = reinterpret_cast<QuantWorkspace *>(p);
  return launch_quantize(a, stream);
}

}  // namespace nvfp4kv
