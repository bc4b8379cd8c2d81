// Chunk attention over the NVFP4 sink + window cache plus the chunk's own bf16 K/V,
// for gfx950.
//
// Computes, per head, out = softmax(q K^T * scale) V with K/V = [cache ; own] and no
// mask (paper text section 2.1: the noisy chunk attends to the clean history and
// its own tokens; section 4.2: the history is the sink + window cache; section 1 and
// the reading note's "The inference infrastructure": the NVFP4 cache is dequantized
// inside the attention kernel).
//
// Design for CDNA4:
//  * A workgroup owns kWaves x 32 queries of one head (8 waves = 256 queries for
//    D = 128: one workgroup per CU, two waves per SIMD; 4 waves for D = 64).  Keys
//    stream in tiles of 64.  Each tile is dequantized ONCE per workgroup into LDS,
//    double-buffered, so a wave's share of the dequantization work shrinks as the
//    workgroup grows.
//  * Software pipeline with one barrier per tile: a wave issues the QK^T MFMAs of
//    tile t, then dequantizes its share of tile t+1 into the other LDS buffer (VALU
//    work that runs while the matrix cores execute), issues the global loads of the
//    packed bytes of tile t+2, and only then takes the softmax and PV of tile t.
//  * Dequantization uses the CDNA4 converts v_cvt_scalef32_pk_f16_fp4 and
//    _pk_f16_fp8 with scale 1.0 (exact: E2M1 and E4M3 values are fp16 numbers) and
//    one v_pk_mul_f16 per two elements.  E2M1 x E4M3 has at most 6 significant bits
//    and lies in [2^-10, 2688], so the product is exact in fp16.  The fp32 tensor
//    scales stay outside the matrix cores: s_K folds into the logit multiplier,
//    s_V into the units of the output accumulator.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_f16: K from LDS as the A operand, Q in
//    registers as the B operand.  Q is held in fp16 with a per-query power-of-two
//    scale (row maximum mapped into [2^14, 2^15)); bf16 values map exactly unless an
//    element is more than ~2^28 below its row maximum.  The scale folds into the
//    per-query logit multiplier, which is a per-lane value: in this layout each lane
//    owns one query column and 16 keys, which is also exactly the lane layout of the
//    B operand of O^T = V^T P^T, so P never leaves registers.  V is stored in LDS as
//    V^T with the keys of each 16-key group permuted to match.
//  * The own segment runs after the cache with Q reloaded as bf16, K_own and V_own
//    in bf16 as given (v_mfma_f32_32x32x16_bf16 for QK^T and PV, P rounded to bf16
//    nearest-even).  V_own is prefetched into registers one tile ahead (transposed
//    there); K_own is fetched at the top of the iteration that stores it.
//  * Online softmax in fp32 with exp2 (log2 e folded into the multiplier).  The
//    running maximum is raised only when a tile's maximum exceeds it by more than
//    8 (in log2 units), so the accumulator rescale is rare; probabilities are then
//    bounded by 2^8, well inside fp16.  Row sums are taken from the fp16-rounded
//    probabilities that enter the PV product.
//  * Work distribution (stream-K style): the (query block, key tile) pairs of all
//    heads form one list, weighted by the measured cost of each tile kind, that is
//    cut into one equal share per resident workgroup (every CU busy, whatever the
//    number of query blocks; the list arithmetic is attn_plan.h, which a CPU check
//    shares).  A share usually ends inside a query block.  Each
//    workgroup walks its share from the end, so it starts at key tile 0 of its last
//    block (keeping all workgroups of a head in step, for L2 reuse) and publishes
//    that range's partial result (unnormalized output, running max, row sum); the
//    workgroup holding a cut block's last tiles processes them last and merges the
//    partials, published long before.
//    Partials pass through memory (each XCD has its own L2): one L2 write-back per
//    publishing workgroup, device-scope reads by the merging one; the wait
//    for a partial is bounded, after which the merging workgroup processes the
//    block's remaining tiles itself.
//  * Workgroups are numbered so that each XCD (own L2) runs a contiguous run of
//    shares, i.e. mostly one head's keys.

#include "device_common.h"
#define NVFP4KV_PLAN_FN __host__ __device__ __forceinline__
#include "attn_plan.h"

namespace nvfp4kv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

namespace {

constexpr int kBN = kAttnKeys;  // keys per tile
constexpr int kQW = 32;        // queries per wave
constexpr float kLazy = 8.0f;  // log2 headroom before the running max is raised

// Workgroup shape per head_dim.
template <int D>
struct Cfg {
  static constexpr int kWaves = D >= 128 ? 8 : 4;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBM = kWaves * kQW;             // queries per workgroup
  static constexpr int kWgPerCu = kWaves == 8 ? 1 : 2;
};

// ---------------------------------------------------------------- LDS layouts
// Rows are padded by 16 bytes: for Ks (row stride 2D+16 B = 68 dwords at D=128) and
// Vs (144 B = 36 dwords) the 16 lanes of one ds_read_b128 phase, which read 16
// consecutive rows at the same column, land on 16 distinct 4-bank groups; and every
// operand address is a per-lane base plus a compile-time offset.
// Ks: [kBN][D + 8] 16-bit (K rows).
template <int D>
__device__ __forceinline__ int ks_off(int row, int chunk) {
  return row * (D + 8) + (chunk << 3);
}
template <int D>
constexpr int kKsElems = kBN * (D + 8);
// MXFP4 with MX-scaled QK^T: the Ks buffer holds the tile's raw K codes, rows of
// D/2 bytes padded by 16 (8 consecutive rows of a b128 read phase land on distinct
// banks: a row stride of 80 or 48 bytes moves 20 or 12 banks), then the E8M0
// scale bytes [kBN][D/32].
template <int D>
constexpr int kRawRow = D / 2 + 16;
template <int D>
constexpr int kRawScales = kBN * kRawRow<D>;

// Vs: [D][kBN + 8] 16-bit (V^T rows).
__device__ __forceinline__ int vs_off(int row, int chunk) {
  return row * (kBN + 8) + (chunk << 3);
}
template <int D>
constexpr int kVsElems = D * (kBN + 8);

__device__ __forceinline__ uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// two fp32 -> packed fp16, round toward zero (exact for values fp16 represents)
__device__ __forceinline__ f16x2 pkrtz(float a, float b) {
  return __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// E2M1 pair (byte SEL of w) -> fp16x2, exact
template <int SEL>
__device__ __forceinline__ f16x2 fp4x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}
// E4M3 pair (word HI of w) -> fp16x2, exact
template <bool HI>
__device__ __forceinline__ f16x2 fp8x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// Packed bytes of one cache tile held by one thread between its load and its
// dequantization: kTasks (key, 16-element block) K tasks and kTasks (d, 16-key
// group) V tasks.
template <int D>
struct Packed {
  static constexpr int kTasks = kBN * (D / 16) / Cfg<D>::kThreads;
  static_assert(kTasks >= 1 && kTasks * Cfg<D>::kThreads == kBN * (D / 16), "task split");
  uint32_t kc[kTasks][2];    // 16 K codes
  uint32_t ks[kTasks];       // K scale byte
  uint32_t vc[kTasks][2];    // 16 V codes (keys 0-7, 8-15)
  uint32_t vs[kTasks][4];    // 16 V scale bytes
};

// One head's cache planes (uniform pointers: the loads below use a scalar base and
// a 32-bit per-lane offset).
struct HeadPlanes {
  const uint8_t *kc, *ks, *vc, *vs;
  uint32_t rows;
};

template <int D, bool MX>
__device__ __forceinline__ HeadPlanes head_planes(const AttnArgs &a, int h) {
  constexpr int nb = D / (MX ? 32 : 16);   // block scales per token
  HeadPlanes p;
  p.rows = uint32_t(a.rows);
  p.kc = a.kcodes + size_t(h) * a.rows * (D / 2);
  p.ks = a.kscales + size_t(h) * a.rows * nb;
  p.vc = a.vcodes + size_t(h) * D * (a.rows / 2);
  p.vs = a.vscales + size_t(h) * nb * a.rows;
  return p;
}

// Loads are unconditional: keys past `nval` (a multiple of 8, >= 8) re-read the
// tile's last valid key or 8-key group, so every loaded byte is a valid code or
// scale; those keys are masked out of the softmax.
template <int D, bool MX>
__device__ __forceinline__ void load_packed(const HeadPlanes &hp, uint32_t tok, int nval,
                                            Packed<D> &p) {
  constexpr int nb = D / 16;                 // 16-element K tasks per key
  constexpr int nbs = D / (MX ? 32 : 16);    // block scales per key
#pragma unroll
  for (int i = 0; i < Packed<D>::kTasks; ++i) {
    const int t = threadIdx.x + i * Cfg<D>::kThreads;
    // K task: (key, block) = (t / nb, t % nb)
    {
      const int key = min(t / nb, nval - 1), b = t % nb;
      const uint32_t row = tok + uint32_t(key);
      const uint2 c = *reinterpret_cast<const uint2 *>(hp.kc + (row * (D / 2) + uint32_t(b) * 8));
      p.kc[i][0] = c.x;
      p.kc[i][1] = c.y;
      p.ks[i] = hp.ks[row * nbs + uint32_t(MX ? b >> 1 : b)];
    }
    // V task: (d, 16-key group) = (t / 4, t % 4); two 8-key halves
    {
      const int d = t >> 2, g = t & 3;
      const int last8 = (nval >> 3) - 1;                 // last valid 8-key group
      const uint32_t h0 = uint32_t(min(2 * g, last8)), h1 = uint32_t(min(2 * g + 1, last8));
      const uint32_t cbase = uint32_t(d) * (hp.rows / 2) + (tok >> 1);
      const uint32_t sbase = uint32_t(d >> (MX ? 5 : 4)) * hp.rows + tok;
      const uint32_t *cp = reinterpret_cast<const uint32_t *>(hp.vc + cbase);
      const uint2 *sp = reinterpret_cast<const uint2 *>(hp.vs + sbase);
      p.vc[i][0] = cp[h0];
      p.vc[i][1] = cp[h1];
      const uint2 s0 = sp[h0], s1 = sp[h1];
      p.vs[i][0] = s0.x;
      p.vs[i][1] = s0.y;
      p.vs[i][2] = s1.x;
      p.vs[i][3] = s1.y;
    }
  }
}

// 16 E2M1 codes (w0: keys/elements 0-7, w1: 8-15) times 8 fp16 scale pairs ->
// 8 fp16 pairs in natural order.
__device__ __forceinline__ void dequant16(uint32_t w0, uint32_t w1, const f16x2 (&s)[8],
                                          uint32_t (&o)[8]) {
  o[0] = as_u32(fp4x2<0>(w0) * s[0]);
  o[1] = as_u32(fp4x2<1>(w0) * s[1]);
  o[2] = as_u32(fp4x2<2>(w0) * s[2]);
  o[3] = as_u32(fp4x2<3>(w0) * s[3]);
  o[4] = as_u32(fp4x2<0>(w1) * s[4]);
  o[5] = as_u32(fp4x2<1>(w1) * s[5]);
  o[6] = as_u32(fp4x2<2>(w1) * s[6]);
  o[7] = as_u32(fp4x2<3>(w1) * s[7]);
}

// MXFP4 tiles dequantize to bf16 (exact: E2M1 x 2^e has at most 2 significant bits and
// bf16 spans every scale the format produces for bf16 inputs).  The E8M0 byte s goes
// into the converts' fp32 scale operand as its exponent field: the converts multiply
// by 2^(exponent field - 127), which is exactly the E8M0 value, and read nothing else
// of the operand (checked on gfx950 for every byte, with the sign and mantissa bits
// set), so one shift places byte `byte` of a word of four scale bytes.
template <int BYTE>
__device__ __forceinline__ float e8m0_operand(uint32_t word) {
  return __uint_as_float(BYTE < 3 ? word << (23 - 8 * BYTE) : word >> 1);
}
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_bf16(uint32_t w, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL));
}
// keys (2 SEL, 2 SEL + 1) of word w, each with its own block scale: the low half
// from the convert with the first key's scale, the high half from the second's
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_bf16_2s(uint32_t w, float sa, float sb) {
  return (fp4x2_bf16<SEL>(w, sa) & 0xFFFFu) | (fp4x2_bf16<SEL>(w, sb) & 0xFFFF0000u);
}

template <int D, bool MX, bool MXS = false>
__device__ __forceinline__ void dequant_store(const Packed<D> &p, uint16_t *Ks, uint16_t *Vs) {
  constexpr int nb = D / 16;
  if constexpr (MX) {
#pragma unroll
    for (int i = 0; i < Packed<D>::kTasks; ++i) {
      const int t = threadIdx.x + i * Cfg<D>::kThreads;
      if constexpr (MXS) {
        // K stays E2M1 codes for the MX-scaled matrix cores: copy the 8 code bytes
        // and (one thread per 32-element block) the block's E8M0 byte
        const int key = t / nb, b = t % nb;
        uint8_t *raw = reinterpret_cast<uint8_t *>(Ks);
        *reinterpret_cast<uint2 *>(raw + key * kRawRow<D> + 8 * b) = make_uint2(p.kc[i][0], p.kc[i][1]);
        if ((b & 1) == 0) raw[kRawScales<D> + key * (D / 32) + (b >> 1)] = uint8_t(p.ks[i]);
      } else {
        const int key = t / nb, b = t % nb;
        const float sk = e8m0_operand<0>(p.ks[i]);
        const uint32_t w0 = p.kc[i][0], w1 = p.kc[i][1];
        *reinterpret_cast<uint4 *>(Ks + ks_off<D>(key, 2 * b)) =
            make_uint4(fp4x2_bf16<0>(w0, sk), fp4x2_bf16<1>(w0, sk), fp4x2_bf16<2>(w0, sk), fp4x2_bf16<3>(w0, sk));
        *reinterpret_cast<uint4 *>(Ks + ks_off<D>(key, 2 * b + 1)) =
            make_uint4(fp4x2_bf16<0>(w1, sk), fp4x2_bf16<1>(w1, sk), fp4x2_bf16<2>(w1, sk), fp4x2_bf16<3>(w1, sk));
      }
      {
        const int d = t >> 2, g = t & 3;
        const uint32_t w0 = p.vc[i][0], w1 = p.vc[i][1];
        uint32_t o[8];
        o[0] = fp4x2_bf16_2s<0>(w0, e8m0_operand<0>(p.vs[i][0]), e8m0_operand<1>(p.vs[i][0]));
        o[1] = fp4x2_bf16_2s<1>(w0, e8m0_operand<2>(p.vs[i][0]), e8m0_operand<3>(p.vs[i][0]));
        o[2] = fp4x2_bf16_2s<2>(w0, e8m0_operand<0>(p.vs[i][1]), e8m0_operand<1>(p.vs[i][1]));
        o[3] = fp4x2_bf16_2s<3>(w0, e8m0_operand<2>(p.vs[i][1]), e8m0_operand<3>(p.vs[i][1]));
        o[4] = fp4x2_bf16_2s<0>(w1, e8m0_operand<0>(p.vs[i][2]), e8m0_operand<1>(p.vs[i][2]));
        o[5] = fp4x2_bf16_2s<1>(w1, e8m0_operand<2>(p.vs[i][2]), e8m0_operand<3>(p.vs[i][2]));
        o[6] = fp4x2_bf16_2s<2>(w1, e8m0_operand<0>(p.vs[i][3]), e8m0_operand<1>(p.vs[i][3]));
        o[7] = fp4x2_bf16_2s<3>(w1, e8m0_operand<2>(p.vs[i][3]), e8m0_operand<3>(p.vs[i][3]));
        *reinterpret_cast<uint4 *>(Vs + vs_off(d, 2 * g)) = make_uint4(o[0], o[1], o[4], o[5]);
        *reinterpret_cast<uint4 *>(Vs + vs_off(d, 2 * g + 1)) = make_uint4(o[2], o[3], o[6], o[7]);
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < Packed<D>::kTasks; ++i) {
    const int t = threadIdx.x + i * Cfg<D>::kThreads;
    {
      const int key = t / nb, b = t % nb;
      const f16x2 s0 = fp8x2<false>(p.ks[i] | (p.ks[i] << 8));   // (s, s)
      const f16x2 sa[8] = {s0, s0, s0, s0, s0, s0, s0, s0};
      uint32_t o[8];
      dequant16(p.kc[i][0], p.kc[i][1], sa, o);
      *reinterpret_cast<uint4 *>(Ks + ks_off<D>(key, 2 * b)) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4 *>(Ks + ks_off<D>(key, 2 * b + 1)) = make_uint4(o[4], o[5], o[6], o[7]);
    }
    {
      const int d = t >> 2, g = t & 3;
      const f16x2 s[8] = {fp8x2<false>(p.vs[i][0]), fp8x2<true>(p.vs[i][0]), fp8x2<false>(p.vs[i][1]),
                          fp8x2<true>(p.vs[i][1]), fp8x2<false>(p.vs[i][2]), fp8x2<true>(p.vs[i][2]),
                          fp8x2<false>(p.vs[i][3]), fp8x2<true>(p.vs[i][3])};
      uint32_t o[8];
      dequant16(p.vc[i][0], p.vc[i][1], s, o);
      // physical key order within the 16-key group: pairs {0,1,4,5} then {2,3,6,7}
      *reinterpret_cast<uint4 *>(Vs + vs_off(d, 2 * g)) = make_uint4(o[0], o[1], o[4], o[5]);
      *reinterpret_cast<uint4 *>(Vs + vs_off(d, 2 * g + 1)) = make_uint4(o[2], o[3], o[6], o[7]);
    }
  }
}

// Own-segment tiles: K_own rows (bf16) are copied to LDS as they are; V_own is
// transposed into fp16 V^T rows with the same permuted key order as the cache.
template <int D>
__device__ __forceinline__ void load_own_k(const AttnArgs &a, int h, int tok, int nval, uint4 (&k)[2]) {
  constexpr int cpk = D / 16;                   // thread pairs of 16-byte chunks per key
  static_assert(kBN * cpk == Cfg<D>::kThreads, "own K split");
  const int t = threadIdx.x;
  const uint16_t *kbase = a.k_own + size_t(h) * a.n_q * D;
  const int key = min(t / cpk, nval - 1), c = t % cpk;   // past the end: re-read a valid key
  const uint4 *src = reinterpret_cast<const uint4 *>(kbase + (uint32_t(tok + key) * D + uint32_t(c) * 16));
  k[0] = src[0];
  k[1] = src[1];
}

template <int D>
__device__ __forceinline__ void load_own_v(const AttnArgs &a, int h, int tok, int nval, uint32_t (&v)[8]) {
  static_assert((D / 2) * (kBN / 8) == Cfg<D>::kThreads, "own V split");
  const int t = threadIdx.x;
  const uint16_t *vbase = a.v_own + size_t(h) * a.n_q * D;
  const int dp = t % (D / 2), g = t / (D / 2);            // d pair, 8-key group
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int key = min(g * 8 + k, nval - 1);
    v[k] = *reinterpret_cast<const uint32_t *>(vbase + (uint32_t(tok + key) * D + uint32_t(2 * dp)));
  }
}

template <int D>
__device__ __forceinline__ void store_own_k(const uint4 (&k)[2], uint16_t *Ks) {
  constexpr int cpk = D / 16;
  const int t = threadIdx.x;
  const int key = t / cpk, c = t % cpk;
  *reinterpret_cast<uint4 *>(Ks + ks_off<D>(key, 2 * c)) = k[0];
  *reinterpret_cast<uint4 *>(Ks + ks_off<D>(key, 2 * c + 1)) = k[1];
}

// V^T as bf16 (the values as given) in the permuted key order
template <int D>
__device__ __forceinline__ void store_own_v(const uint32_t (&v)[8], uint16_t *Vs) {
  const int t = threadIdx.x;
  const int dp = t % (D / 2), g = t / (D / 2);
  const int d = 2 * dp;
  uint32_t lo[4], hi[4];   // bf16 pairs (key 2i, key 2i+1) of row d and of row d+1
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo[i] = (v[2 * i] & 0xFFFFu) | (v[2 * i + 1] << 16);
    hi[i] = (v[2 * i] >> 16) | (v[2 * i + 1] & 0xFFFF0000u);
  }
  // 8-key group g is half (g & 1) of 16-key group g >> 1: its pairs (0,1),(2,3) go
  // to chunk 2(g>>1) and its pairs (4,5),(6,7) to chunk 2(g>>1)+1, at 8-byte offset
  // 8 (g & 1) within each chunk
  const int g16 = g >> 1, off = 4 * (g & 1);
  *reinterpret_cast<uint2 *>(Vs + vs_off(d, 2 * g16) + off) = make_uint2(lo[0], lo[1]);
  *reinterpret_cast<uint2 *>(Vs + vs_off(d, 2 * g16 + 1) + off) = make_uint2(lo[2], lo[3]);
  *reinterpret_cast<uint2 *>(Vs + vs_off(d + 1, 2 * g16) + off) = make_uint2(hi[0], hi[1]);
  *reinterpret_cast<uint2 *>(Vs + vs_off(d + 1, 2 * g16 + 1) + off) = make_uint2(hi[2], hi[3]);
}

// Value of lane l ^ 32 combined with lane l's own, through the lane-half swap
// (no LDS round trip); both halves get the same result.
__device__ __forceinline__ float other_half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float other_half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ uint32_t other_half_umax(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max(uint32_t(r[0]), uint32_t(r[1]));
}

struct Softmax {
  float m;      // running max (log2 units) of the lane's query
  float l;      // partial row sum over this lane's keys
};

// S^T = K Q^T for the wave's 32 queries (all K fragments read before the MFMAs).
template <int D, bool BF16>
__device__ __forceinline__ void qk_tile(const uint16_t *Ks, const u32x4 (&qr)[D / 16], f32x16 (&s)[2]) {
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  u32x4 kf[2][D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      kf[kb][st] = *reinterpret_cast<const u32x4 *>(Ks + ks_off<D>(kb * 32 + l32, 2 * st + half));
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (BF16)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, kf[kb][st]), __builtin_bit_cast(bf16x8, qr[st]), s[kb], 0, 0, 0);
      else
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
            __builtin_bit_cast(f16x8, kf[kb][st]), __builtin_bit_cast(f16x8, qr[st]), s[kb], 0, 0, 0);
    }
}

// ---- MX-scaled QK^T (MXFP4 cache, queries in MXFP8)
// v_mfma_scale_f32_32x32x64_f8f6f4 with A = the K tile's E2M1 codes and B = the
// queries in E4M3, both with E8M0 scales per 32 elements of the reduction.  Operand
// layouts (checked on gfx950 with one-hot probes): for E2M1, lane (row, h) holds the
// 32 elements 32h + [0, 32) of the 64-wide k-step and its scale operand scales all of
// them; for E4M3, lane (column, h) holds bytes 0-15 = elements 16h + [0, 16) and
// bytes 16-31 = 32 + 16h + [0, 16), and the elements of 32-block c are scaled by
// the operand of lane (column, c).  The op_sel immediate picks the operand's byte.

typedef short short2_ __attribute__((ext_vector_type(2)));

// The wave's queries as MXFP8 B operands: q[s] for k-step s, and one scale operand
// per lane whose byte 2s is the E8M0 byte of block 2s + h.
template <int D>
struct QFp8 {
  i32x8 q[D / 64];
  uint32_t scale;
};

// E8M0 exponent of an E4M3 block whose largest |x| has the bf16 bit pattern m:
// floor(log2 m) - 8 (448 = 1.75 * 2^8), clamped to [-127, 127]; -127 for zero.
__device__ __forceinline__ int e4m3_block_exponent(uint32_t m) {
  const int ef = int(m >> 7);
  const int fl = ef > 0 ? ef - 127 : -133 + (31 - __builtin_clz(m | 1u));
  return m == 0 ? -127 : max(-127, min(127, fl - 8));
}

template <int D>
__device__ __forceinline__ void quantize_q_mxfp8(const AttnArgs &a, int h, int q0, QFp8<D> &qf) {
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  const int qi = q0 + l32;
  const bool ok = qi < a.n_q;
  const uint16_t *qp = a.q + (int64_t(h) * a.n_q + (ok ? qi : 0)) * D + 16 * half;
  qf.scale = 0;
#pragma unroll
  for (int st = 0; st < D / 64; ++st) {
    uint32_t out[8];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      // 16 values d = 64 st + 32 c + 16 h + [0, 16) of block 2 st + c; the other 16 of
      // the block are the other lane half's
      const uint4 *src = reinterpret_cast<const uint4 *>(qp + 64 * st + 32 * c);
      const uint4 u0 = ok ? src[0] : make_uint4(0, 0, 0, 0), u1 = ok ? src[1] : make_uint4(0, 0, 0, 0);
      const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
      uint32_t m = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) m = max(m, max(w[k] & 0x7FFFu, (w[k] >> 16) & 0x7FFFu));
      const int e = e4m3_block_exponent(other_half_umax(m));
      const float inv = __uint_as_float(uint32_t(127 - e) << 23);   // 2^-e, a normal fp32
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        short2_ pk = {0, 0};
        const float x0 = __uint_as_float(w[2 * k] << 16) * inv, x1 = __uint_as_float(w[2 * k] & 0xFFFF0000u) * inv;
        const float x2 = __uint_as_float(w[2 * k + 1] << 16) * inv, x3 = __uint_as_float(w[2 * k + 1] & 0xFFFF0000u) * inv;
        pk = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pk, fminf(fmaxf(x0, -448.0f), 448.0f),
                                                      fminf(fmaxf(x1, -448.0f), 448.0f), 1.0f, false);
        pk = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pk, fminf(fmaxf(x2, -448.0f), 448.0f),
                                                      fminf(fmaxf(x3, -448.0f), 448.0f), 1.0f, true);
        out[4 * c + k] = __builtin_bit_cast(uint32_t, pk);
      }
      if (c == half) qf.scale |= uint32_t(e + 127) << (16 * st);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) qf.q[st][k] = int(out[k]);
  }
}

// D += A B with A in E2M1 and B in E4M3, scaled by byte SEL of each lane's operands
template <int SEL>
__device__ __forceinline__ f32x16 mfma_e2m1_e4m3(const i32x8 &A, const i32x8 &B, const f32x16 &C, uint32_t sa,
                                                 uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, C, 4, 0, SEL, int(sa), SEL, int(sb));
}

// S^T = K Q^T for the wave's 32 queries from the tile's raw K codes.
template <int D>
__device__ __forceinline__ void qk_tile_mxs(const uint16_t *Ks, const QFp8<D> &qf, f32x16 (&s)[2]) {
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  const uint8_t *raw = reinterpret_cast<const uint8_t *>(Ks);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = kb * 32 + l32;
    // the key's E8M0 bytes, shifted so that this lane's block of k-step st is byte 2 st
    uint32_t sw;
    if constexpr (D == 128)
      sw = *reinterpret_cast<const uint32_t *>(raw + kRawScales<D> + key * 4) >> (8 * half);
    else
      sw = uint32_t(*reinterpret_cast<const uint16_t *>(raw + kRawScales<D> + key * 2)) >> (8 * half);
#pragma unroll
    for (int st = 0; st < D / 64; ++st) {
      const u32x4 c = *reinterpret_cast<const u32x4 *>(raw + key * kRawRow<D> + 32 * st + 16 * half);
      const i32x8 A = {int(c.x), int(c.y), int(c.z), int(c.w), 0, 0, 0, 0};
      s[kb] = st == 0 ? mfma_e2m1_e4m3<0>(A, qf.q[st], s[kb], sw, qf.scale)
                      : mfma_e2m1_e4m3<2>(A, qf.q[st], s[kb], sw, qf.scale);
    }
  }
}

// Online softmax of S^T, then O^T += V^T P^T.
// `bias` (per lane, i.e. per query; log2 units) is added to every logit of the
// tile: the K-smoothing term q . mean of the tile's chunk, or 0.
// PB: V^T in LDS is bf16 (MXFP4 tiles) and P enters the product as bf16 (rounded to
// nearest-even); otherwise both are fp16 (P rounded toward zero).
template <int D, bool MASK, bool PB = false>
__device__ __forceinline__ void softmax_pv(const uint16_t *Vs, f32x16 (&s)[2], float cmul, float bias,
                                           int nval, Softmax &sm, f32x16 (&acc)[D / 32]) {
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  // keys past the end of the segment (only in a segment's last tile): excluded
  // from the maximum here and given probability 0 below
  if constexpr (MASK) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (key >= nval) s[kb][r] = -INFINITY;
      }
  }
  // one chain of 3-input maxima over the lane's 32 logits
  float mx = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
#pragma unroll
  for (int j = 3; j < 31; j += 2) {
    const float x0 = j < 16 ? s[0][j] : s[1][j - 16];
    const float x1 = j + 1 < 16 ? s[0][j + 1] : s[1][j + 1 - 16];
    mx = fmaxf(fmaxf(mx, x0), x1);
  }
  mx = fmaxf(mx, s[1][15]);
  mx = other_half_max(mx);
  const float tmax = mx * cmul + bias;
  // raise the running max only when this tile exceeds it by more than kLazy
  if (__any(tmax > sm.m + kLazy)) {
    const float mnew = fmaxf(sm.m, tmax);
    const float alpha = __builtin_amdgcn_exp2f(sm.m - mnew);
    sm.m = mnew;
    sm.l *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
  }
  u32x4 vf[D / 32][4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      vf[db][ks] = *reinterpret_cast<const u32x4 *>(Vs + vs_off(db * 32 + l32, 2 * ks + half));
  const float mneg = bias - sm.m;
  float lsum = 0.0f;
  u32x4 p[4];    // [16-key step], P as fp16 or bf16 pairs
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      u32x4 v;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * hh + i], cmul, mneg));
        float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * hh + i + 1], cmul, mneg));
        if constexpr (MASK) {
          const int r0 = 8 * hh + i;
          const int key0 = kb * 32 + 8 * (r0 >> 2) + 4 * half + (r0 & 3);
          if (key0 >= nval) e0 = 0.0f;
          if (key0 + 1 >= nval) e1 = 0.0f;
        }
        if constexpr (PB) {
          const bf16x2 pr = __builtin_convertvector(f32x2{e0, e1}, bf16x2);
          lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, bf16x2{__bf16(1.0f), __bf16(1.0f)}, lsum, false);
          v[i / 2] = __builtin_bit_cast(uint32_t, pr);
        } else {
          const f16x2 pr = pkrtz(e0, e1);
          lsum = __builtin_amdgcn_fdot2(pr, f16x2{1.0f16, 1.0f16}, lsum, false);
          v[i / 2] = as_u32(pr);
        }
      }
      p[2 * kb + hh] = v;
    }
  sm.l += lsum;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      if constexpr (PB)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf[db][ks]),
                                                          __builtin_bit_cast(bf16x8, p[ks]), acc[db], 0, 0, 0);
      else
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, vf[db][ks]),
                                                         __builtin_bit_cast(f16x8, p[ks]), acc[db], 0, 0, 0);
    }
}

// Loads the wave's 32 query rows as MFMA B operands (bf16 bits).
template <int D>
__device__ __forceinline__ void load_q(const AttnArgs &a, int h, int q0, u32x4 (&qr)[D / 16]) {
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  const int qi = q0 + l32;
  const bool ok = qi < a.n_q;
  const uint16_t *qp = a.q + (int64_t(h) * a.n_q + (ok ? qi : 0)) * D + 8 * half;
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
    qr[st] = ok ? *reinterpret_cast<const u32x4 *>(qp + 16 * st) : u32x4{0, 0, 0, 0};
}

// Order of the cache tiles: the full 64-key tiles of every segment, then each
// segment's ragged tail (fewer than 64 keys), so that the main loop never masks.
// Cursors are (segment, first key) pairs of plain integers (uniform values).
__device__ __forceinline__ bool first_full(const AttnArgs &a, int from, int &seg, int &k0) {
  for (int sg = from; sg < a.n_seg; ++sg)
    if (a.seg[sg].ntok >= kBN) {
      seg = sg;
      k0 = 0;
      return true;
    }
  return false;
}

__device__ __forceinline__ bool next_full(const AttnArgs &a, int &seg, int &k0) {
  if (k0 + 2 * kBN <= a.seg[seg].ntok) {
    k0 += kBN;
    return true;
  }
  return first_full(a, seg + 1, seg, k0);
}

// i-th full cache tile of a query block -> (segment, first key)
__device__ __forceinline__ void nth_full(const AttnArgs &a, int i, int &seg, int &k0) {
  int sg = 0;
  for (; sg < a.n_seg; ++sg) {
    const int nf = a.seg[sg].ntok / kBN;
    if (i < nf) break;
    i -= nf;
  }
  seg = sg;
  k0 = i * kBN;
}

// i-th ragged cache tail of a query block -> segment
__device__ __forceinline__ int nth_tail(const AttnArgs &a, int i) {
  int sg = 0;
  for (; sg < a.n_seg; ++sg) {
    if (a.seg[sg].ntok % kBN == 0) continue;
    if (i == 0) break;
    --i;
  }
  return sg;
}

// Partial result of a range of a query block's tiles: the accumulator in absolute
// units of V, then per lane the running max and the partial row sum.  Each thread
// stores and later reads back only its own elements, 16 bytes at a time, so the
// layout is private to the kernel and every access is coalesced.
template <int D>
__device__ __forceinline__ void store_partial(float *ps, const f32x16 (&acc)[D / 32], float vunit,
                                              const Softmax &sm) {
  constexpr int kT = Cfg<D>::kThreads;
  const int tid = threadIdx.x;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4 *>(ps + ((db * 4 + g) * kT + tid) * 4) =
          make_float4(acc[db][4 * g] * vunit, acc[db][4 * g + 1] * vunit, acc[db][4 * g + 2] * vunit,
                      acc[db][4 * g + 3] * vunit);
  *reinterpret_cast<float2 *>(ps + Cfg<D>::kBM * D + 2 * tid) = make_float2(sm.m, sm.l);
}

// Device-scope (sc1) 64-bit read: coherent across XCDs without invalidating the
// reader's L2, which holds the K/V tiles every workgroup on that XCD is streaming.
__device__ __forceinline__ float2 get_pair(const float *p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(uint32_t(v)), __uint_as_float(uint32_t(v >> 32)));
}

template <int D>
__device__ __forceinline__ void write_out(const AttnArgs &a, int h, int qi, const f32x16 (&acc)[D / 32],
                                          float fin) {
  const int half = (threadIdx.x >> 5) & 1;
  if (qi >= a.n_q) return;
  float *op = a.out + (int64_t(h) * a.n_q + qi) * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = db * 32 + 8 * gq + 4 * half;
      *reinterpret_cast<float4 *>(op + d) = make_float4(acc[db][4 * gq] * fin, acc[db][4 * gq + 1] * fin,
                                                        acc[db][4 * gq + 2] * fin, acc[db][4 * gq + 3] * fin);
    }
}

}  // namespace

// MX: the cache holds MXFP4 (dequantized to bf16, QK^T and PV of its tiles on the
// bf16 matrix cores with plain bf16 Q); otherwise NVFP4.  MXS (with MX): QK^T of the
// cache tiles on the MX-scaled matrix cores from the raw codes, queries in MXFP8.
template <int D, bool MX, bool MXS>
__global__ __launch_bounds__(Cfg<D>::kThreads, Cfg<D>::kWgPerCu) void chunk_attention_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kKsElems<D>];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kVsElems<D>];
  __shared__ int s_ready;
  static_assert(kRawScales<D> + kBN * (D / 32) <= 2 * kKsElems<D>, "raw K tile fits the Ks buffer");
  static_assert(!MXS || MX, "the MX-scaled product reads MXFP4 codes");
  constexpr int kBM = Cfg<D>::kBM;
  constexpr size_t kSlotFloats = attn_slot_bytes(D) / 4;
  static_assert(kBM == attn_block_queries(D) && Cfg<D>::kThreads == attn_threads(D) &&
                Cfg<D>::kWgPerCu == attn_wg_per_cu(D), "scratch sizing");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;

  // XCD-aware numbering: hardware places workgroup `bid` on XCD bid % 8; give each
  // XCD a contiguous run of work ranges, i.e. mostly one head's keys.
  const int G = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7;
  const int g = xcd * (G >> 3) + min(xcd, G & 7) + (bid >> 3);
  // this workgroup's share [ubeg, u) of the weighted list of all (query block, key
  // tile) pairs; it processes the tiles that start inside its share (every share is
  // at least one tile long, so every workgroup has tiles), one query block at a time
  // from the share's END (next_range): every workgroup starts at key tile 0 and all
  // workgroups of a head stay within a few tiles of each other (their K/V stays in
  // L2).
  const int64_t U = a.work;
  const int T = a.tiles, WB = a.w_block;
  const int cache_tiles = a.n_cfull + a.n_ctail;
  const int qblocks = (a.n_q + kBM - 1) / kBM;
  const int64_t ubeg = U * g / G;
  int64_t u = U * (g + 1) / G;

  int b, t0, t1;
  while (next_range(a, ubeg, u, b, t0, t1)) {
    const int64_t b64 = b;
    const int h = b / qblocks;
    const int q0 = (b - h * qblocks) * kBM + w * kQW;
    const int qi = q0 + l32;

    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
    Softmax sm;
    sm.m = -INFINITY;
    sm.l = 0.0f;
    float vunit = 1.0f;
    f32x16 s[2];
    u32x4 qr[D / 16];

    // Tiles [r0, r1) of block b.  Normally r0 = t0, r1 = t1, once.  The workgroup
    // that holds a cut block's last tiles waits (bounded) for the partials of the
    // workgroups holding its earlier tiles; if one is still missing it processes the
    // block's earlier tiles [0, r0) itself (a second pass of this loop) instead of
    // merging.
    int r0 = t0, r1 = t1;
    while (true) {
      // ---- cache tiles (NVFP4)
      if (r0 < cache_tiles) {
        // NVFP4: Q as fp16 with a per-query power-of-two scale 2^sh (row max -> [2^14,
        // 2^15)); MXFP4: plain bf16 Q
        QFp8<D> qf;
        if constexpr (MXS) quantize_q_mxfp8<D>(a, h, q0, qf);
        else load_q<D>(a, h, q0, qr);
        float cq = 1.0f;
        if constexpr (!MX) {
          uint32_t mx = 0;
#pragma unroll
          for (int st = 0; st < D / 16; ++st)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t v = qr[st][j] & 0x7FFF7FFFu;
              mx = max(mx, max(v & 0xFFFFu, v >> 16));
            }
          mx = other_half_umax(mx);
          const int e = int(mx >> 7) - 127;   // floor(log2(row max)) (bf16 normals)
          int sh = mx ? 14 - e : 0;
          sh = max(-110, min(100, sh));
          cq = __builtin_ldexpf(1.0f, -sh);
#pragma unroll
          for (int st = 0; st < D / 16; ++st)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t v = qr[st][j];
              qr[st][j] = as_u32(pkrtz(__builtin_ldexpf(__uint_as_float(v << 16), sh),
                                       __builtin_ldexpf(__uint_as_float(v & 0xFFFF0000u), sh)));
            }
        }
        const HeadPlanes hp = head_planes<D, MX>(a, h);
        int cur_seg = -1;
        float cmul = 0.0f;
        // per segment: s_K folds into the logit multiplier; the accumulator moves to
        // units of the segment's s_V (an all-zero V chunk has s_V = 0 and contributes
        // nothing: keep the current units)
        float kbias = 0.0f;
        auto enter_segment = [&](int sg) {
          if (sg == cur_seg) return;
          cur_seg = sg;
          const int slot = a.seg[sg].scale_slot;
          const float sk = a.scale_table[2 * slot];
          const float sv = a.scale_table[2 * slot + 1];
          cmul = a.sm_scale_log2 * sk * cq;
          if (a.k_mean) {
            // K-smoothing: the chunk's K was quantized minus its channel means mu, so
            // every logit of its keys gains q . mu (the same for all of them)
            const float *mu = a.k_mean + (int64_t(slot) * a.H + h) * D + 8 * half;
            float dot = 0.0f;
#pragma unroll
            for (int st = 0; st < D / 16; ++st) {
              const f16x8 qv = __builtin_bit_cast(f16x8, qr[st]);
              const float4 m0 = *reinterpret_cast<const float4 *>(mu + 16 * st);
              const float4 m1 = *reinterpret_cast<const float4 *>(mu + 16 * st + 4);
              dot += float(qv[0]) * m0.x + float(qv[1]) * m0.y + float(qv[2]) * m0.z + float(qv[3]) * m0.w +
                     float(qv[4]) * m1.x + float(qv[5]) * m1.y + float(qv[6]) * m1.z + float(qv[7]) * m1.w;
            }
            dot = other_half_sum(dot);
            kbias = dot * cq * a.sm_scale_log2;
          }
          if (sv > 0.0f) {
            const float r = vunit / sv;
  #pragma unroll
            for (int db = 0; db < D / 32; ++db) acc[db] *= r;
            vunit = sv;
          }
        };

        // full tiles [r0, f1), software-pipelined: tile i in LDS buffer (i - r0) % 2,
        // the packed bytes of tile i+1 in registers.  Past the range's last tile the
        // pipeline re-stages the last one into the free buffer (never read).
        const int f1 = min(r1, a.n_cfull);
        if (r0 < f1) {
          int cs, ck;
          nth_full(a, r0, cs, ck);
          Packed<D> pk;
          load_packed<D, MX>(hp, uint32_t(a.seg[cs].tok0 + ck), kBN, pk);
          dequant_store<D, MX, MXS>(pk, Ks[0], Vs[0]);
          int ns = cs, nk = ck;
          bool have_next = r0 + 1 < f1 && next_full(a, ns, nk);
          int ltok = have_next ? a.seg[ns].tok0 + nk : a.seg[cs].tok0 + ck;
          load_packed<D, MX>(hp, uint32_t(ltok), kBN, pk);
          __syncthreads();
          int buf = 0;
          for (int i = r0;; ++i) {
            enter_segment(cs);
            if constexpr (MXS) qk_tile_mxs<D>(Ks[buf], qf, s);
            else qk_tile<D, MX>(Ks[buf], qr, s);
            // stage tile i+1 while the MFMAs run, then fetch the bytes of tile i+2
            dequant_store<D, MX, MXS>(pk, Ks[buf ^ 1], Vs[buf ^ 1]);
            int s2 = ns, k2 = nk;
            const bool have_n2 = have_next && i + 2 < f1 && next_full(a, s2, k2);
            if (have_n2) ltok = a.seg[s2].tok0 + k2;
            load_packed<D, MX>(hp, uint32_t(ltok), kBN, pk);
            softmax_pv<D, false, MX>(Vs[buf], s, cmul, kbias, kBN, sm, acc);
            __syncthreads();
            if (!have_next) break;
            buf ^= 1;
            cs = ns;
            ck = nk;
            ns = s2;
            nk = k2;
            have_next = have_n2;
          }
        }
        // ragged tails, one at a time
        const int c1 = min(r1, cache_tiles) - a.n_cfull;
        for (int i = max(r0, a.n_cfull) - a.n_cfull; i < c1; ++i) {
          const int cs = nth_tail(a, i);
          const int tn = a.seg[cs].ntok % kBN;
          const int ck = a.seg[cs].ntok - tn;
          Packed<D> pk;
          load_packed<D, MX>(hp, uint32_t(a.seg[cs].tok0 + ck), tn, pk);
          dequant_store<D, MX, MXS>(pk, Ks[0], Vs[0]);
          enter_segment(cs);
          __syncthreads();
          if constexpr (MXS) qk_tile_mxs<D>(Ks[0], qf, s);
          else qk_tile<D, MX>(Ks[0], qr, s);
          softmax_pv<D, true, MX>(Vs[0], s, cmul, kbias, tn, sm, acc);
          __syncthreads();
        }
      }

      // ---- own segment (bf16 K/V of the chunk itself): full tiles pipelined like the
      // cache, then the ragged tail
      if (r1 > cache_tiles) {
        load_q<D>(a, h, q0, qr);   // plain bf16 Q
        const float cmul = a.sm_scale_log2;
  #pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] *= vunit;   // to s_V = 1 units
        vunit = 1.0f;
        const int o0 = max(r0 - cache_tiles, 0), o1 = r1 - cache_tiles;
        const int e = min(o1, a.n_ofull);
        if (o0 < e) {
          uint4 rk[2];
          uint32_t rv[8];
          load_own_k<D>(a, h, o0 * kBN, kBN, rk);
          load_own_v<D>(a, h, o0 * kBN, kBN, rv);
          store_own_k<D>(rk, Ks[0]);
          store_own_v<D>(rv, Vs[0]);
          load_own_v<D>(a, h, min(o0 + 1, e - 1) * kBN, kBN, rv);
          __syncthreads();
          int buf = 0;
          for (int t = o0; t < e; ++t) {
            // K of tile t+1 is fetched at the top of the iteration (its latency runs
            // under the QK^T MFMAs); V of tile t+1 was fetched one iteration ahead
            load_own_k<D>(a, h, min(t + 1, e - 1) * kBN, kBN, rk);
            qk_tile<D, true>(Ks[buf], qr, s);
            store_own_v<D>(rv, Vs[buf ^ 1]);
            store_own_k<D>(rk, Ks[buf ^ 1]);
            load_own_v<D>(a, h, min(t + 2, e - 1) * kBN, kBN, rv);
            softmax_pv<D, false, true>(Vs[buf], s, cmul, 0.0f, kBN, sm, acc);
            __syncthreads();
            buf ^= 1;
          }
        }
        if (o1 > a.n_ofull) {
          const int nval = a.n_q - a.n_ofull * kBN;
          uint4 rk[2];
          uint32_t rv[8];
          load_own_k<D>(a, h, a.n_ofull * kBN, nval, rk);
          load_own_v<D>(a, h, a.n_ofull * kBN, nval, rv);
          store_own_k<D>(rk, Ks[0]);
          store_own_v<D>(rv, Vs[0]);
          __syncthreads();
          qk_tile<D, true>(Ks[0], qr, s);
          softmax_pv<D, true, true>(Vs[0], s, cmul, 0.0f, nval, sm, acc);
        }
      }

      if (r0 == 0 || t1 < T) break;
      // the block's last tiles, its first ones done by workgroups gf..g-1 (each as
      // the first range it processed): wait, bounded, for their partials
      if (tid == 0) {
        const int gf = owner_of(b64 * WB, U, G);
        bool ready = true;
        for (int gg = gf; gg < g && ready; ++gg) {
          int spin = 0;
          while (__hip_atomic_load(a.flags + gg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != a.epoch) {
            if (spin++ >= a.spin_limit) {
              ready = false;
              break;
            }
            __builtin_amdgcn_s_sleep(8);
          }
        }
        s_ready = ready;
      }
      __syncthreads();
      if (s_ready) break;
      r1 = r0;   // one is still missing: process the block's first tiles here
      r0 = 0;
    }

    if (t1 < T) {
      // ---- not the block's last tiles: publish this range's partial result for the
      // workgroup that holds the block's end (the partial lives in this workgroup's
      // slot; its flag carries the launch's epoch once the slot is complete)
      store_partial<D>(a.partials + size_t(g) * kSlotFloats, acc, vunit, sm);
      __builtin_amdgcn_s_waitcnt(0);   // every wave's stores are in this XCD's L2
      __syncthreads();
      if (tid == 0) {
        // one release for the workgroup: writes the L2's dirty lines back to memory,
        // where the merging workgroup (possibly on another XCD) reads them
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_store(a.flags + g, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else if (r0 > 0) {
      // ---- the block's last tiles: merge the partials of workgroups gf..g-1 with the
      // registers, in workgroup order
      const int gf = owner_of(b64 * WB, U, G);   // holds the block's first tile
      float mx = sm.m;
      for (int gg = gf; gg < g; ++gg)
        mx = fmaxf(mx, get_pair(a.partials + size_t(gg) * kSlotFloats + kBM * D + 2 * tid).x);
      const float f0 = __builtin_amdgcn_exp2f(sm.m - mx);
      float lsum = sm.l * f0;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] *= vunit * f0;
      for (int gg = gf; gg < g; ++gg) {
        // issue every load of the partial before using any (one round trip, not 2 per 16 B)
        const float *ps = a.partials + size_t(gg) * kSlotFloats;
        float2 o[D / 32][4][2];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const float *p = ps + ((db * 4 + gq) * Cfg<D>::kThreads + tid) * 4;
            o[db][gq][0] = get_pair(p);
            o[db][gq][1] = get_pair(p + 2);
          }
        const float2 ml = get_pair(ps + kBM * D + 2 * tid);
        const float f = __builtin_amdgcn_exp2f(ml.x - mx);
        lsum += ml.y * f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            acc[db][4 * gq] += o[db][gq][0].x * f;
            acc[db][4 * gq + 1] += o[db][gq][0].y * f;
            acc[db][4 * gq + 2] += o[db][gq][1].x * f;
            acc[db][4 * gq + 3] += o[db][gq][1].y * f;
          }
      }
      write_out<D>(a, h, qi, acc, 1.0f / other_half_sum(lsum));
    } else {
      // ---- the whole block here (or all of it after giving up waiting)
      write_out<D>(a, h, qi, acc, vunit / other_half_sum(sm.l));
    }
    __syncthreads();   // LDS buffers and s_ready are reused by the next range
  }
}

namespace {
int g_attn_cus[64];

int attn_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kAttnMaxCus;
  if (g_attn_cus[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return kAttnMaxCus;
    g_attn_cus[dev] = cus;
  }
  return g_attn_cus[dev];
}

template <int D>
int launch_attention_d(AttnArgs a, hipStream_t s) {
  if (!a.partials || !a.flags) return NVFP4KV_EINVAL;
  // one workgroup per resident slot (every CU busy), each with an equal share of the
  // weighted work
  const int64_t grid = attn_plan(a, Cfg<D>::kBM, int64_t(min(attn_cu_count(), kAttnMaxCus)) * Cfg<D>::kWgPerCu);
  if (grid < 0) return int(grid);
  if (a.mx == 2)
    hipLaunchKernelGGL((chunk_attention_kernel<D, true, true>), dim3(unsigned(grid)), dim3(Cfg<D>::kThreads), 0, s, a);
  else if (a.mx == 1)
    hipLaunchKernelGGL((chunk_attention_kernel<D, true, false>), dim3(unsigned(grid)), dim3(Cfg<D>::kThreads), 0, s,
                       a);
  else
    hipLaunchKernelGGL((chunk_attention_kernel<D, false, false>), dim3(unsigned(grid)), dim3(Cfg<D>::kThreads), 0,
                       s, a);
  return NVFP4KV_HIP_OK(hipGetLastError());
}
}  // namespace

int launch_attention(const AttnArgs &a, void *stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (a.D == 128) return launch_attention_d<128>(a, s);
  if (a.D == 64) return launch_attention_d<64>(a, s);
  return NVFP4KV_EINVAL;
}

}  // namespace nvfp4kv
