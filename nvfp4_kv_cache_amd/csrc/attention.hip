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
//  * A workgroup owns 128 queries of one head (4 waves x 32).  Keys stream in tiles
//    of 64.  Each tile's K and V are dequantized ONCE per workgroup into LDS (K as
//    bf16, V as fp16) and shared by the 4 waves, so the dequantization VALU work is
//    not repeated per wave.  E2M1 x E4M3 has at most 6 significant bits and lies in
//    [2^-10, 2688], so both conversions are exact; the fp32 tensor scales stay
//    outside the matrix cores (s_K folds into the logit scale, s_V into the units of
//    the output accumulator).
//  * S^T = K Q^T runs on v_mfma_f32_32x32x16_bf16 with K from LDS as the A operand
//    and Q held in registers as the B operand.  The accumulator layout then gives
//    each lane one query and 16 keys, which is exactly the lane layout of the B
//    operand of the PV product O^T = V^T P^T; P never leaves registers.  V is
//    stored in LDS as V^T with the keys of each 16-key group permuted to match.
//  * PV runs on v_mfma_f32_32x32x16_f16: V^ is exact in fp16 and P in [0,1] keeps 11
//    significant bits (bf16 would keep 8).  The own segment's bf16 V is converted to
//    fp16 on staging (|v| < 65504 is required).
//  * Online softmax in fp32 with exp2 (log2(e) folded into the logit scale).  Row
//    sums are taken from the fp16-rounded probabilities that enter the PV product.
//  * Workgroups are numbered so that each XCD (own L2) runs a contiguous range of
//    (head, query-tile) pairs, i.e. mostly one head's keys.

#include "device_common.h"

namespace nvfp4kv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int kBN = 64;        // keys per tile
constexpr int kWaves = 4;
constexpr int kQW = 32;        // queries per wave
constexpr int kBM = kWaves * kQW;

// 16-key group permutation of V^T in LDS: physical position p holds key kk(p),
// kk swaps bits 2 and 3 of p (an involution).
__device__ __forceinline__ int vperm(int p) {
  return (p & 3) | ((p & 4) << 1) | ((p & 8) >> 1);
}

// E2M1 magnitude code -> fp32 value.
__device__ __forceinline__ float e2m1_value(uint32_t m) {
  // 0, 0.5, 1, 1.5, 2, 3, 4, 6
  const float lo = (m & 1u) ? 1.5f : 1.0f;
  const uint32_t e = m >> 1;
  return e == 0 ? ((m & 1u) ? 0.5f : 0.0f) : lo * __uint_as_float((126u + e) << 23);
}

__device__ __forceinline__ float nvfp4_value(uint32_t code, float scale) {
  const float v = e2m1_value(code & 7u) * scale;
  return (code & 8u) ? -v : v;
}

// Ks: [kBN][D] bf16, 16-byte chunks of each row XOR-swizzled by the row index.
template <int D>
__device__ __forceinline__ int ks_off(int row, int chunk) {
  return row * D + ((chunk ^ (row & (D / 8 - 1))) << 3);
}
// Vs: [D][kBN] fp16 (V^T), 16-byte chunks swizzled by the row (d) index.
__device__ __forceinline__ int vs_off(int row, int chunk) {
  return row * kBN + ((chunk ^ (row & 7)) << 3);
}

template <int D>
__device__ __forceinline__ void stage_cache_tile(const AttnArgs &a, int h, int tok, int nval,
                                                 uint16_t *Ks, uint16_t *Vs) {
  constexpr int nb = D / 16;
  const int tid = threadIdx.x;
  // ---- K: (key, block) tasks, 16 codes + 1 scale each -> 16 bf16
  for (int task = tid; task < kBN * nb; task += kWaves * 64) {
    const int key = task / nb, b = task % nb;
    uint32_t c0 = 0, c1 = 0, sc = 0;
    if (key < nval) {
      const int64_t row = int64_t(h) * a.rows + tok + key;
      const uint32_t *cp = reinterpret_cast<const uint32_t *>(a.kcodes + row * (D / 2) + b * 8);
      c0 = cp[0];
      c1 = cp[1];
      sc = a.kscales[row * nb + b];
    }
    const float s = e4m3_value(sc);
    uint32_t o[8];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const uint32_t w = e < 8 ? c0 : c1;
      const uint32_t n0 = (w >> (4 * (e & 7))) & 0xFu, n1 = (w >> (4 * ((e + 1) & 7))) & 0xFu;
      // exact in bf16: truncating the fp32 bits loses nothing
      const uint32_t b0 = __float_as_uint(nvfp4_value(n0, s)) >> 16;
      const uint32_t b1 = __float_as_uint(nvfp4_value(n1, s)) >> 16;
      o[e >> 1] = b0 | (b1 << 16);
    }
    *reinterpret_cast<uint4 *>(Ks + ks_off<D>(key, 2 * b)) = make_uint4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<uint4 *>(Ks + ks_off<D>(key, 2 * b + 1)) = make_uint4(o[4], o[5], o[6], o[7]);
  }
  // ---- V^T: (d, 16-key group) tasks, 16 codes + 16 scales each -> 16 fp16
  for (int task = tid; task < D * (kBN / 16); task += kWaves * 64) {
    const int d = task >> 2, g = task & 3;
    uint32_t cw[2] = {0u, 0u}, sw[4] = {0u, 0u, 0u, 0u};
    const int64_t crow = (int64_t(h) * D + d) * (a.rows / 2) + (tok >> 1) + g * 8;
    const int64_t srow = (int64_t(h) * nb + (d >> 4)) * a.rows + tok + g * 16;
    const uint32_t *cp = reinterpret_cast<const uint32_t *>(a.vcodes + crow);
    const uint32_t *sp = reinterpret_cast<const uint32_t *>(a.vscales + srow);
    if (g * 16 < nval) {      // nval is a multiple of 8
      cw[0] = cp[0];
      sw[0] = sp[0];
      sw[1] = sp[1];
    }
    if (g * 16 + 8 < nval) {
      cw[1] = cp[1];
      sw[2] = sp[2];
      sw[3] = sp[3];
    }
    _Float16 v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t code = (cw[k >> 3] >> (4 * (k & 7))) & 0xFu;
      const uint32_t sb = (sw[k >> 2] >> (8 * (k & 3))) & 0xFFu;
      v[k] = _Float16(nvfp4_value(code, e4m3_value(sb)));   // exact
    }
    f16x8 lo, hi;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      lo[p] = v[vperm(p)];
      hi[p] = v[vperm(p + 8)];
    }
    *reinterpret_cast<f16x8 *>(Vs + vs_off(d, 2 * g)) = lo;
    *reinterpret_cast<f16x8 *>(Vs + vs_off(d, 2 * g + 1)) = hi;
  }
}

template <int D>
__device__ __forceinline__ void stage_own_tile(const AttnArgs &a, int h, int tok, int nval,
                                               uint16_t *Ks, uint16_t *Vs) {
  constexpr int nb = D / 16;
  const int tid = threadIdx.x;
  for (int task = tid; task < kBN * nb; task += kWaves * 64) {
    const int key = task / nb, b = task % nb;
    uint4 k0 = make_uint4(0, 0, 0, 0), k1 = k0, v0 = k0, v1 = k0;
    if (key < nval) {
      const int64_t off = (int64_t(h) * a.n_q + tok + key) * D + b * 16;
      const uint4 *kp = reinterpret_cast<const uint4 *>(a.k_own + off);
      const uint4 *vp = reinterpret_cast<const uint4 *>(a.v_own + off);
      k0 = kp[0];
      k1 = kp[1];
      v0 = vp[0];
      v1 = vp[1];
    }
    *reinterpret_cast<uint4 *>(Ks + ks_off<D>(key, 2 * b)) = k0;
    *reinterpret_cast<uint4 *>(Ks + ks_off<D>(key, 2 * b + 1)) = k1;
    // V: bf16 -> fp16, scattered into V^T
    const uint32_t vw[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    const int g = key >> 4, kk = key & 15;
    const int p = vperm(kk);
    const int chunk = 2 * g + (p >> 3);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t hb = (e & 1) ? (vw[e >> 1] >> 16) : (vw[e >> 1] & 0xFFFFu);
      const _Float16 hv = _Float16(bf16_bits_to_float(hb));
      const int d = b * 16 + e;
      Vs[vs_off(d, chunk) + (p & 7)] = __builtin_bit_cast(uint16_t, hv);
    }
  }
}

}  // namespace

template <int D>
__global__ __launch_bounds__(kWaves * 64, 2) void chunk_attention_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBN * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[D * kBN];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;

  // XCD-aware numbering: hardware places workgroup `bid` on XCD bid % 8; give each
  // XCD a contiguous range of logical (head, query-tile) ids.
  const int n = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7;
  const int logical = xcd * (n >> 3) + min(xcd, n & 7) + (bid >> 3);
  const int qtiles = (a.n_q + kBM - 1) / kBM;
  const int h = logical / qtiles;
  const int qt = logical - h * qtiles;
  const int qi = qt * kBM + w * kQW + l32;   // this lane's query
  const bool qok = qi < a.n_q;

  bf16x8 qreg[D / 16];
  {
    const uint16_t *qp = a.q + (int64_t(h) * a.n_q + (qok ? qi : 0)) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      if (qok) qreg[s] = *reinterpret_cast<const bf16x8 *>(qp + 16 * s);
      else
        for (int e = 0; e < 8; ++e) qreg[s][e] = __bf16(0.0f);
    }
  }
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
  float m = -INFINITY, lsum = 0.0f, vunit = 1.0f;

  for (int si = 0; si <= a.n_seg; ++si) {
    const bool own = si == a.n_seg;
    int tok0, ntok;
    float sk = 1.0f, sv = 1.0f;
    if (own) {
      tok0 = 0;
      ntok = a.n_q;
    } else {
      tok0 = a.seg[si].tok0;
      ntok = a.seg[si].ntok;
      sk = a.scale_table[2 * a.seg[si].scale_slot];
      sv = a.scale_table[2 * a.seg[si].scale_slot + 1];
    }
    const float C = a.sm_scale_log2 * sk;
    // keep the accumulator in units of this segment's s_V (an all-zero V chunk has
    // s_V = 0 and contributes nothing, so it keeps the current units)
    if (sv > 0.0f) {
      const float r = vunit / sv;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) acc[i] *= r;
      vunit = sv;
    }
    for (int k0 = 0; k0 < ntok; k0 += kBN) {
      const int nval = min(kBN, ntok - k0);
      __syncthreads();
      if (own) stage_own_tile<D>(a, h, k0, nval, Ks, Vs);
      else stage_cache_tile<D>(a, h, tok0 + k0, nval, Ks, Vs);
      __syncthreads();

      // S^T = K Q^T for the wave's 32 queries: two 32-key blocks
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
        const int row = kb * 32 + l32;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(Ks + ks_off<D>(row, 2 * s + half));
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[s], sacc[kb], 0, 0, 0);
        }
      }
      // online softmax (lane = one query, 32 of the tile's keys; partner lane^32 has the rest)
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key < nval) mx = fmaxf(mx, sacc[kb][r]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(m, mx * C);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;
      f16x8 pf[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          const float p = key < nval ? __builtin_amdgcn_exp2f(sacc[kb][r] * C - m) : 0.0f;
          const _Float16 ph = _Float16(p);
          lsum += float(ph);
          pf[2 * kb + (r >> 3)][r & 7] = ph;
        }
      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int row = db * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const f16x8 vf = *reinterpret_cast<const f16x8 *>(Vs + vs_off(row, 2 * ks + half));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[ks], acc[db], 0, 0, 0);
        }
      }
    }
  }
  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  const float fin = vunit / ltot;
  if (qok) {
    float *op = a.out + (int64_t(h) * a.n_q + qi) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * half;
        *reinterpret_cast<float4 *>(op + d) =
            make_float4(acc[db][4 * g] * fin, acc[db][4 * g + 1] * fin,
                        acc[db][4 * g + 2] * fin, acc[db][4 * g + 3] * fin);
      }
  }
}

int launch_attention(const AttnArgs &a, void *stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int qtiles = (a.n_q + kBM - 1) / kBM;
  const int64_t nblk = int64_t(qtiles) * a.H;
  if (nblk >= (int64_t(1) << 31)) return NVFP4KV_EINVAL;
  if (a.D == 128)
    hipLaunchKernelGGL(chunk_attention_kernel<128>, dim3(unsigned(nblk)), dim3(kWaves * 64), 0, s, a);
  else if (a.D == 64)
    hipLaunchKernelGGL(chunk_attention_kernel<64>, dim3(unsigned(nblk)), dim3(kWaves * 64), 0, s, a);
  else
    return NVFP4KV_EINVAL;
  return NVFP4KV_HIP_OK(hipGetLastError());
}

}  // namespace nvfp4kv
