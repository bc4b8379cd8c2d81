"""NVFP4 codec oracle (plain numpy; test infrastructure only).

What the pages fix
------------------
* Paper text, section 2.2 "NVFP4 Training": quantization works on 16-element
  blocks; the block scale is FP8 E4M3 whose largest magnitude is 448; the
  elements are FP4 E2M1 whose largest magnitude is 6.  (The quantizer equation
  itself did not survive extraction; only its legend did.)
* Reading note, section II "The NVFP4 quantization format": E2M1 is 1 sign,
  2 exponent and 1 mantissa bit; storage is three-level -- one FP32 tensor-wide
  scale, one E4M3 scale per 16 elements, and the FP4 element -- and the
  dequantized value is the product of the three (the formula after "The
  dequantization formula is therefore:" is missing; the product is the plain
  reading of the three-level description).
* Reading note, "The inference infrastructure": K and V are quantized per
  frame chunk; the packed form costs 9/16 byte per element (4 bits of code plus
  one byte of scale per 16 elements), i.e. 9/8 T_c H d bytes for K and V.

Readings taken where the pages are silent
---------------------------------------------------------------------------
* Tensor scale  s_t = amax_t / (6 * 448) = amax_t / 2688, one fp32 division,
  where amax_t is the largest |x| of one chunk tensor (all heads).
* Block scale   bs  = (amax_b / 6) / s_t, two fp32 divisions in that order,
  then rounded to E4M3 (OCP E4M3FN -- the flavour whose max is 448) with
  round-to-nearest-even and saturation at 448.  0x7F (NaN) is never produced.
* Element       q   = |x| / eff  with  eff = E4M3(bs) * s_t  (one fp32
  multiply, one fp32 division), rounded to E2M1 with round-to-nearest-even,
  saturating at 6.  code = sign << 3 | magnitude; the sign of -0.0 is kept.
* When eff == 0 (all-zero block, zero tensor, or a product that underflows)
  every code in the block is sign << 3.
* Blocks run along the last (head_dim) axis; codes are packed two per byte,
  the even element in the low nibble; scales are stored as raw E4M3 bytes.

All fp32 steps use numpy float32 arithmetic, which is IEEE-754 correctly
rounded with subnormals kept, so the steps above define every bit.

Optional steps for the KV cache (reading note, "The inference infrastructure":
within each frame chunk, K-smoothing is applied to K and adaptive scale selection
to V; the paper text, section 2.2 and related work, cites Four Over Six as the
adaptive block-scale selection with candidate scale magnitudes {4, 6}).  The
pages give no formulas; the readings are:
* K-smoothing: subtract from every K element its channel mean over the chunk's
  tokens, mu[h, d], before quantizing; mu is kept in fp32 and added back on
  dequantization.  mu is fixed bit for bit: the channel's values (fp32), padded
  with +0.0 to a power-of-two count, are summed pairwise level by level
  (v'[i] = v[2i] + v[2i+1], each an fp32 add), and the root is divided by the
  token count (one fp32 division).  The smoothed element is x - mu (one fp32
  subtraction) and the recipe above runs on those fp32 values (their amax gives
  s_t, their sign bit the code's sign).
* Adaptive block scale (V): each block is encoded twice, with the block maximum
  mapped to 6 (the plain recipe) and to 4 (bs = (amax_b / 4) / s_t, the same
  rounding), keeping s_t; the candidate with the smaller squared error wins, ties
  going to 6.  The error of a candidate is the sum over the block's 16 elements,
  in order, of (|x| - value * eff)^2, every operation an fp32 operation.
"""

import numpy as np

# --------------------------------------------------------------------------
# Code tables, built from the bit-field definitions.
# --------------------------------------------------------------------------


def _e2m1_magnitudes():
    """Values of the 8 non-negative E2M1 codes (1 sign, 2 exponent bits with
    bias 1, 1 mantissa bit; exponent field 0 is subnormal)."""
    vals = []
    for code in range(8):
        e, m = code >> 1, code & 1
        if e == 0:
            vals.append(m * 0.5)
        else:
            vals.append((1.0 + m / 2.0) * 2.0 ** (e - 1))
    return np.array(vals, dtype=np.float64)


def _e4m3_magnitudes():
    """Values of the 127 non-negative, non-NaN E4M3FN codes 0x00..0x7E
    (4 exponent bits with bias 7, 3 mantissa bits, exponent 0 subnormal;
    0x7F is NaN and has no value)."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        if e == 0:
            vals.append(m * 2.0 ** -9)
        else:
            vals.append((1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


E2M1_VALUES = _e2m1_magnitudes()   # index = 3-bit magnitude code
E4M3_VALUES = _e4m3_magnitudes()   # index = scale byte 0x00..0x7E


def nearest_code_rne(v, table):
    """Index of the entry of the increasing ``table`` nearest to each v >= 0.

    Ties go to the even index (for these codes the even index is the one whose
    mantissa LSB is 0, i.e. round-half-to-even); values above the last entry
    saturate to it.  The midpoint test compares 2v with lo + hi, both exact in
    float64 for fp32 inputs and these tables, so no rounding enters the choice.
    """
    v = np.asarray(v, dtype=np.float64)
    assert not np.any(np.isnan(v)), "NaN has no NVFP4 code"
    assert np.all(v >= 0.0)
    n = len(table)
    idx = np.searchsorted(table, v, side="left")      # table[idx-1] < v <= table[idx]
    idx = np.clip(idx, 1, n - 1)
    lo = table[idx - 1]
    hi = table[idx]
    twice = 2.0 * v
    mid = lo + hi
    pick_hi = (twice > mid) | ((twice == mid) & (idx % 2 == 0))
    out = np.where(pick_hi, idx, idx - 1)
    out = np.where(v >= table[-1], n - 1, out)
    return out.astype(np.int64)


def e2m1_encode(q):
    """3-bit E2M1 magnitude code of q >= 0: nearest grid value, ties to the
    even code, saturating at 6 (code 7)."""
    return nearest_code_rne(q, E2M1_VALUES).astype(np.uint8)


def e4m3_encode(v):
    """E4M3FN byte of v >= 0: nearest representable value, ties to the even
    code, saturating at 448 (0x7E)."""
    return nearest_code_rne(v, E4M3_VALUES).astype(np.uint8)


# --------------------------------------------------------------------------
# bf16 input handling (inputs are bf16 bit patterns, uint16).
# --------------------------------------------------------------------------


def bf16_bits_to_f32(bits):
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# Quantizer / dequantizer
# --------------------------------------------------------------------------

F32 = np.float32
BLOCK = 16


def channel_mean_ref(x_bits):
    """K-smoothing channel means mu[h, d] of one chunk tensor x_bits [H, T, D]
    (bf16 bits): pairwise fp32 sums over the +0.0-padded power-of-two token
    count, then one fp32 division by T (module docstring)."""
    x = bf16_bits_to_f32(np.asarray(x_bits, dtype=np.uint16))
    H, T, D = x.shape
    assert T >= 1
    P = 1
    while P < T:
        P *= 2
    v = np.zeros((H, P, D), dtype=F32)
    v[:, :T] = x
    while v.shape[1] > 1:
        v = (v[:, 0::2] + v[:, 1::2]).astype(F32)
    return (v[:, 0] / F32(T)).astype(F32)


def _encode_blocks(ax, amax_b, s_t, M):
    """One candidate: block maxima mapped to M (6 or 4).  Returns the scale bytes
    [..., nb], the magnitude codes [..., nb, 16] and the per-block squared error
    (fp32, summed over the 16 elements in order)."""
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        if s_t > 0:
            bs = ((amax_b / F32(M)) / s_t).astype(F32)   # two fp32 divisions
        else:
            bs = np.zeros_like(amax_b)
    scale_codes = e4m3_encode(bs)
    eff = (E4M3_VALUES[scale_codes].astype(F32) * s_t).astype(F32)   # fp32 multiply
    live = eff > 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = (ax / np.where(live, eff, F32(1.0))[..., None]).astype(F32)
    mag = e2m1_encode(q)
    mag = np.where(live[..., None], mag, 0).astype(np.uint8)
    with np.errstate(over="ignore", invalid="ignore"):   # huge blocks: the error is +inf
        val = (E2M1_VALUES[mag].astype(F32) * eff[..., None]).astype(F32)
        d = (ax - val).astype(F32)
        e = (d * d).astype(F32)
        err = np.zeros(amax_b.shape, dtype=F32)
        for i in range(BLOCK):
            err = (err + e[..., i]).astype(F32)
    return scale_codes, mag, err


def quantize_ref(x_bits, mean=None, adaptive=False):
    """Quantize one chunk tensor to NVFP4.

    x_bits: uint16 bf16 bit patterns, shape [..., D] with D % 16 == 0 (the
    whole array is one tensor: one fp32 tensor scale for all of it).
    mean:   optional K-smoothing channel means, fp32 [H, D] for x [H, T, D]; the
            tensor quantized is then x - mean (fp32).
    adaptive: choose each block's scale between the 6- and 4-candidates.

    Returns (codes uint8 [..., D/2], scales uint8 [..., D/16], s_t float32).
    Steps follow the module docstring, in order.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    D = x_bits.shape[-1]
    assert D % BLOCK == 0
    x = bf16_bits_to_f32(x_bits)
    assert np.all(np.isfinite(x)), "inputs must be finite"
    if mean is not None:
        x = (x - np.asarray(mean, dtype=F32)[:, None, :]).astype(F32)   # fp32 subtraction
        sign_bits = np.signbit(x).astype(np.uint8)
    else:
        sign_bits = ((x_bits >> 15) & 1).astype(np.uint8)
    ax = np.abs(x)                                   # float32, exact

    # tensor scale
    amax_t = F32(ax.max()) if ax.size else F32(0.0)
    s_t = F32(amax_t / F32(6.0 * 448.0))             # one fp32 division

    lead = x.shape[:-1]
    nb = D // BLOCK
    blocks = ax.reshape(lead + (nb, BLOCK))
    amax_b = blocks.max(axis=-1)                     # float32

    scale_codes, mag, err6 = _encode_blocks(blocks, amax_b, s_t, 6)
    if adaptive:
        sc4, mag4, err4 = _encode_blocks(blocks, amax_b, s_t, 4)
        four = err4 < err6                           # ties keep 6
        scale_codes = np.where(four, sc4, scale_codes)
        mag = np.where(four[..., None], mag4, mag)

    sign = sign_bits.reshape(lead + (nb, BLOCK))
    code = (sign << 3) | mag                         # 4-bit codes
    code = code.reshape(lead + (D,))
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, scale_codes.astype(np.uint8), s_t


def unpack_codes(packed):
    """uint8 [..., D/2] -> 4-bit codes uint8 [..., D] (low nibble first)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out


def dequantize_ref(packed, scales, s_t):
    """x_hat = E2M1(code) * E4M3(scale) * s_t, in float64 (exact)."""
    code = unpack_codes(packed)
    mag = E2M1_VALUES[code & 7]
    sgn = np.where(code >> 3, -1.0, 1.0)
    scales = np.asarray(scales, dtype=np.uint8)
    assert np.all(scales < 0x7F), "scale byte 0x7F is NaN and is never produced"
    D = code.shape[-1]
    bsv = np.repeat(E4M3_VALUES[scales], BLOCK, axis=-1)
    assert bsv.shape[-1] == D
    return sgn * mag * bsv * float(s_t)
