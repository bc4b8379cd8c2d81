"""MXFP4 codec oracle (plain numpy; test infrastructure only).

What the pages fix
------------------
Paper text, appendix A.2 "FP4 Quantization": MXFP4 is the other block-scaled FP4
format.  Set against it, NVFP4 has the finer 16-element blocks, E4M3 block scales
and a tensor-level scale on top; so MXFP4 has coarser blocks, a block scale that
is not E4M3 and no tensor-level scale.  For the format itself the appendix cites
the OCP Microscaling Formats (MX) specification, version 1.0.

Readings (the cited specification's MXFP4, restated)
-----------------------------------------------------------------------------
* Block: 32 consecutive elements along the last (head_dim) axis.
* Block scale: a power of two X = 2^E, stored as an E8M0 byte E + 127 (E in
  [-127, 127]; the byte 0xFF is NaN and is never produced).  E is the block
  maximum's binary exponent, floor(log2(amax_b)), minus 2 -- the exponent of
  E2M1's largest magnitude, 6 = 1.5 * 2^2 -- clamped to [-127, 127].  An all-zero
  block takes E = -127 (byte 0x00).
* Element: x / X, which is exact (a power-of-two scaling of a bf16 value), rounded
  to E2M1 to nearest with ties to the even code and saturating at 6.  Because
  amax_b / X lies in [4, 8), block maxima above 6 X clip to 6 X, which the
  specification accepts.  code = sign << 3 | magnitude; the sign of -0.0 is kept.
* Packing as for NVFP4: two codes per byte, the even element in the low nibble;
  scales are the raw E8M0 bytes.
* Dequantized value: E2M1(code) * 2^(byte - 127), exact in float64.

Every step is exact or an integer decision, so the steps above define every bit.

MXFP8 queries (for the variant whose cache logits run on gfx950's MX-scaled matrix
cores, which take both operands in an MX format): the same specification's MXFP8
with E4M3 elements -- 32-element blocks along head_dim, E = floor(log2(block max))
- 8 (8 = the exponent of E4M3's largest magnitude 448 = 1.75 * 2^8) clamped to
[-127, 127], elements E4M3(x / 2^E) nearest-even and saturating at 448 (block maxima
in (448, 512) * 2^E clip), the sign kept (-0 -> 0x80).
"""

import numpy as np

from .nvfp4_ref import E2M1_VALUES, E4M3_VALUES, bf16_bits_to_f32, e2m1_encode, e4m3_encode, unpack_codes

MX_BLOCK = 32
E2M1_EMAX = 2          # 6 = 1.5 * 2^2
E4M3_EMAX = 8          # 448 = 1.75 * 2^8
E8M0_BIAS = 127


def mx_block_exponent(amax_b, emax=E2M1_EMAX):
    """E = floor(log2(amax_b)) - emax clamped to [-127, 127]; -127 for a zero block.
    amax_b: float values >= 0 (finite); emax: the element format's largest exponent."""
    a = np.asarray(amax_b, dtype=np.float64)
    mant, ex = np.frexp(a)              # a = mant * 2^ex, mant in [0.5, 1) for a > 0
    e = (ex - 1) - emax                 # floor(log2 a) = ex - 1, exactly
    e = np.where(a > 0, e, -E8M0_BIAS)
    return np.clip(e, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)


def mx_quantize_ref(x_bits):
    """Quantize bf16 bit patterns x_bits [..., D] (D % 32 == 0) to MXFP4.

    Returns (codes uint8 [..., D/2], scales uint8 [..., D/32] as E8M0 bytes).
    Steps follow the module docstring, in order.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    D = x_bits.shape[-1]
    assert D % MX_BLOCK == 0
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    assert np.all(np.isfinite(x)), "inputs must be finite"
    sign = ((x_bits >> 15) & 1).astype(np.uint8)
    lead = x.shape[:-1]
    nb = D // MX_BLOCK
    ax = np.abs(x).reshape(lead + (nb, MX_BLOCK))
    E = mx_block_exponent(ax.max(axis=-1))
    q = ax * np.exp2(-E.astype(np.float64))[..., None]      # exact power-of-two scaling
    mag = e2m1_encode(q)
    code = (sign.reshape(lead + (nb, MX_BLOCK)) << 3) | mag
    code = code.reshape(lead + (D,))
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, (E + E8M0_BIAS).astype(np.uint8)


def mx_dequantize_ref(packed, scales):
    """x_hat = E2M1(code) * 2^(scale byte - 127), in float64 (exact)."""
    code = unpack_codes(packed)
    mag = E2M1_VALUES[code & 7]
    sgn = np.where(code >> 3, -1.0, 1.0)
    scales = np.asarray(scales, dtype=np.uint8)
    assert np.all(scales < 0xFF), "E8M0 byte 0xFF is NaN and is never produced"
    X = np.exp2(scales.astype(np.float64) - E8M0_BIAS)
    Xv = np.repeat(X, MX_BLOCK, axis=-1)
    assert Xv.shape[-1] == code.shape[-1]
    return sgn * mag * Xv


def mxfp8_quantize_ref(x_bits):
    """Quantize bf16 bit patterns x_bits [..., D] (D % 32 == 0) to MXFP8 (E4M3
    elements).  Returns (codes uint8 [..., D] as E4M3 bytes, scales uint8 [..., D/32]
    as E8M0 bytes).  Steps follow the module docstring."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    D = x_bits.shape[-1]
    assert D % MX_BLOCK == 0
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    assert np.all(np.isfinite(x)), "inputs must be finite"
    sign = ((x_bits >> 15) & 1).astype(np.uint8)
    lead = x.shape[:-1]
    nb = D // MX_BLOCK
    ax = np.abs(x).reshape(lead + (nb, MX_BLOCK))
    E = mx_block_exponent(ax.max(axis=-1), E4M3_EMAX)
    q = ax * np.exp2(-E.astype(np.float64))[..., None]      # exact power-of-two scaling
    mag = e4m3_encode(q).reshape(lead + (D,))               # nearest-even, saturating at 448
    return ((sign << 7) | mag).astype(np.uint8), (E + E8M0_BIAS).astype(np.uint8)


def mxfp8_dequantize_ref(codes, scales):
    """x_hat = E4M3(code) * 2^(scale byte - 127), in float64 (exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    assert np.all((codes & 0x7F) != 0x7F), "E4M3 0x7F / 0xFF is NaN and is never produced"
    mag = E4M3_VALUES[codes & 0x7F]
    sgn = np.where(codes >> 7, -1.0, 1.0)
    X = np.repeat(np.exp2(np.asarray(scales, dtype=np.float64) - E8M0_BIAS), MX_BLOCK, axis=-1)
    return sgn * mag * X
