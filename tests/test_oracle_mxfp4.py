"""Pins for the MXFP4 codec oracle against facts it does not compute itself: a
hand-derived worked example, torch's own E8M0 decoding, an independent statement
of the shared-exponent rule (the unique power of two that puts the block maximum
in [4, 8)), a brute-force nearest-grid search for the element codes, the scaling
invariance a power-of-two block scale must have, exact round trips of
representable values and the error bound of the grid."""

import json
import os

import numpy as np
import torch

from oracle import mxfp4_ref as M
from oracle import nvfp4_ref as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_blocks.json")


def bf16_bits(x):
    """float32 values exactly representable in bf16 -> bf16 bits."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all(b & 0xFFFF == 0)
    return (b >> 16).astype(np.uint16)


def random_bf16(rng, shape, scale=1.0):
    x = (rng.standard_t(4, size=shape) * scale).astype(np.float32)
    b = x.view(np.uint32)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16          # RNE to bf16
    return b.astype(np.uint16)


def test_golden_blocks():
    g = json.load(open(GOLDEN))
    rows, D = g["shape"]
    x = np.zeros((rows, D), dtype=np.float32)
    for blk in g["blocks"]:
        vals = np.array(blk["x"], dtype=np.float32)
        base = blk["block"] * 32
        x[blk["row"], base:base + len(vals)] = vals
    codes, scales = M.mx_quantize_ref(bf16_bits(x))
    unpacked = R.unpack_codes(codes)
    for blk in g["blocks"]:
        r, b = blk["row"], blk["block"]
        assert scales[r, b] == blk["scale_byte"], blk["name"]
        n = len(blk["codes"])
        got = unpacked[r, 32 * b:32 * b + 32]
        assert list(got[:n]) == blk["codes"], blk["name"]
        # the unlisted elements are +0: code 0
        assert not np.any(got[n:]), blk["name"]
    # nibble order: element 2i in the low nibble
    assert codes[0, 0] == (7 | (4 << 4))


def test_e8m0_decode_matches_torch():
    # the dequantizer's power of two for every byte, against torch's float8_e8m0fnu
    b = np.arange(0, 255, dtype=np.uint8)
    tv = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    packed = np.full((255, 16), 0x22, dtype=np.uint8)          # every element 1.0
    xh = M.mx_dequantize_ref(packed, b[:, None])
    assert np.array_equal(xh[:, 0], tv)
    assert np.all(xh == tv[:, None])


def test_shared_exponent_by_search():
    # independent statement: E is the integer with 4 <= amax / 2^E < 8, clamped
    rng = np.random.default_rng(11)
    amax = np.concatenate([np.exp2(rng.uniform(-140, 130, 4000)), [4.0, 7.999, 8.0, 1.0, 6.0, 2.0 ** -126]])
    amax = amax[np.isfinite(amax)]
    got = M.mx_block_exponent(amax)
    for a, e in zip(amax, got):
        E = 0
        while a / 2.0 ** E >= 8.0:
            E += 1
        while a / 2.0 ** E < 4.0:
            E -= 1
        assert e == min(max(E, -127), 127), a
    assert M.mx_block_exponent(np.array([0.0]))[0] == -127


def test_element_codes_by_brute_force():
    # every code is the nearest grid value of x / X (ties to the even code),
    # found here by exhaustive comparison with the 8 magnitudes
    rng = np.random.default_rng(12)
    xb = random_bf16(rng, (6, 40, 64))
    codes, scales = M.mx_quantize_ref(xb)
    x = R.bf16_bits_to_f32(xb).astype(np.float64)
    X = np.repeat(np.exp2(scales.astype(np.float64) - 127), 32, axis=-1)
    q = np.abs(x) / X
    grid = R.E2M1_VALUES
    d = np.abs(q[..., None] - grid)                 # [..., 8]
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # among equally near entries take the even index; beyond 6 the last one
    idx = np.where(cand[..., ::2].any(axis=-1), np.argmax(cand * (np.arange(8) % 2 == 0), axis=-1),
                   np.argmax(cand, axis=-1))
    idx = np.where(q >= 6.0, 7, idx)
    c = R.unpack_codes(codes)
    assert np.array_equal(c & 7, idx)
    assert np.array_equal(c >> 3, (xb >> 15).astype(np.uint8))


def test_scaling_invariance():
    # multiplying a tensor by 2^k (exact in bf16) shifts every scale byte by k and
    # leaves the codes alone, as long as no exponent leaves the clamp range
    rng = np.random.default_rng(13)
    xb = random_bf16(rng, (3, 20, 64))
    c0, s0 = M.mx_quantize_ref(xb)
    for k in (-20, -3, 1, 7, 40):
        xk = (R.bf16_bits_to_f32(xb) * np.float32(2.0 ** k)).astype(np.float32)
        ck, sk = M.mx_quantize_ref(bf16_bits(xk))
        assert np.array_equal(ck, c0)
        assert np.array_equal(sk.astype(int), s0.astype(int) + k)


def test_representable_values_round_trip():
    # blocks made of grid values times one power of two, with a 4 or 6 in them,
    # come back exactly
    rng = np.random.default_rng(14)
    for E in (-127, -60, -2, 0, 5, 100, 125):
        mags = rng.integers(0, 8, size=(4, 64))
        mags[:, 0] = 7
        mags[:, 32] = 6
        sign = rng.integers(0, 2, size=(4, 64))
        x = (np.where(sign, -1.0, 1.0) * R.E2M1_VALUES[mags] * 2.0 ** E).astype(np.float32)
        xb = bf16_bits(x)
        codes, scales = M.mx_quantize_ref(xb)
        assert np.all(scales == E + 127)
        xh = M.mx_dequantize_ref(codes, scales)
        assert np.array_equal(xh, x.astype(np.float64))


def test_error_bound():
    # |x - x_hat| is at most half the grid step at |x| / X, except above 6 X (clipped)
    rng = np.random.default_rng(15)
    xb = random_bf16(rng, (4, 50, 128), scale=3.0)
    codes, scales = M.mx_quantize_ref(xb)
    x = R.bf16_bits_to_f32(xb).astype(np.float64)
    xh = M.mx_dequantize_ref(codes, scales)
    X = np.repeat(np.exp2(scales.astype(np.float64) - 127), 32, axis=-1)
    q = np.abs(x) / X
    half_step = np.where(q < 2, 0.25, np.where(q < 4, 0.5, 1.0)) * X
    ok = np.abs(x - xh) <= half_step
    clipped = q > 6
    assert np.all(ok | clipped)
    assert np.all(np.abs(xh[clipped]) == 6 * X[clipped])
    # the block maximum lands in [4, 8) X whenever the exponent is not clamped
    blocks = np.abs(x).reshape(4, 50, 4, 32).max(axis=-1)
    r = blocks / np.exp2(scales.astype(np.float64) - 127)
    assert np.all((r >= 4) & (r < 8))
