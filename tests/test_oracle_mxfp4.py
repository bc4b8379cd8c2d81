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


# ---------------------------------------------------------------- MXFP8 queries


def test_mxfp8_golden_blocks():
    g = json.load(open(GOLDEN))["mxfp8"]
    rows, D = g["shape"]
    x = np.zeros((rows, D), dtype=np.float32)
    for blk in g["blocks"]:
        vals = np.array(blk["x"], dtype=np.float32)
        x[blk["row"], :len(vals)] = vals
    codes, scales = M.mxfp8_quantize_ref(bf16_bits(x))
    for blk in g["blocks"]:
        r, n = blk["row"], len(blk["codes"])
        assert scales[r, 0] == blk["scale_byte"], blk["name"]
        assert list(codes[r, :n]) == blk["codes"], blk["name"]
        assert not np.any(codes[r, n:]), blk["name"]


def test_mxfp8_against_torch_e4m3_and_exponent_search():
    # the elements against torch's float8_e4m3fn cast of x / 2^E (nearest-even; only
    # where no saturation is involved), saturated ones at 0x7E, E by search
    rng = np.random.default_rng(21)
    xb = random_bf16(rng, (5, 40, 128), scale=2.0)
    codes, scales = M.mxfp8_quantize_ref(xb)
    x = R.bf16_bits_to_f32(xb).astype(np.float64)
    X = np.repeat(np.exp2(scales.astype(np.float64) - 127), 32, axis=-1)
    q = np.abs(x) / X
    small = q <= 448.0
    t = torch.from_numpy(q[small]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes[small] & 0x7F, t)
    assert np.all(codes[~small] & 0x7F == 0x7E)
    assert np.array_equal(codes >> 7, (xb >> 15).astype(np.uint8))
    amax = np.abs(x).reshape(5, 40, 4, 32).max(axis=-1)
    r = amax / np.exp2(scales.astype(np.float64) - 127)
    assert np.all((r >= 256) & (r < 512))


def test_mxfp8_dequantize_every_code():
    # every non-NaN E4M3 byte times every E8M0 byte, against torch's two decoders
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    e4 = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for s in (0, 1, 100, 127, 130, 254):
        e8 = torch.tensor([s], dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).item()
        blk = np.zeros((len(codes) + 31) // 32 * 32, dtype=np.uint8)
        blk[:len(codes)] = codes
        xh = M.mxfp8_dequantize_ref(blk.reshape(-1, 32), np.full((blk.size // 32, 1), s, np.uint8))
        assert np.array_equal(xh.reshape(-1)[:len(codes)], e4 * e8)


def test_two_query_attention_reduces_to_plain():
    # the oracle's cache-query option with the bf16 queries themselves is plain attention,
    # and with different cache queries it changes only the cache logits
    from oracle import chunk_attention_ref
    rng = np.random.default_rng(22)
    H, nq, nc, D = 2, 5, 7, 32
    q, ko, vo = (random_bf16(rng, (H, nq, D)) for _ in range(3))
    kc, vc = rng.standard_normal((H, nc, D)), rng.standard_normal((H, nc, D))
    plain = chunk_attention_ref(q, ko, vo, kc, vc, 0.3)
    q64 = R.bf16_bits_to_f32(q).astype(np.float64)
    assert np.allclose(chunk_attention_ref(q, ko, vo, kc, vc, 0.3, q_cache64=q64), plain, rtol=1e-13, atol=1e-13)
    # brute force for one row with cache queries scaled by 2
    got = chunk_attention_ref(q, ko, vo, kc, vc, 0.3, q_cache64=2 * q64, rows=np.array([3]))
    ko64, vo64 = (R.bf16_bits_to_f32(t).astype(np.float64) for t in (ko, vo))
    for h in range(H):
        s = [0.3 * float(np.dot(2 * q64[h, 3], kc[h, j])) for j in range(nc)]
        s += [0.3 * float(np.dot(q64[h, 3], ko64[h, j])) for j in range(nq)]
        w = np.exp(np.array(s) - max(s))
        w /= w.sum()
        want = w @ np.concatenate([vc[h], vo64[h]], axis=0)
        assert np.allclose(got[h, 0], want, rtol=1e-12, atol=1e-12)
