"""Pins for the NVFP4 codec oracle against facts it does not compute itself:
the format constants of the pages, a hand-derived worked example, an
independent interval formulation of E2M1 rounding, torch's float8_e4m3fn cast,
and algebraic invariants of the quantizer."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nvfp4_ref as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_hand_example.json")


def f32(x):
    return np.asarray(x, dtype=np.float32)


def to_bf16_exact(vals):
    """float list (with "-0") -> bf16 bits, asserting each value is exact."""
    out = []
    for v in vals:
        fv = -0.0 if v == "-0" else float(v)
        b = np.array([fv], dtype=np.float32).view(np.uint32)[0]
        assert b & 0xFFFF == 0, f"{v} is not exactly a bf16 value"
        out.append(b >> 16)
    return np.array(out, dtype=np.uint16)


# ---------------------------------------------------------------- formats

def test_e2m1_grid_matches_format():
    # reading note, section II: E2M1 = 1 sign, 2 exponent, 1 mantissa bit;
    # paper section 2.2: largest magnitude 6.
    assert list(R.E2M1_VALUES) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e4m3_grid_matches_format():
    # paper section 2.2: E4M3 largest magnitude 448 (OCP E4M3FN, not FNUZ's 240)
    v = R.E4M3_VALUES
    assert len(v) == 127 and v[-1] == 448.0
    assert np.all(np.diff(v) > 0)
    assert v[1] == 2.0 ** -9 and v[8] == 2.0 ** -6 and v[0x38] == 1.0
    # cross-check every code against torch's own float8_e4m3fn decoding
    codes = torch.arange(0, 127, dtype=torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(tv, v)


# ---------------------------------------------------------------- E2M1

def e2m1_by_intervals(q):
    """Independent statement of E2M1 round-half-to-even: the closed/open ends
    of each interval encode where the ties go (to the even code)."""
    q = np.asarray(q, dtype=np.float64)
    out = np.full(q.shape, 7, dtype=np.uint8)
    rules = [  # (upper bound, inclusive?, code) scanned from the top down
        (5.0, True, 6), (3.5, False, 5), (2.5, True, 4), (1.75, False, 3),
        (1.25, True, 2), (0.75, False, 1), (0.25, True, 0)]
    for ub, incl, code in rules:
        m = (q <= ub) if incl else (q < ub)
        out[m] = code
    return out


def test_e2m1_hand_points_and_ties():
    q = [0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 7, 1e30]
    want = [0, 0, 1, 2, 2, 2, 3, 4, 4, 4, 5, 6, 6, 6, 7, 7, 7]
    assert list(R.e2m1_encode(f32(q))) == want


def _ulp_neighbourhood(points, span):
    base = f32(points).view(np.int32)
    offs = np.arange(-span, span + 1, dtype=np.int32)
    b = (base[:, None] + offs[None, :]).ravel()
    b = b[b >= 0]
    return b.view(np.float32)


def test_e2m1_matches_interval_rule_dense():
    pts = [0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6]
    near = _ulp_neighbourhood(pts, 4096)
    rng = np.random.default_rng(7)
    rnd = rng.uniform(0, 8, 2_000_000).astype(np.float32)
    big = f32([6.5, 7.9, 8.0, 100.0, 3e38])
    tiny = np.arange(0, 4096, dtype=np.int32).view(np.float32)   # zero and subnormals
    q = np.concatenate([near, rnd, big, tiny])
    assert np.array_equal(R.e2m1_encode(q), e2m1_by_intervals(q))


# ---------------------------------------------------------------- E4M3

def test_e4m3_matches_torch_cast():
    v = R.E4M3_VALUES
    mids = (v[:-1] + v[1:]) / 2
    pts = np.concatenate([v, mids, [464.0]])
    near = _ulp_neighbourhood(pts.astype(np.float32), 64)
    near = near[near <= 464.0]
    rng = np.random.default_rng(11)
    logu = np.exp2(rng.uniform(-12, np.log2(464), 2_000_000)).astype(np.float32)
    sub = np.arange(0, 200000, 7, dtype=np.int32).view(np.float32)
    x = np.concatenate([near, logu, sub])
    x = x[x <= 464.0]
    ours = R.e4m3_encode(x)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_e4m3_hand_points():
    x = f32([2.0 ** -10, 1.5 * 2 ** -9, 2.5 * 2 ** -9, 42.6667, 448.0, 460.0, 1e9])
    assert list(R.e4m3_encode(x)) == [0x00, 0x02, 0x02, 0x63, 0x7E, 0x7E, 0x7E]


# ---------------------------------------------------------------- worked example

@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_golden_hand_example(case):
    shape = tuple(case["shape"])
    bits = np.stack([to_bf16_exact(row) for row in case["x"]]).reshape(shape)
    codes, scales, s_t = R.quantize_ref(bits)
    assert np.float32(s_t) == np.float32(case["s_t"])
    assert np.array_equal(scales.reshape(len(case["scales"]), -1), np.array(case["scales"]))
    unpacked = R.unpack_codes(codes).reshape(len(case["codes"]), -1)
    assert np.array_equal(unpacked, np.array(case["codes"]))
    assert np.array_equal(codes.reshape(len(case["packed"]), -1), np.array(case["packed"]))
    # packing rule: even element in the low nibble
    c = np.array(case["codes"])
    assert np.array_equal(c[:, 0::2] | (c[:, 1::2] << 4), np.array(case["packed"]))


# ---------------------------------------------------------------- invariants

def _grid_tensor(rng, H, T, D, log2_st):
    """Values exactly on the NVFP4 grid: every block holds a +-6 code, so its
    amax is 6 * bs * s_t and the quantizer must reproduce bs and the codes.
    One block uses bs = 448 so the tensor amax gives s_t = 2^log2_st."""
    nb = D // 16
    s_t = 2.0 ** log2_st
    scales = rng.integers(0x20, 0x7E, size=(H, T, nb))     # normal E4M3 codes
    scales[0, 0, 0] = 0x7E
    codes = rng.integers(0, 16, size=(H, T, D))
    blk = codes.reshape(H, T, nb, 16)
    pos = rng.integers(0, 16, size=(H, T, nb))
    np.put_along_axis(blk, pos[..., None], 7 + 8 * rng.integers(0, 2, size=(H, T, nb, 1)), axis=-1)
    codes = blk.reshape(H, T, D)
    mag = R.E2M1_VALUES[codes & 7]
    sgn = np.where(codes >> 3, -1.0, 1.0)
    vals = sgn * mag * np.repeat(R.E4M3_VALUES[scales], 16, axis=-1) * s_t
    x32 = vals.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), vals)
    bits = x32.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    return (bits >> 16).astype(np.uint16), codes.astype(np.uint8), scales.astype(np.uint8), s_t


@pytest.mark.parametrize("log2_st", [-8, -3, 0, 4])
def test_round_trip_on_grid(log2_st):
    rng = np.random.default_rng(100 + log2_st)
    bits, codes, scales, s_t = _grid_tensor(rng, 2, 33, 64, log2_st)
    pc, ps, st = R.quantize_ref(bits)
    assert float(st) == s_t
    assert np.array_equal(ps, scales)
    assert np.array_equal(R.unpack_codes(pc), codes)
    # and dequantization is exact
    x = R.bf16_bits_to_f32(bits).astype(np.float64)
    assert np.array_equal(R.dequantize_ref(pc, ps, st), x)


def _random_bf16(rng, shape, scale=1.0):
    x = (rng.standard_t(4, size=shape) * scale).astype(np.float32)
    b = x.view(np.uint32)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def test_amax_block_maps_to_six_and_tensor_block_to_448():
    rng = np.random.default_rng(3)
    bits = _random_bf16(rng, (3, 50, 128))
    codes, scales, s_t = R.quantize_ref(bits)
    x = R.bf16_bits_to_f32(bits)
    ax = np.abs(x).reshape(3, 50, 8, 16)
    c = R.unpack_codes(codes).reshape(3, 50, 8, 16)
    arg = ax.argmax(-1)
    cmax = np.take_along_axis(c, arg[..., None], -1)[..., 0] & 7
    normal = scales >= 0x08          # normal E4M3 scale: relative error <= 2^-4
    assert np.all(cmax[normal] == 7)
    # the block holding the tensor amax gets 448
    h, t, b = np.unravel_index(np.argmax(ax.max(-1)), ax.shape[:3])
    assert scales[h, t, b] == 0x7E


def test_error_bound_and_bytes():
    rng = np.random.default_rng(5)
    bits = _random_bf16(rng, (2, 40, 64), scale=3.0)
    codes, scales, s_t = R.quantize_ref(bits)
    assert codes.shape == (2, 40, 32) and scales.shape == (2, 40, 4)
    # byte budget: 1/2 + 1/16 byte per element (reading note: 9/8 T H d for K+V)
    assert codes.nbytes + scales.nbytes == 2 * 40 * 64 * 9 // 16
    x = R.bf16_bits_to_f32(bits).astype(np.float64)
    xh = R.dequantize_ref(codes, scales, s_t)
    eff = np.repeat(R.E4M3_VALUES[scales], 16, axis=-1) * float(s_t)
    err = np.abs(x - xh)
    sat = np.abs(x) > 6 * eff
    # away from saturation the largest E2M1 half-gap is 1 (between 4 and 6),
    # plus fp32 rounding of q
    assert np.all(err[~sat] <= eff[~sat] * (1 + 1e-6))
    assert np.all(np.abs(err[sat] - (np.abs(x[sat]) - 6 * eff[sat])) <= 1e-12 * np.abs(x[sat]) + 1e-300)
    # sign is kept, and the sign of the code matches the sign bit
    c = R.unpack_codes(codes)
    assert np.array_equal((c >> 3).astype(bool), (bits >> 15).astype(bool))


def test_dequantize_exact_rational():
    rng = np.random.default_rng(9)
    bits = _random_bf16(rng, (1, 4, 32))
    codes, scales, s_t = R.quantize_ref(bits)
    xh = R.dequantize_ref(codes, scales, s_t)
    c = R.unpack_codes(codes)
    for t in range(4):
        for d in range(32):
            code = int(c[0, t, d])
            e, m = (code & 7) >> 1, code & 1
            mag = Fraction(m, 2) if e == 0 else (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)
            sb = int(scales[0, t, d // 16])
            se, sm = sb >> 3, sb & 7
            sv = Fraction(sm, 512) if se == 0 else (1 + Fraction(sm, 8)) * Fraction(2) ** (se - 7)
            want = (-1 if code >> 3 else 1) * mag * sv * Fraction(float(s_t))
            assert Fraction(float(xh[0, t, d])) == want


# ---------------------------------------------------------------- K-smoothing, adaptive 4/6

from nvfp4_kv_cache_amd import workloads as W

quantize_ref, dequantize_ref, unpack_codes = R.quantize_ref, R.dequantize_ref, R.unpack_codes
bf16_to_f32 = R.bf16_bits_to_f32

GOLDEN_KA = os.path.join(os.path.dirname(__file__), "golden", "kv_smoothing_adaptive_example.json")


def test_channel_mean_hand_cases():
    from oracle import channel_mean_ref
    for case in json.load(open(GOLDEN_KA))["channel_mean"]:
        ch = np.array(case["channel"], dtype=np.float32)
        x = W.f32_to_bf16_bits(ch.reshape(1, -1, 1) * np.ones((1, 1, 16), np.float32))
        mu = channel_mean_ref(x)
        assert mu.shape == (1, 16)
        assert np.all(mu == np.float32(case["mu"])), case["name"]


@pytest.mark.parametrize("T", [1, 2, 3, 7, 64, 100, 1000, 4680])
def test_channel_mean_exact_cases(T):
    """Constant channels give the constant; small-integer channels (every partial
    sum an exact fp32 integer) give RN(exact sum / T), the sum taken in Python
    integers."""
    from oracle import channel_mean_ref
    rng = np.random.default_rng(T)
    c = W.f32_to_bf16_bits(rng.standard_normal((2, 1, 16)).astype(np.float32))
    x = np.repeat(c, T, axis=1)
    assert np.array_equal(channel_mean_ref(x), bf16_to_f32(c[:, 0]))
    ints = rng.integers(-100, 101, size=(3, T, 32))
    xb = W.f32_to_bf16_bits(ints.astype(np.float32))
    mu = channel_mean_ref(xb)
    want = np.array([[np.float32(int(ints[h, :, d].sum())) / np.float32(T) for d in range(32)]
                     for h in range(3)], dtype=np.float32)
    assert np.array_equal(mu, want)


def test_adaptive_hand_case():
    g = json.load(open(GOLDEN_KA))["adaptive"]
    bits = W.f32_to_bf16_bits(np.array(g["x"], dtype=np.float32).reshape(g["shape"]))
    c0, s0, t0 = quantize_ref(bits)
    c1, s1, t1 = quantize_ref(bits, adaptive=True)
    assert t0 == t1 == np.float32(g["s_t"])
    assert list(s0.reshape(-1)) == g["plain_scales"]
    assert list(s1.reshape(-1)) == g["adaptive_scales"]
    assert list(unpack_codes(c1)[0, 1]) == g["adaptive_codes_token1"]
    assert np.array_equal(unpack_codes(c1)[0, 0], unpack_codes(c0)[0, 0])   # tie: 6 kept


def test_adaptive_never_worse_than_plain():
    """Per block, the adaptive choice's reconstruction error (fp64) is not above
    the plain recipe's, and every block either keeps the plain encoding or takes
    a strictly smaller fp64 error (the fp32 comparison can only flip near-ties)."""
    rng = np.random.default_rng(5)
    x = (rng.standard_t(4, size=(3, 200, 64)) * 2.0).astype(np.float32)
    bits = W.f32_to_bf16_bits(x)
    xf = bf16_to_f32(bits).astype(np.float64)
    out = {}
    for ad in (False, True):
        c, s, t = quantize_ref(bits, adaptive=ad)
        xh = dequantize_ref(c, s, t)
        out[ad] = ((xh - xf) ** 2).reshape(3, 200, 4, 16).sum(-1), s
    e0, s0 = out[False]
    e1, s1 = out[True]
    changed = s0 != s1
    assert changed.any() and not changed.all()
    assert np.all(e1[~changed] == e0[~changed])
    assert np.all(e1[changed] <= e0[changed] * (1 + 1e-6))
    assert e1.sum() < e0.sum()


def test_smoothing_reconstruction():
    """x_hat = dequant(codes of x - mu) + mu is within the per-block error bound of
    the smoothed values, and removing a per-channel offset makes the error
    independent of that offset's size."""
    from oracle import channel_mean_ref
    rng = np.random.default_rng(6)
    base = rng.standard_normal((2, 96, 32)).astype(np.float32)
    offs = (rng.standard_normal((2, 1, 32)) * 40).astype(np.float32)
    bits = W.f32_to_bf16_bits(base + offs)
    mu = channel_mean_ref(bits)
    c, s, t = quantize_ref(bits, mean=mu)
    xs = (bf16_to_f32(bits) - mu[:, None, :]).astype(np.float32).astype(np.float64)
    xh = dequantize_ref(c, s, t)
    from oracle import E4M3_VALUES
    eff = np.repeat(E4M3_VALUES[s] * float(t), 16, axis=-1)
    assert np.all(np.abs(xh - xs) <= eff + 1e-30)
    err_s = np.abs(xh + mu[:, None, :] - bf16_to_f32(bits)).max()
    c2, s2, t2 = quantize_ref(bits)
    err_p = np.abs(dequantize_ref(c2, s2, t2) - bf16_to_f32(bits)).max()
    assert err_s < 0.25 * err_p
