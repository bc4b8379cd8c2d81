"""Pins of the oracle's dequantized cache, CacheModel.dequantized_kv: the float64 K
and V of the effective key set that the attention oracle consumes.

Paper text, section 4.2 (global sink, shot-level sink, sliding window, duplicates
removed) fixes WHICH frames are attended; the reading note, "The inference
infrastructure", fixes that each appended chunk is quantized on its own (its own
tensor scales, K-smoothing means and adaptive V scales) and dequantized for
attention.  So every attended row must be the dequantization of its own chunk's
bytes, with that chunk's scales and (K-smoothing) that chunk's means added back.

Two independent checks, each on a hand-worked schedule with an eviction, a scene
cut and a shot-level-sink frame kept after the window rolled past it:
  * assembly: the expected K/V are built here from whole-chunk codec calls and a
    hand-derived list of attended frame numbers, then compared element by element;
  * accuracy: every attended row must lie within the format's own error bound of the
    bf16 values that were appended at that frame (per 16-element NVFP4 block:
    |x - x_hat| <= eff <= (1 + 2^-4) amax_b / 6; per 32-element MXFP4 block:
    |x - x_hat| <= 2 * 2^E <= amax_b / 2), which ties the model to its inputs
    without using the model's own bookkeeping.
Planted mistakes (V decoded with K's scale, another chunk's scales, a dropped
K-smoothing mean, a frame taken from the wrong position, MXFP4 bytes decoded as
NVFP4) must each fail one of the checks."""

import copy

import numpy as np
import pytest

from oracle import CacheModel, channel_mean_ref, dequantize_ref, mx_dequantize_ref, mx_quantize_ref, quantize_ref
from oracle.nvfp4_ref import bf16_bits_to_f32
from nvfp4_kv_cache_amd import workloads as W

H, D, T_F = 2, 32, 8
SINK, WINDOW, SHOT = 1, 3, 2

# Hand-worked schedule.  Frames are numbered in append order; chunk c brings the
# frames listed in CHUNK_FRAMES[c].  After each step, the attended frames in the
# model's documented order (global sink, shot-level-sink frames that left the
# window, window oldest first):
#   append 2  (frames 0,1)   sink [0], window [1]                      -> 0 1
#   append 2  (frames 2,3)   window [1 2 3]                            -> 0 1 2 3
#   scene cut: the shot-level sink becomes frames [4, 6)
#   append 2  (frames 4,5)   1 and 2 leave the window (not shot frames) -> 0 3 4 5
#   append 3  (frames 6,7,8) 3 leaves; 4 and 5 leave but are shot frames -> 0 4 5 6 7 8
#   evict 1                  6 leaves                                  -> 0 4 5 7 8
#   append 1  (frame 9)      window [7 8 9]                            -> 0 4 5 7 8 9
SCHEDULE = [("append", 2, [0, 1]), ("append", 2, [0, 1, 2, 3]), ("cut", 0, None),
            ("append", 2, [0, 3, 4, 5]), ("append", 3, [0, 4, 5, 6, 7, 8]),
            ("evict", 1, [0, 4, 5, 7, 8]), ("append", 1, [0, 4, 5, 7, 8, 9])]
CHUNK_FRAMES = [[0, 1], [2, 3], [4, 5], [6, 7, 8], [9]]
# per-chunk magnitudes (so that any other chunk's scale is off by >= 4x) and V at
# 8x K (so that K's scale applied to V is off by 8x)
MAG = [1.0, 16.0, 0.25, 4.0, 64.0]

CONFIGS = {
    "nvfp4": dict(),
    "smooth_adaptive": dict(k_smooth=True, v_adaptive=True),
    "mxfp4": dict(mxfp4=True),
}


def make_chunks(seed):
    rng = np.random.default_rng(seed)
    chunks = []
    for c, frames in enumerate(CHUNK_FRAMES):
        T = len(frames) * T_F
        # K with large per-channel offsets: K-smoothing's means are far from zero
        k = (rng.standard_normal((H, T, D)) + 6.0 * rng.standard_normal((H, 1, D))) * MAG[c]
        v = rng.standard_normal((H, T, D)) * MAG[c] * 8.0
        chunks.append((W.f32_to_bf16_bits(k.astype(np.float32)), W.f32_to_bf16_bits(v.astype(np.float32))))
    return chunks


def chunk_dequant(k, v, cfg):
    """Whole-chunk codec round trip: float64 K_hat (means added back), V_hat."""
    if cfg.get("mxfp4"):
        return mx_dequantize_ref(*mx_quantize_ref(k)), mx_dequantize_ref(*mx_quantize_ref(v))
    mu = channel_mean_ref(k) if cfg.get("k_smooth") else None
    kc, ks, sk = quantize_ref(k, mean=mu)
    vc, vs, sv = quantize_ref(v, adaptive=cfg.get("v_adaptive", False))
    kh = dequantize_ref(kc, ks, sk)
    if mu is not None:
        kh = kh + mu.astype(np.float64)[:, None, :]
    return kh, dequantize_ref(vc, vs, sv)


def frame_rows(frame):
    """(chunk, token slice within the chunk) of a frame number, from CHUNK_FRAMES."""
    for c, frames in enumerate(CHUNK_FRAMES):
        if frame in frames:
            i = frames.index(frame)
            return c, slice(i * T_F, (i + 1) * T_F)
    raise AssertionError(frame)


def check_assembly(model, chunks, keff, cfg):
    """dequantized_kv() equals the hand-assembled rows of the attended frames."""
    got_k, got_v = model.dequantized_kv()
    deq = [chunk_dequant(k, v, cfg) for k, v in chunks]
    want_k = np.concatenate([deq[frame_rows(f)[0]][0][:, frame_rows(f)[1]] for f in keff], axis=1)
    want_v = np.concatenate([deq[frame_rows(f)[0]][1][:, frame_rows(f)[1]] for f in keff], axis=1)
    assert got_k.shape == want_k.shape == (H, len(keff) * T_F, D)
    assert np.array_equal(got_k, want_k), "K rows differ from their chunks' own dequantization"
    assert np.array_equal(got_v, want_v), "V rows differ from their chunks' own dequantization"


def block_bound_ok(x, x_hat, cfg, smooth_mean=None):
    """Per-block error bound of the format against the appended bf16 values."""
    x = np.asarray(x, dtype=np.float64)
    err = np.abs(x - x_hat)
    if cfg.get("mxfp4"):
        blk, frac = 32, 0.5
    else:
        blk, frac = 16, (1.0 + 2.0 ** -4) / 6.0
    y = x if smooth_mean is None else x - smooth_mean
    amax = np.abs(y).reshape(y.shape[:-1] + (D // blk, blk)).max(axis=-1)
    bound = np.repeat(amax * frac * (1 + 1e-6), blk, axis=-1) + 1e-30
    return bool(np.all(err <= bound))


def check_accuracy(model, chunks, keff, cfg):
    got_k, got_v = model.dequantized_kv()
    for j, f in enumerate(keff):
        c, sl = frame_rows(f)
        rows = slice(j * T_F, (j + 1) * T_F)
        k = bf16_bits_to_f32(chunks[c][0][:, sl]).astype(np.float64)
        v = bf16_bits_to_f32(chunks[c][1][:, sl]).astype(np.float64)
        mu = None
        if cfg.get("k_smooth"):
            mu = channel_mean_ref(chunks[c][0]).astype(np.float64)[:, None, :]
        assert block_bound_ok(k, got_k[:, rows], cfg, mu), f"frame {f}: K beyond the format's error bound"
        assert block_bound_ok(v, got_v[:, rows], cfg), f"frame {f}: V beyond the format's error bound"


def run_schedule(cfg, seed, checks, mutate=None):
    chunks = make_chunks(seed)
    model = CacheModel(H, D, T_F, SINK, WINDOW, shot_frames=SHOT, **cfg)
    nxt = 0
    for op, n, keff in SCHEDULE:
        if op == "cut":
            model.begin_shot()
            continue
        if op == "append":
            k, v = chunks[nxt]
            assert k.shape[1] == n * T_F
            model.append(k, v)
            nxt += 1
        else:
            model.evict(n)
        m = mutate(model) if mutate else model
        for chk in checks:
            chk(m, chunks[:nxt], keff, cfg)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_dequantized_kv_assembly_and_bound(name):
    run_schedule(CONFIGS[name], 7, [check_assembly, check_accuracy])


# ---------------------------------------------------------------- planted mistakes

def _mutated(fn):
    def mutate(model):
        m = copy.deepcopy(model)
        fn(m)
        return m
    return mutate


def _v_takes_k_scale(m):
    for f in m.frames():
        f.s_v = f.s_k


def _newest_chunk_scales(m):
    fs = m.frames()
    newest = max(fs, key=lambda f: f.chunk_id)
    for f in fs:
        f.s_k, f.s_v = newest.s_k, newest.s_v


def _previous_chunk_scales(m):
    # the scales of the chunk appended before the frame's own (a stale scale slot)
    for f in m.frames():
        prev = m.chunk_codes.get(f.chunk_id - 1)
        if prev is not None:
            f.s_k, f.s_v = prev[2], prev[5]


def _drop_mean(m):
    for f in m.frames():
        f.k_mean = None


def _wrong_frame_of_chunk(m):
    # a frame of a multi-frame chunk reads its neighbour's rows
    for f in m.frames():
        kc, ks, _, vc, vs, _ = m.chunk_codes[f.chunk_id]
        n = kc.shape[1] // m.T_f
        if n > 1:
            j = (f.frame_in_chunk + 1) % n
            sl = slice(j * m.T_f, (j + 1) * m.T_f)
            f.k_codes, f.k_scales, f.v_codes, f.v_scales = kc[:, sl], ks[:, sl], vc[:, sl], vs[:, sl]
            return


def _mx_as_nvfp4(m):
    for f in m.frames():
        f.mx = False


PLANTED = [
    ("nvfp4", _v_takes_k_scale), ("nvfp4", _newest_chunk_scales), ("nvfp4", _previous_chunk_scales),
    ("nvfp4", _wrong_frame_of_chunk), ("smooth_adaptive", _drop_mean),
    ("smooth_adaptive", _v_takes_k_scale), ("mxfp4", _mx_as_nvfp4), ("mxfp4", _wrong_frame_of_chunk),
]


@pytest.mark.parametrize("name,fn", PLANTED, ids=[f"{n}-{f.__name__}" for n, f in PLANTED])
def test_planted_mistakes_fail_both_checks(name, fn):
    cfg = CONFIGS[name]
    with pytest.raises(AssertionError):
        run_schedule(cfg, 7, [check_assembly], mutate=_mutated(fn))
    if fn is not _wrong_frame_of_chunk:   # a neighbour frame still meets the format's bound
        with pytest.raises(AssertionError):
            run_schedule(cfg, 7, [check_accuracy], mutate=_mutated(fn))
