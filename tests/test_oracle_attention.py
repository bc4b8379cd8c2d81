"""Pins for the attention oracle: closed forms, invariances, a pure-Python
brute force on a tiny case, and the cache model against the effective-key-set
definition (paper text, section 4.2)."""

import math

import numpy as np
import pytest

from oracle import attention_from_kv, chunk_attention_ref, CacheModel
from oracle.nvfp4_ref import bf16_bits_to_f32
from nvfp4_kv_cache_amd import workloads as W


def test_brute_force_tiny():
    rng = np.random.default_rng(0)
    q, k, v = rng.normal(size=(1, 3, 4)), rng.normal(size=(1, 5, 4)), rng.normal(size=(1, 5, 4))
    s = 0.37
    got = attention_from_kv(q, k, v, s)
    for i in range(3):
        logits = [s * sum(q[0, i, d] * k[0, j, d] for d in range(4)) for j in range(5)]
        w = [math.exp(z) for z in logits]
        tot = sum(w)
        for d in range(4):
            want = sum(w[j] * v[0, j, d] for j in range(5)) / tot
            assert abs(got[0, i, d] - want) < 1e-13


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(1)
    k, v = rng.normal(size=(2, 37, 8)), rng.normal(size=(2, 37, 8))
    q = np.zeros((2, 5, 8))
    got = attention_from_kv(q, k, v, 0.5)
    assert np.allclose(got, v.mean(axis=1, keepdims=True).repeat(5, axis=1), atol=1e-14)


def test_constant_value_rows():
    rng = np.random.default_rng(2)
    q, k = rng.normal(size=(1, 9, 16)), rng.normal(size=(1, 50, 16))
    row = rng.normal(size=16)
    v = np.tile(row, (1, 50, 1))
    assert np.allclose(attention_from_kv(q, k, v, 0.25), row, atol=1e-14)


def test_dominant_key():
    rng = np.random.default_rng(3)
    q, k, v = rng.normal(size=(1, 4, 16)), rng.normal(size=(1, 20, 16)), rng.normal(size=(1, 20, 16))
    k[0, 7] = q[0, 2] * 100.0
    got = attention_from_kv(q, k, v, 1.0)
    assert np.allclose(got[0, 2], v[0, 7], atol=1e-12)


def test_key_permutation_and_block_split_invariance():
    rng = np.random.default_rng(4)
    q, k, v = rng.normal(size=(2, 70, 16)), rng.normal(size=(2, 41, 16)), rng.normal(size=(2, 41, 16))
    base = attention_from_kv(q, k, v, 0.3, block=16)
    perm = rng.permutation(41)
    assert np.allclose(attention_from_kv(q, k[:, perm], v[:, perm], 0.3), base, atol=1e-13)
    # log-sum-exp merge of two key segments equals the whole
    def part(ks, vs):
        s = np.einsum("hqd,hkd->hqk", q, ks) * 0.3
        m = s.max(-1, keepdims=True)
        p = np.exp(s - m)
        return np.einsum("hqk,hkd->hqd", p, vs), p.sum(-1, keepdims=True), m
    o1, l1, m1 = part(k[:, :20], v[:, :20])
    o2, l2, m2 = part(k[:, 20:], v[:, 20:])
    m = np.maximum(m1, m2)
    merged = (o1 * np.exp(m1 - m) + o2 * np.exp(m2 - m)) / (l1 * np.exp(m1 - m) + l2 * np.exp(m2 - m))
    assert np.allclose(merged, base, atol=1e-13)


def test_rows_subset_matches_full():
    rng = np.random.default_rng(5)
    q, k, v = rng.normal(size=(3, 50, 8)), rng.normal(size=(3, 30, 8)), rng.normal(size=(3, 30, 8))
    rows = np.array([0, 7, 49, 13])
    assert np.array_equal(attention_from_kv(q, k, v, 0.2, rows=rows),
                          attention_from_kv(q, k, v, 0.2)[:, rows])


def test_chunk_attention_unquantized_cache_equals_direct():
    """A cache whose values are already exact (any float64 K/V) plus the own
    bf16 segment: the result equals softmax attention over the concatenation."""
    rng = np.random.default_rng(6)
    wl = W.WORKLOADS["tiny"]
    q, ko, vo = W.noisy_chunk(wl, 1)
    ck, cv = rng.normal(size=(1, 256, 64)), rng.normal(size=(1, 256, 64))
    got = chunk_attention_ref(q, ko, vo, ck, cv, wl.softmax_scale)
    k = np.concatenate([ck, bf16_bits_to_f32(ko).astype(np.float64)], axis=1)
    v = np.concatenate([cv, bf16_bits_to_f32(vo).astype(np.float64)], axis=1)
    qq = bf16_bits_to_f32(q).astype(np.float64)
    # direct, written differently: per-row loop with log-sum-exp
    for i in range(0, 64, 9):
        z = k[0] @ qq[0, i] * wl.softmax_scale
        lse = np.logaddexp.reduce(z)
        want = np.exp(z - lse) @ v[0]
        assert np.allclose(got[0, i], want, atol=1e-12)


# ---------------------------------------------------------------- cache model

@pytest.mark.parametrize("seed", range(8))
def test_cache_model_matches_keff_definition(seed):
    """Paper text, section 4.2: K_eff = global sink (first S_g frames) union the
    last-W window, duplicates removed.  Index arithmetic: the window is the
    run of non-sink frame numbers [lo, n), where lo only moves forward -- by an
    explicit eviction, or to n - W when the window overflows."""
    rng = np.random.default_rng(seed)
    sink, window, T_f = int(rng.integers(0, 4)), int(rng.integers(1, 7)), 16
    cm = CacheModel(1, 16, T_f, sink, window)
    n, lo = 0, sink
    for _ in range(30):
        n_win = max(0, n - max(lo, sink))
        if rng.random() < 0.25 and n_win > 0:
            e = int(rng.integers(1, n_win + 1))
            cm.evict(e)
            lo = max(lo, sink) + e
        nf = int(rng.integers(1, window + 1))
        k = (rng.integers(0, 2 ** 14, size=(1, nf * T_f, 16))).astype(np.uint16)
        cm.append(k, k)
        n += nf
        lo = max(lo, n - window, sink)
        starts, acc = {}, 0
        for c in sorted(cm.chunk_codes):
            starts[c] = acc
            acc += cm.chunk_codes[c][0].shape[1] // T_f
        ids = [starts[f.chunk_id] + f.frame_in_chunk for f in cm.frames()]
        want = list(range(min(n, sink))) + list(range(max(lo, sink), n))
        assert ids == want
        assert cm.n_tokens() == len(want) * T_f


def _frame_numbers(cm):
    starts, acc = {}, 0
    for c in sorted(cm.chunk_codes):
        starts[c] = acc
        acc += cm.chunk_codes[c][0].shape[1] // cm.T_f
    return [starts[f.chunk_id] + f.frame_in_chunk for f in cm.frames()]


def test_shot_sink_hand_schedule():
    """The hand-worked multi-shot schedule of tests/golden/shot_sink_schedule.json
    (paper text, section 4.2, 'Multi-Shot Attention Sink')."""
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "shot_sink_schedule.json")))
    c = g["config"]
    T_f = 8
    cm = CacheModel(1, 16, T_f, c["sink_frames"], c["window_frames"], shot_frames=c["shot_frames"])
    for st in g["steps"]:
        if st["op"] == "cut":
            cm.begin_shot()
            continue
        if st["op"] == "append":
            k = np.zeros((1, st["frames"] * T_f, 16), dtype=np.uint16)
            cm.append(k, k)
        else:
            cm.evict(st["frames"])
        assert _frame_numbers(cm) == st["keff"], st.get("why")


@pytest.mark.parametrize("seed", range(8))
def test_cache_model_shot_sink_matches_keff_definition(seed):
    """Paper text, section 4.2: K_eff = A_g U A_s U window, duplicates removed, with
    A_g the first S_g frames, A_s = [s0, s0 + S_s) for the current shot's first frame
    s0 (moved to the next frame number at a scene cut) and the window the run of
    non-sink frame numbers [lo, n) (lo moves forward by evictions and overflow).
    Set arithmetic on frame numbers, independent of the model's frame lists."""
    rng = np.random.default_rng(100 + seed)
    sink, window, shot, T_f = int(rng.integers(0, 4)), int(rng.integers(1, 7)), int(rng.integers(0, 5)), 8
    cm = CacheModel(1, 16, T_f, sink, window, shot_frames=shot)
    n, lo, s0 = 0, sink, 0
    for _ in range(40):
        if rng.random() < 0.2:
            cm.begin_shot()
            s0 = n
        n_win = max(0, n - max(lo, sink))
        if rng.random() < 0.2 and n_win > 0:
            e = int(rng.integers(1, n_win + 1))
            cm.evict(e)
            lo = max(lo, sink) + e
        nf = int(rng.integers(1, window + 1))
        k = np.zeros((1, nf * T_f, 16), dtype=np.uint16)
        cm.append(k, k)
        n += nf
        lo = max(lo, n - window, sink)
        a_g = list(range(min(n, sink)))
        win = list(range(max(lo, sink), n))
        a_s_out = [f for f in range(s0, min(s0 + shot, n)) if sink <= f < lo]
        want = a_g + a_s_out + win
        got = _frame_numbers(cm)
        assert got == want
        assert len(set(got)) == len(got)
        assert cm.n_tokens() == len(want) * T_f
