"""GPU parity of chunk attention over the NVFP4 cache: the oracle builds its own
cache from the same seeded chunks (its own quantizer) and computes float64
softmax attention; the GPU's fp32 output must agree within max-abs 1e-2 and
relative-L2 5e-3, over every output of every head (the full-size Wan-shaped
workloads and the streaming rollout included)."""

import numpy as np
import pytest

from oracle import CacheModel, chunk_attention_ref
from nvfp4_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops(gpu):
    from nvfp4_kv_cache_amd import ops as _ops
    return _ops


def build_both(ops, H, D, T_f, sink, window, chunks):
    """GPU cache and oracle cache fed with the same list of (k_bits, v_bits)."""
    from gpu_util import dev
    cache = ops.KVCache(H, D, T_f, sink, window)
    model = CacheModel(H, D, T_f, sink, window)
    for k, v in chunks:
        nf = k.shape[1] // T_f
        cache.append(dev(k), dev(v), nf)
        model.append(k, v)
    return cache, model


def run_case(ops, cache, model, q, ko, vo, scale, rows=None, what=""):
    from gpu_util import dev, host, check_attention
    print(f"[{what}] n_q={q.shape[1]} cache_tokens={model.n_tokens()}", flush=True)
    out = host(cache.attention(dev(q), dev(ko), dev(vo), scale))
    ck, cv = model.dequantized_kv()
    want = chunk_attention_ref(q, ko, vo, ck, cv, scale, rows=rows)
    got = out if rows is None else out[:, rows]
    return check_attention(got, want, what)


def test_tiny_workload(ops):
    wl = W.WORKLOADS["tiny"]
    cache, model = build_both(ops, wl.n_heads, wl.head_dim, wl.tokens_per_frame, wl.sink_frames,
                              wl.window_frames, [W.clean_chunk(wl, 0)])
    assert model.n_tokens() == 256
    q, ko, vo = W.noisy_chunk(wl, 1)
    run_case(ops, cache, model, q, ko, vo, wl.softmax_scale, what="tiny")


def rand_bits(rng, shape, outliers=True):
    x = rng.standard_normal(shape).astype(np.float32)
    if outliers:
        m = rng.random(shape) < 0.02
        x[m] = rng.standard_t(4, size=int(m.sum())).astype(np.float32)
    return W.f32_to_bf16_bits(x)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("n_q", [1, 100, 257])
def test_ragged_multi_segment(ops, D, n_q):
    """Several chunks with their own scales, a window that wraps (so segments are
    split and reordered), 40-token frames (ragged 64-key tiles) and ragged query
    counts."""
    rng = np.random.default_rng(D + n_q)
    H, T_f, sink, window = 3, 40, 2, 5
    chunks = []
    for nf in (3, 2, 1, 3, 2):
        chunks.append((rand_bits(rng, (H, nf * T_f, D)) , rand_bits(rng, (H, nf * T_f, D))))
    cache, model = build_both(ops, H, D, T_f, sink, window, chunks)
    q, ko, vo = (rand_bits(rng, (H, n_q, D)) for _ in range(3))
    run_case(ops, cache, model, q, ko, vo, 1.0 / np.sqrt(D), what=f"ragged D{D} nq{n_q}")


def test_empty_cache_is_plain_self_attention(ops):
    rng = np.random.default_rng(3)
    H, D = 2, 128
    cache = ops.KVCache(H, D, 64, 1, 3)
    model = CacheModel(H, D, 64, 1, 3)
    q, ko, vo = (rand_bits(rng, (H, 77, D)) for _ in range(3))
    run_case(ops, cache, model, q, ko, vo, 0.0884, what="empty cache")


def test_evicted_frames_are_not_attended(ops):
    rng = np.random.default_rng(4)
    H, D, T_f = 2, 128, 32
    chunks = [(rand_bits(rng, (H, 2 * T_f, D)), rand_bits(rng, (H, 2 * T_f, D))) for _ in range(3)]
    cache, model = build_both(ops, H, D, T_f, 1, 4, chunks)
    cache.evict(2)
    model.evict(2)
    q, ko, vo = (rand_bits(rng, (H, 50, D)) for _ in range(3))
    run_case(ops, cache, model, q, ko, vo, 0.1, what="after evict")


def test_large_logits_and_zero_chunk(ops):
    """A chunk of all-zero K/V (s_t = 0) and queries aligned with one key so that
    a single key dominates its rows."""
    rng = np.random.default_rng(5)
    H, D, T_f = 1, 128, 64
    k0 = np.zeros((H, T_f, D), dtype=np.uint16)
    k1 = rand_bits(rng, (H, 2 * T_f, D))
    v1 = rand_bits(rng, (H, 2 * T_f, D))
    cache, model = build_both(ops, H, D, T_f, 1, 3, [(k0, k0), (k1, v1)])
    q = rand_bits(rng, (H, 64, D), outliers=False)
    kf = W.f32_to_bf16_bits(np.zeros((H, 64, D), dtype=np.float32))
    x = np.zeros((H, 64, D), dtype=np.float32)
    x[0, :, :] = 0.0
    qf = (q.astype(np.uint32) << 16).view(np.float32)
    x[0, 10] = qf[0, 3] * 4.0                        # own key 10 dominates query 3's row
    ko = W.f32_to_bf16_bits(x)
    vo = rand_bits(rng, (H, 64, D))
    run_case(ops, cache, model, q, ko, vo, 1.0, what="dominant key")


@pytest.mark.parametrize("name", ["wan13b", "wan5b"])
def test_wan_shaped_workloads_whole_output(ops, name):
    """The 1.3B- and 5B-shaped workloads at full size, in the launch configuration
    the bench times: every output of every head against the oracle."""
    wl = W.WORKLOADS[name]
    chunks = [W.clean_chunk(wl, c) for c in range(wl.n_cache_chunks)]
    cache, model = build_both(ops, wl.n_heads, wl.head_dim, wl.tokens_per_frame, wl.sink_frames,
                              wl.window_frames, chunks)
    assert model.n_tokens() == (wl.sink_frames + wl.window_frames) * wl.tokens_per_frame
    q, ko, vo = W.noisy_chunk(wl, wl.n_cache_chunks)
    run_case(ops, cache, model, q, ko, vo, wl.softmax_scale, what=name)


def test_wan13b_k_smoothing_adaptive_whole_output(ops):
    """The 1.3B-shaped workload over a cache with K-smoothing and adaptive V scales
    (the configuration the bench times as wan13b_k_smooth_v_adaptive): every output
    of every head against the oracle."""
    from gpu_util import dev, host, check_attention
    wl = W.WORKLOADS["wan13b"]
    cache = ops.KVCache(wl.n_heads, wl.head_dim, wl.tokens_per_frame, wl.sink_frames, wl.window_frames,
                        k_smooth=True, v_adaptive=True)
    model = CacheModel(wl.n_heads, wl.head_dim, wl.tokens_per_frame, wl.sink_frames, wl.window_frames,
                       k_smooth=True, v_adaptive=True)
    for c in range(wl.n_cache_chunks):
        k, v = W.clean_chunk(wl, c)
        cache.append(dev(k), dev(v), wl.chunk_frames)
        model.append(k, v)
    q, ko, vo = W.noisy_chunk(wl, wl.n_cache_chunks)
    out = host(cache.attention(dev(q), dev(ko), dev(vo), wl.softmax_scale))
    ck, cv = model.dequantized_kv()
    want = chunk_attention_ref(q, ko, vo, ck, cv, wl.softmax_scale)
    check_attention(out, want, "wan13b k-smoothing + adaptive V")
    cache.close()


@pytest.mark.parametrize("fmt", [dict(), dict(k_smooth=True, v_adaptive=True), dict(mxfp4=True)],
                         ids=["nvfp4", "ksmooth-adaptive", "mxfp4"])
def test_head_dim_64_at_scale(ops, fmt):
    """head_dim 64 (4-wave workgroups of 128 queries, two per CU) at a size that cuts
    most query blocks between workgroups: 16 heads, 2085 queries (a ragged last
    block) over a full 2 + 8-frame cache of 1024-token frames appended as five
    2-frame chunks (one eviction-free fill), every output against the oracle."""
    from gpu_util import dev, host, check_attention
    H, D, T_f, sink, window, n_q = 16, 64, 1024, 2, 8, 2085
    rng = np.random.default_rng(77)
    cache = ops.KVCache(H, D, T_f, sink, window, **fmt)
    model = CacheModel(H, D, T_f, sink, window, **fmt)
    for _ in range(5):
        k, v = rand_bits(rng, (H, 2 * T_f, D)), rand_bits(rng, (H, 2 * T_f, D))
        cache.append(dev(k), dev(v), 2)
        model.append(k, v)
    assert model.n_tokens() == (sink + window) * T_f
    q, ko, vo = (rand_bits(rng, (H, n_q, D)) for _ in range(3))
    out = host(cache.attention(dev(q), dev(ko), dev(vo), 0.125))
    ck, cv = model.dequantized_kv()
    want = chunk_attention_ref(q, ko, vo, ck, cv, 0.125)
    check_attention(out, want, f"D64 at scale {fmt}")
    cache.close()


def test_attention_deterministic(ops):
    from gpu_util import dev, host
    rng = np.random.default_rng(6)
    H, D, T_f = 2, 128, 48
    chunks = [(rand_bits(rng, (H, 3 * T_f, D)), rand_bits(rng, (H, 3 * T_f, D)))]
    cache, _ = build_both(ops, H, D, T_f, 1, 2, chunks)
    q, ko, vo = (dev(rand_bits(rng, (H, 200, D))) for _ in range(3))
    a = host(cache.attention(q, ko, vo, 0.1))
    b = host(cache.attention(q, ko, vo, 0.1))
    assert np.array_equal(a, b)


def _rollout_checks():
    """(chunk, step) pairs checked in the streaming rollout: an empty cache, sinks
    only, the first full window (all four denoising steps), the first eviction,
    mid-run and the end; one seeded step elsewhere."""
    wl = W.WORKLOADS["rollout"]
    rng = np.random.default_rng(5)
    checks = []
    for c in (0, 1, 4, 5, 17, wl.n_chunks - 1):
        if c == 4:
            checks += [(c, s) for s in range(wl.steps_per_chunk)]
        else:
            checks.append((c, int(rng.integers(wl.steps_per_chunk))))
    return checks


ROLLOUT_CHECKS = _rollout_checks()


@pytest.fixture(scope="module")
def rollout_run(ops):
    """Streaming rollout workload: 40 chunks appended to a 3 sink + 9 window cache of
    1560-token frames, GPU cache and oracle cache model in lockstep.  At each checked
    (chunk, step) the GPU output over the current cache is kept with a snapshot of
    the oracle's attended frames; the first and last chunks' resident codes are
    exported."""
    import copy
    from gpu_util import dev, host
    wl = W.WORKLOADS["rollout"]
    cache, model = build_both(ops, wl.n_heads, wl.head_dim, wl.tokens_per_frame, wl.sink_frames,
                              wl.window_frames, [])
    results, exports, kept = {}, {}, {}
    for c in range(wl.n_chunks):
        for cc, step in ROLLOUT_CHECKS:
            if cc != c:
                continue
            q, ko, vo = W.noisy_chunk(wl, c, step=step)
            print(f"[rollout] chunk {c} step {step} cache_tokens={model.n_tokens()}", flush=True)
            out = host(cache.attention(dev(q), dev(ko), dev(vo), wl.softmax_scale))
            snap = copy.copy(model)
            snap.sinks, snap.pinned, snap.window = list(model.sinks), list(model.pinned), list(model.window)
            results[(c, step)] = (out, snap)
        k, v = W.clean_chunk(wl, c)
        cache.append(dev(k), dev(v), wl.chunk_frames)
        model.append(k, v)
        if c in (0, wl.n_chunks - 1):
            kept[c] = (k, v)
    assert cache.tokens() == (wl.sink_frames * wl.tokens_per_frame,
                              wl.window_frames * wl.tokens_per_frame)
    for c in kept:
        exports[c] = tuple(host(t) for t in cache.export_chunk(c))
    cache.close()
    return results, exports, kept


@pytest.mark.parametrize("check", ROLLOUT_CHECKS, ids=[f"chunk{c}-step{s}" for c, s in ROLLOUT_CHECKS])
def test_streaming_rollout(rollout_run, check):
    """Every output of every head at each checked point of the rollout against the
    oracle over the same cache state."""
    from gpu_util import check_attention
    wl = W.WORKLOADS["rollout"]
    results, _, _ = rollout_run
    c, step = check
    out, snap = results[check]
    q, ko, vo = W.noisy_chunk(wl, c, step=step)
    ck, cv = snap.dequantized_kv()
    want = chunk_attention_ref(q, ko, vo, ck, cv, wl.softmax_scale)
    check_attention(out, want, f"rollout chunk {c} step {step} cache_tokens={snap.n_tokens()}")


def test_streaming_rollout_resident_codes(rollout_run):
    """The first chunk (held as the sink through all 40 appends) and the last chunk
    are resident at the end: their codes, scale bytes and tensor scales equal the
    oracle codec of the same tensors byte for byte."""
    from oracle import quantize_ref
    _, exports, kept = rollout_run
    for c, (k, v) in kept.items():
        kc, ks, vc, vs, sk, sv = exports[c]
        for got, want, what in (((kc, ks, sk[0]), quantize_ref(k), "K"),
                                ((vc, vs, sv[0]), quantize_ref(v), "V")):
            assert np.array_equal(got[0], want[0]), f"chunk {c} {what} codes"
            assert np.array_equal(got[1], want[1]), f"chunk {c} {what} scales"
            assert np.float32(got[2]) == want[2], f"chunk {c} {what} tensor scale"


@pytest.mark.parametrize("D", [64, 128])
def test_cut_blocks_wait_fallback(ops, D):
    """Small problems spread one query block over many workgroups (one key tile
    each).  The workgroup holding a block's last tiles merges the partial results
    the workgroups holding its earlier tiles publish; with a zero wait limit it stops
    waiting for a missing partial at once and processes the block's earlier tiles
    itself.  Both paths must match the oracle."""
    rng = np.random.default_rng(40 + D)
    H, T_f, sink, window, n_q = 2, 40, 2, 5, 300
    chunks = [(rand_bits(rng, (H, nf * T_f, D)), rand_bits(rng, (H, nf * T_f, D))) for nf in (2, 3, 2, 1)]
    cache, model = build_both(ops, H, D, T_f, sink, window, chunks)
    q, ko, vo = (rand_bits(rng, (H, n_q, D)) for _ in range(3))
    try:
        for limit in (0, 1 << 16, 0):
            ops.set_wait_limit(limit)
            run_case(ops, cache, model, q, ko, vo, 1.0 / np.sqrt(D), what=f"D{D} wait limit {limit}")
    finally:
        ops.set_wait_limit(1 << 16)


@pytest.mark.parametrize("D", [64, 128])
def test_multi_shot_sink(ops, D):
    """Global sink + shot-level sink + window (paper text, section 4.2): scene cuts
    re-bind the shot-level sink, whose frames stay attended after the window rolls
    past them; attention after every append matches the oracle's cache model, and a
    pinned chunk's codes are still byte-exact."""
    from gpu_util import dev, host
    from oracle import quantize_ref
    rng = np.random.default_rng(60 + D)
    H, T_f, sink, window, shot = 2, 24, 1, 3, 2
    cache = ops.KVCache(H, D, T_f, sink, window, shot_frames=shot)
    model = CacheModel(H, D, T_f, sink, window, shot_frames=shot)
    schedule = [1, 2, "cut", 1, 2, 2, "cut", 1, 1, 3, 2]
    chunks = []
    for i, op in enumerate(schedule):
        if op == "cut":
            cache.begin_shot()
            model.begin_shot()
            continue
        k, v = rand_bits(rng, (H, op * T_f, D)), rand_bits(rng, (H, op * T_f, D))
        chunks.append((k, v))
        cache.append(dev(k), dev(v), op)
        model.append(k, v)
        st, n, extra = cache.shot_sink()
        assert (st, n, extra) == (model.shot_start, min(shot, model.n_frames - model.shot_start),
                                  len(model.pinned) * T_f)
        s_tok, w_tok = cache.tokens()
        assert s_tok + w_tok + extra == model.n_tokens()
        q, ko, vo = (rand_bits(rng, (H, 70, D)) for _ in range(3))
        run_case(ops, cache, model, q, ko, vo, 1.0 / np.sqrt(D),
                 what=f"D{D} step {i} frames {model.n_frames} pinned {len(model.pinned)}")
    # chunk 6 (frame 9, the second frame after the second cut) is held only as the
    # shot-level sink: the window rolled past it two appends ago
    idx = 6
    assert [f.index for f in model.pinned] == [8, 9] and model.window[0].index > 9
    kc, ks, vc, vs, sk, sv = cache.export_chunk(idx)
    k, v = chunks[idx]
    for got, want, what in (((host(kc), host(ks), host(sk)[0]), quantize_ref(k), "K"),
                            ((host(vc), host(vs), host(sv)[0]), quantize_ref(v), "V")):
        gc, gs, gt = got
        wc, ws_, wt = want
        assert np.array_equal(gc, wc) and np.array_equal(gs, ws_) and np.float32(gt) == wt, what


@pytest.mark.parametrize("D", [64, 128])
def test_k_smoothing_and_adaptive_v_attention(ops, D):
    """Attention over a cache built with K-smoothing (the chunk's channel means added
    back as a per-chunk logit term q . mean) and adaptive V scales matches the
    oracle's cache model, over several chunks with different means and a wrapped
    window."""
    from gpu_util import dev
    rng = np.random.default_rng(70 + D)
    H, T_f, sink, window = 2, 40, 1, 4
    cache = ops.KVCache(H, D, T_f, sink, window, k_smooth=True, v_adaptive=True)
    model = CacheModel(H, D, T_f, sink, window, k_smooth=True, v_adaptive=True)
    for nf in (2, 1, 2, 2):
        T = nf * T_f
        kx = (rng.standard_normal((H, T, D)) + rng.standard_normal((H, 1, D)) * 3).astype(np.float32)
        k, v = W.f32_to_bf16_bits(kx), rand_bits(rng, (H, T, D))
        cache.append(dev(k), dev(v), nf)
        model.append(k, v)
        q, ko, vo = (rand_bits(rng, (H, 100, D)) for _ in range(3))
        run_case(ops, cache, model, q, ko, vo, 1.0 / np.sqrt(D), what=f"smooth D{D} tokens {model.n_tokens()}")


def test_own_values_beyond_fp16_range(ops):
    """The chunk's own K/V enter the bf16 matrix cores as given: values far beyond
    fp16's range (|v| up to ~1e6) and tiny ones.  The bar is scaled by the size of V
    (max-abs 1e-2 relative to max |V|, relative L2 5e-3)."""
    from gpu_util import dev, host
    rng = np.random.default_rng(71)
    H, D, T_f = 2, 128, 64
    k1, v1 = rand_bits(rng, (H, 2 * T_f, D)), rand_bits(rng, (H, 2 * T_f, D))
    cache, model = build_both(ops, H, D, T_f, 1, 3, [(k1, v1)])
    q, ko = rand_bits(rng, (H, 150, D)), rand_bits(rng, (H, 150, D))
    vf = rng.standard_normal((H, 150, D)).astype(np.float32)
    vf[0] *= 1e6
    vf[1, :, :64] *= 1e-20
    vo = W.f32_to_bf16_bits(vf)
    scale = 1.0 / np.sqrt(D)
    out = host(cache.attention(dev(q), dev(ko), dev(vo), scale))
    ck, cv = model.dequantized_kv()
    want = chunk_attention_ref(q, ko, vo, ck, cv, scale)
    for h in range(H):
        vmax = max(np.abs(cv[h]).max(), np.abs((vo[h].astype(np.uint32) << 16).view(np.float32)).max())
        err = np.abs(out[h] - want[h]).max()
        rel = np.linalg.norm(out[h] - want[h]) / np.linalg.norm(want[h])
        print(f"[own beyond fp16, head {h}] max_abs/max|V| = {err / vmax:.3e} rel_l2 = {rel:.3e}", flush=True)
        assert np.all(np.isfinite(out[h]))
        assert err <= 1e-2 * vmax and rel <= 5e-3


@pytest.mark.parametrize("fmt", [dict(), dict(mxfp4=True)])
def test_largest_frame_count(ops, fmt):
    """The largest cache the configuration accepts: 4 sink + 60 window frames (64
    frames, 65,536 tokens of 1024-token frames), filled by single-frame appends and
    rolled past once; attention over all of it (every output), and the last chunk's
    codes bit-exact."""
    from gpu_util import dev, host, check_attention
    from oracle import quantize_ref, mx_quantize_ref
    rng = np.random.default_rng(81)
    H, D, T_f, sink, window = 2, 128, 1024, 4, 60
    cache = ops.KVCache(H, D, T_f, sink, window, **fmt)
    model = CacheModel(H, D, T_f, sink, window, **fmt)
    for c in range(sink + window + 3):
        k, v = rand_bits(rng, (H, T_f, D)), rand_bits(rng, (H, T_f, D))
        cache.append(dev(k), dev(v), 1)
        model.append(k, v)
    assert model.n_tokens() == (sink + window) * T_f
    kc, ks, vc, vs, _, _ = (host(t) for t in cache.export_chunk(sink + window + 2))
    qz = mx_quantize_ref if fmt else (lambda x: quantize_ref(x)[:2])
    assert all(np.array_equal(a, b) for a, b in zip((kc, ks, vc, vs), (*qz(k), *qz(v))))
    n_q = 700
    q, ko, vo = (rand_bits(rng, (H, n_q, D)) for _ in range(3))
    out = host(cache.attention(dev(q), dev(ko), dev(vo), 1.0 / np.sqrt(D)))
    ck, cv = model.dequantized_kv()
    want = chunk_attention_ref(q, ko, vo, ck, cv, 1.0 / np.sqrt(D))
    check_attention(out, want, f"64 frames x 1024 tokens {fmt}")
