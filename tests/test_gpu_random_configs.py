"""Seeded random cache configurations and schedules on the GPU, each checked against
the oracle: head count, head_dim, frame size, sink / window / shot-level-sink sizes,
the cache format and options (NVFP4 plain, K-smoothing, adaptive V, both, MXFP4, MXFP4
with the MX-scaled QK^T),
chunk sizes, evictions, scene cuts and query counts are drawn per seed.  Resident
chunks must export bit-exact codes and scales; attention must meet the tolerance."""

import numpy as np
import pytest

from oracle import (CacheModel, channel_mean_ref, chunk_attention_ref, mx_quantize_ref, mxfp8_dequantize_ref,
                    mxfp8_quantize_ref, quantize_ref)
from nvfp4_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

FORMATS = [dict(), dict(k_smooth=True), dict(v_adaptive=True), dict(k_smooth=True, v_adaptive=True),
           dict(mxfp4=True), dict(mxfp4=True, mx_scaled_qk=True)]


@pytest.fixture(scope="module")
def ops(gpu):
    from nvfp4_kv_cache_amd import ops as _ops
    return _ops


def draw_bits(rng, shape):
    kind = rng.integers(0, 3)
    if kind == 0:
        x = rng.standard_normal(shape)
    elif kind == 1:
        x = rng.standard_t(4, size=shape) * 10.0 ** rng.uniform(-1, 0.5)
    else:
        x = rng.standard_normal(shape) + rng.standard_normal(shape[-1]) * 3.0   # channel offsets
    return W.f32_to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("seed", range(24))
def test_random_config(ops, seed):
    from gpu_util import MAX_ABS, bf16_p_bar, check_attention, dev, host
    rng = np.random.default_rng(1000 + seed)
    H = int(rng.integers(1, 4))
    D = int(rng.choice([64, 128]))
    T_f = 8 * int(rng.integers(1, 9))
    sink, window = int(rng.integers(0, 3)), int(rng.integers(1, 5))
    shot = int(rng.integers(0, 3))
    fmt = FORMATS[seed % len(FORMATS)]
    print(f"[seed {seed}] H={H} D={D} T_f={T_f} sink={sink} window={window} shot={shot} {fmt}", flush=True)
    cache = ops.KVCache(H, D, T_f, sink, window, shot_frames=shot, **fmt)
    model = CacheModel(H, D, T_f, sink, window, shot_frames=shot,
                       **{k: v for k, v in fmt.items() if k != "mx_scaled_qk"})
    chunk = 0
    for step in range(int(rng.integers(3, 8))):
        if shot and rng.random() < 0.3:
            cache.begin_shot()
            model.begin_shot()
        if rng.random() < 0.2 and len(model.window) > 1:
            cache.evict(1)
            model.evict(1)
        nf = int(rng.integers(1, window + 1))
        k, v = draw_bits(rng, (H, nf * T_f, D)), draw_bits(rng, (H, nf * T_f, D))
        cache.append(dev(k), dev(v), nf)
        model.append(k, v)
        # the chunk just appended is resident: its codes must be the oracle's
        kc, ks, vc, vs, sk, sv = (host(t) for t in cache.export_chunk(chunk))
        if fmt.get("mxfp4"):
            wk, wv = mx_quantize_ref(k), mx_quantize_ref(v)
        else:
            mu = channel_mean_ref(k) if fmt.get("k_smooth") else None
            wk = quantize_ref(k, mean=mu)[:2]
            wv = quantize_ref(v, adaptive=fmt.get("v_adaptive", False))[:2]
        assert np.array_equal(kc, wk[0]) and np.array_equal(ks, wk[1]), f"seed {seed} chunk {chunk} K"
        assert np.array_equal(vc, wv[0]) and np.array_equal(vs, wv[1]), f"seed {seed} chunk {chunk} V"
        chunk += 1
        n_q = int(rng.integers(1, 300))
        q, ko, vo = (draw_bits(rng, (H, n_q, D)) for _ in range(3))
        scale = float(rng.uniform(0.02, 0.2))
        out = host(cache.attention(dev(q), dev(ko), dev(vo), scale))
        ck, cv = model.dequantized_kv()
        qc = mxfp8_dequantize_ref(*mxfp8_quantize_ref(q)) if fmt.get("mx_scaled_qk") else None
        want = chunk_attention_ref(q, ko, vo, ck, cv, scale, q_cache64=qc)
        # NVFP4 formats: the plain bar.  MXFP4 formats: the probabilities of their
        # tiles enter PV as bf16 (the converts' bf16 output sets the product's type), so
        # the max-abs bar is the larger of 1e-2 and 1.05x the error that rounding P to
        # bf16 alone produces on these inputs; rel-L2 keeps its bar either way
        bar = MAX_ABS
        if fmt.get("mxfp4"):
            bar = bf16_p_bar(q, ko, vo, ck, cv, scale, want, q_cache64=qc)
        check_attention(out, want, f"seed {seed} step {step} n_q={n_q} cache={model.n_tokens()}",
                        max_abs_bar=bar)
    cache.close()
