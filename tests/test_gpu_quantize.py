"""GPU parity of the NVFP4 codec and of the cache append path: codes, scale bytes
and fp32 tensor scales must equal the oracle's bit for bit."""

import json
import os

import numpy as np
import pytest

from oracle import quantize_ref
from nvfp4_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_hand_example.json")


@pytest.fixture(scope="module")
def ops(gpu):
    from nvfp4_kv_cache_amd import ops as _ops
    return _ops


@pytest.fixture(scope="module")
def ws(ops):
    return ops.quantize_workspace()


def codec_gpu(ops, ws, bits):
    from gpu_util import dev, host
    c, s, t = ops.quantize_kv(dev(bits), ws)
    return host(c), host(s), host(t)[0]


def assert_codec_equal(got, want, what):
    from gpu_util import f32_bits
    gc, gs, gt = got
    wc, ws_, wt = want
    print(f"[{what}] s_t gpu={gt!r} oracle={wt!r}", flush=True)
    assert f32_bits(gt) == f32_bits(wt), what
    assert np.array_equal(gs, ws_), f"{what}: {np.count_nonzero(gs != ws_)} scale bytes differ"
    assert np.array_equal(gc, wc), f"{what}: {np.count_nonzero(gc != wc)} code bytes differ"


def t4_bits(rng, shape, scale=1.0):
    return W.f32_to_bf16_bits((rng.standard_t(4, size=shape) * scale).astype(np.float32))


def test_codec_golden(ops, ws):
    for case in json.load(open(GOLDEN))["cases"]:
        vals = [[-0.0 if v == "-0" else float(v) for v in row] for row in case["x"]]
        bits = W.f32_to_bf16_bits(np.array(vals, dtype=np.float32)).reshape(case["shape"])
        got = codec_gpu(ops, ws, bits)
        assert_codec_equal(got, quantize_ref(bits), case["name"])


@pytest.mark.parametrize("shape,scale", [((3, 50, 64), 1.0), ((2, 37, 128), 3.0), ((1, 1, 32), 1.0),
                                         ((4, 1000, 16), 1.0), ((1, 3, 48), 2.0),
                                         ((5, 129, 96), 1e-3), ((2, 300, 256), 1e4)])
def test_codec_random(ops, ws, shape, scale):
    rng = np.random.default_rng(hash(shape) % 1000)
    bits = t4_bits(rng, shape, scale)
    assert_codec_equal(codec_gpu(ops, ws, bits), quantize_ref(bits), f"t4 {shape} x{scale}")


@pytest.mark.parametrize("e", [-68, -70, -72, -75, -80, -85, -90, -95])
def test_small_tensor_scales(ops, ws, e):
    """Tensors whose s_t falls between 2^-102 and 2^-78: around the range limit
    below which the encoder moves x and eff by a power of two so that every element
    quotient and its remainder stay normal fp32 numbers.  Codec and cache append
    (both tensors of one append at different scales) against the oracle."""
    from gpu_util import dev, host
    rng = np.random.default_rng(500 - e)
    a = t4_bits(rng, (3, 120, 128), 2.0 ** e)
    b = t4_bits(rng, (3, 120, 128), 2.0 ** (e - 3))
    assert_codec_equal(codec_gpu(ops, ws, a), quantize_ref(a), f"codec 2^{e}")
    cache = ops.KVCache(3, 128, 40, 1, 3)
    cache.append(dev(a), dev(b), 3)
    kc, ks, vc, vs, sk, sv = cache.export_chunk(0)
    assert_codec_equal((host(kc), host(ks), host(sk)[0]), quantize_ref(a), f"append 2^{e} K")
    assert_codec_equal((host(vc), host(vs), host(sv)[0]), quantize_ref(b), f"append 2^{e} V")
    cache.close()


def test_codec_special_values(ops, ws):
    """Zeros of both signs, bf16 subnormals, values on E2M1 thresholds after
    scaling, and a block far below the tensor amax (subnormal E4M3 scales)."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 64, 64)).astype(np.float32)
    x[0, 0, :16] = 0.0
    x[0, 1, :16] = -0.0
    x[0, 2, :] *= 1e-6
    x[0, 3, :] = np.float32(2.0 ** -130) * rng.integers(-50, 50, 64)   # bf16 subnormals
    x[1, 5, 0] = 4096.0                                                  # tensor amax
    x[1, 6, :16] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 6] * 2) * 1.5
    bits = W.f32_to_bf16_bits(x)
    assert_codec_equal(codec_gpu(ops, ws, bits), quantize_ref(bits), "special")
    zero = np.zeros((1, 8, 32), dtype=np.uint16)
    zero[0, ::2] = 0x8000
    assert_codec_equal(codec_gpu(ops, ws, zero), quantize_ref(zero), "all zero")
    tiny = np.full((1, 16, 32), 0x0001, dtype=np.uint16)                 # smallest subnormal
    assert_codec_equal(codec_gpu(ops, ws, tiny), quantize_ref(tiny), "min subnormal")


def test_codec_workspace_reuse_is_deterministic(ops, ws):
    rng = np.random.default_rng(2)
    bits = t4_bits(rng, (4, 500, 128))
    first = codec_gpu(ops, ws, bits)
    for _ in range(3):
        again = codec_gpu(ops, ws, bits)
        assert_codec_equal(again, first, "repeat")


@pytest.mark.parametrize("name", ["tiny", "quantize"])
def test_codec_workload_tensors(ops, ws, name):
    wl = W.WORKLOADS[name]
    k, v = W.clean_chunk(wl, 0)
    for bits, what in ((k, "K"), (v, "V")):
        assert_codec_equal(codec_gpu(ops, ws, bits), quantize_ref(bits), f"{name} {what}")


def test_append_quantize_workload_steady_state(ops):
    """Quantize-only workload: K, V [12, 4680, 128] appended as one 3-frame chunk
    into a full 3 sink + 9 window cache; exported codes must equal the oracle's
    codec of the same tensors, and the sink chunk must be untouched."""
    from gpu_util import dev, host
    wl = W.WORKLOADS["quantize"]
    cache = ops.KVCache(wl.n_heads, wl.head_dim, wl.tokens_per_frame, wl.sink_frames,
                        wl.window_frames)
    chunks = [W.clean_chunk(wl, c) for c in range(5)]
    for c, (k, v) in enumerate(chunks):
        cache.append(dev(k), dev(v), wl.chunk_frames)
    assert cache.tokens() == (3 * 1560, 9 * 1560)
    # the headline append path: one single-pass kernel (456 workgroups resident at once)
    assert cache.append_schedule(wl.chunk_frames) == 1
    for c in (0, 4):
        kc, ks, vc, vs, sk, sv = cache.export_chunk(c)
        k, v = chunks[c]
        assert_codec_equal((host(kc), host(ks), host(sk)[0]), quantize_ref(k), f"chunk {c} K")
        assert_codec_equal((host(vc), host(vs), host(sv)[0]), quantize_ref(v), f"chunk {c} V")
    with pytest.raises(ops.NVFP4KVError):
        cache.export_chunk(1)          # evicted by chunk 4


@pytest.mark.parametrize("D", [64, 128])
def test_append_extreme_and_special_chunks(ops, D):
    """Appends whose tensors have extreme, zero or special-valued contents, one after
    another into one cache (each append computes its own s_t), with a frame length
    that leaves a ragged quantizer tile; every resident chunk's codes, scale bytes
    and tensor scales must equal the oracle's codec of the appended tensors."""
    from gpu_util import dev, host
    H, T_f, nf = 3, 40, 2
    T = nf * T_f
    rng = np.random.default_rng(7 + D)
    cache = ops.KVCache(H, D, T_f, 2, 8)

    def special():
        x = rng.standard_normal((H, T, D)).astype(np.float32)
        x[0, 0, :16] = 0.0
        x[0, 1, :16] = -0.0
        x[1, 2, :] *= 1e-6
        x[1, 3, :] = np.float32(2.0 ** -130) * rng.integers(-50, 50, D)
        x[2, 5, 0] = 4096.0
        return W.f32_to_bf16_bits(x)

    zero = np.zeros((H, T, D), dtype=np.uint16)
    zero[:, ::3] = 0x8000
    chunks = [
        (t4_bits(rng, (H, T, D), 1e-30), t4_bits(rng, (H, T, D), 1e30)),
        (special(), t4_bits(rng, (H, T, D), 1e-3)),
        (zero, special()),
        (np.full((H, T, D), 0x0001, dtype=np.uint16), t4_bits(rng, (H, T, D), 1e4)),
        (t4_bits(rng, (H, T, D)), zero),
    ]
    for k, v in chunks:
        cache.append(dev(k), dev(v), nf)
    for c, (k, v) in enumerate(chunks):
        kc, ks, vc, vs, sk, sv = cache.export_chunk(c)
        assert_codec_equal((host(kc), host(ks), host(sk)[0]), quantize_ref(k), f"D{D} chunk {c} K")
        assert_codec_equal((host(vc), host(vs), host(sv)[0]), quantize_ref(v), f"D{D} chunk {c} V")


@pytest.mark.parametrize("k_smooth", [False, True])
def test_append_adaptive_v_extreme_and_special_chunks(ops, k_smooth):
    """Adaptive-V appends (with and without K-smoothing, i.e. both encodes of the
    single-pass kernel) of V tensors at extreme scales (s_t below 2^-80 and above
    2^100, where the encoder rescales x and eff), a subnormal-only tensor, zeros of
    both signs and special values, with a ragged quantizer tile: V's codes, scale
    bytes and tensor scales equal the oracle's adaptive codec bit for bit."""
    from gpu_util import dev, host
    from oracle import channel_mean_ref
    H, D, T_f, nf = 3, 128, 40, 2
    T = nf * T_f
    rng = np.random.default_rng(31 + k_smooth)
    cache = ops.KVCache(H, D, T_f, 2, 8, k_smooth=k_smooth, v_adaptive=True)
    assert cache.append_schedule(nf) == 4

    def special():
        x = rng.standard_normal((H, T, D)).astype(np.float32)
        x[0, 0, :16] = 0.0
        x[0, 1, :16] = -0.0
        x[1, 2, :] *= 1e-6
        x[1, 3, :] = np.float32(2.0 ** -130) * rng.integers(-50, 50, D)
        x[2, 5, 0] = 4096.0
        return W.f32_to_bf16_bits(x)

    zero = np.zeros((H, T, D), dtype=np.uint16)
    zero[:, ::3] = 0x8000
    vs = [t4_bits(rng, (H, T, D), 1e-30), t4_bits(rng, (H, T, D), 1e33), special(),
          np.full((H, T, D), 0x0001, dtype=np.uint16), zero]
    chunks = [(t4_bits(rng, (H, T, D)), v) for v in vs]
    for k, v in chunks:
        cache.append(dev(k), dev(v), nf)
    for c, (k, v) in enumerate(chunks):
        kc, ks, vc, vs_, sk, sv = cache.export_chunk(c)
        wk = quantize_ref(k, mean=channel_mean_ref(k)) if k_smooth else quantize_ref(k)
        assert_codec_equal((host(kc), host(ks), host(sk)[0]), wk, f"ks={k_smooth} chunk {c} K")
        assert_codec_equal((host(vc), host(vs_), host(sv)[0]), quantize_ref(v, adaptive=True),
                           f"ks={k_smooth} chunk {c} V")
    cache.close()


@pytest.mark.parametrize("k_smooth,v_adaptive", [(False, False), (True, False), (False, True), (True, True)])
def test_append_two_pass_large_chunk(ops, k_smooth, v_adaptive):
    """A chunk whose tiles cannot all be resident at once (16 heads x 8192 tokens,
    1024 workgroups) takes the two-pass quantizer (kvcache_append_schedule 2): the
    channel means (K-smoothing), the amax pass and the encode pass with each option
    combination, V written transposed into the cache; codes, scale bytes and tensor
    scales equal the oracle's bit for bit."""
    from gpu_util import dev, host
    from oracle import channel_mean_ref
    H, D, T_f, nf = 16, 128, 2048, 4
    rng = np.random.default_rng(140 + 2 * k_smooth + v_adaptive)
    cache = ops.KVCache(H, D, T_f, 1, 4, k_smooth=k_smooth, v_adaptive=v_adaptive)
    assert cache.append_schedule(nf) == 2
    kx = rng.standard_t(4, size=(H, nf * T_f, D)) * 1.5
    if k_smooth:
        kx = kx + rng.standard_normal((H, 1, D)) * 6
    k = W.f32_to_bf16_bits(kx.astype(np.float32))
    v = t4_bits(rng, (H, nf * T_f, D), 2.0)
    cache.append(dev(k), dev(v), nf)
    kc, ks, vc, vs, sk, sv = cache.export_chunk(0)
    wk = quantize_ref(k, mean=channel_mean_ref(k)) if k_smooth else quantize_ref(k)
    assert_codec_equal((host(kc), host(ks), host(sk)[0]), wk, f"two-pass ks={k_smooth} va={v_adaptive} K")
    assert_codec_equal((host(vc), host(vs), host(sv)[0]), quantize_ref(v, adaptive=v_adaptive),
                       f"two-pass ks={k_smooth} va={v_adaptive} V")
    cache.close()


def test_append_wait_fallback_help(ops):
    """With a zero poll limit, every workgroup of the single-pass append quantizer that
    does not find all maxima published on its first look helps: it computes missing
    workgroups' tile maxima and publishes them in their place; with limits 1 and 2 it
    first waits a little.  Codes, scale bytes and tensor scales must not change, for a
    small grid and for the quantize workload's 456 workgroups."""
    from gpu_util import dev, host
    rng = np.random.default_rng(11)
    cases = []
    H, D, T_f = 4, 128, 256         # 16 workgroups per append
    cases.append((H, D, T_f, 2, [(t4_bits(rng, (H, 2 * T_f, D), s), t4_bits(rng, (H, 2 * T_f, D), 1.0 / s))
                                 for s in (1.0, 1e-20, 3e5)]))
    wl = W.WORKLOADS["quantize"]
    cases.append((wl.n_heads, wl.head_dim, wl.tokens_per_frame, wl.chunk_frames,
                  [W.clean_chunk(wl, c) for c in range(2)]))
    for H, D, T_f, nf, chunks in cases:
        results = []
        for limit in (0, 1, 2, 1 << 16):
            print(f"[append help] H={H} T_f={T_f} wait limit {limit}", flush=True)
            ops.set_wait_limit(limit)
            try:
                cache = ops.KVCache(H, D, T_f, 2, 4 * nf)
                assert cache.append_schedule(nf) == 1
                for k, v in chunks:
                    cache.append(dev(k), dev(v), nf)
                results.append([tuple(host(t) for t in cache.export_chunk(c)) for c in range(len(chunks))])
            finally:
                ops.set_wait_limit(1 << 16)
        for c, (k, v) in enumerate(chunks):
            wk, wv = quantize_ref(k), quantize_ref(v)
            for r in results:
                kc, ks, vc, vs, sk, sv = r[c]
                assert_codec_equal((kc, ks, sk[0]), wk, f"chunk {c} K")
                assert_codec_equal((vc, vs, sv[0]), wv, f"chunk {c} V")
    with pytest.raises(ops.NVFP4KVError):
        ops.set_wait_limit(-1)


@pytest.mark.parametrize("D,T_f,frames", [(128, 40, [2, 1, 3]), (64, 8, [1, 2, 4]), (128, 1560, [3]),
                                          (64, 64, [4, 1]), (128, 3000, [3]), (64, 5800, [3])])
def test_append_k_smoothing_and_adaptive_v(ops, D, T_f, frames):
    """Cache appends with K-smoothing and adaptive 4/6 V scales: the channel means
    (pairwise fp32 tree; token counts 8 to 17400, padded to powers of two: up to 64
    aligned tile nodes per head, i.e. two batches at the top of the tree), K codes of
    x - mean, V codes with the chosen block scales, and both tensor scales equal the
    oracle's bit for bit.  K has per-channel offsets, a constant channel and a -0
    channel; V has heavy tails so that both scale candidates occur.  These appends
    take the single pass with the options (schedule 4)."""
    from gpu_util import dev, host
    from oracle import channel_mean_ref
    rng = np.random.default_rng(D + T_f)
    H = 3
    cache = ops.KVCache(H, D, T_f, 1, 6, k_smooth=True, v_adaptive=True)
    chunks = []
    for nf in frames:
        assert cache.append_schedule(nf) == 4
        T = nf * T_f
        kx = (rng.standard_normal((H, T, D)) + rng.standard_normal((H, 1, D)) * 8).astype(np.float32)
        kx[0, :, 3] = 1.5
        kx[1, :, 5] = -0.0
        k = W.f32_to_bf16_bits(kx)
        v = t4_bits(rng, (H, T, D), 2.0)
        cache.append(dev(k), dev(v), nf)
        chunks.append((k, v))
    for c, (k, v) in enumerate(chunks):
        mu_want = channel_mean_ref(k)
        mu = host(cache.export_k_mean(c))
        assert np.array_equal(mu.view(np.uint32), mu_want.view(np.uint32)), f"chunk {c} means"
        kc, ks, vc, vs, sk, sv = cache.export_chunk(c)
        assert_codec_equal((host(kc), host(ks), host(sk)[0]), quantize_ref(k, mean=mu_want), f"chunk {c} K")
        want_v = quantize_ref(v, adaptive=True)
        plain_v = quantize_ref(v)
        print(f"chunk {c}: {np.count_nonzero(want_v[1] != plain_v[1])} of {want_v[1].size} V blocks take the 4-scale",
              flush=True)
        assert_codec_equal((host(vc), host(vs), host(sv)[0]), want_v, f"chunk {c} V")


@pytest.mark.parametrize("D,T_f,frames", [(128, 1560, [3]), (64, 40, [2, 1]), (128, 8, [4, 2])])
def test_append_adaptive_v_only(ops, D, T_f, frames):
    """Adaptive 4/6 V scales without K-smoothing: K codes by the plain recipe, V with
    the per-block choice; codes, scale bytes and tensor scales equal the oracle's bit
    for bit."""
    from gpu_util import dev, host
    rng = np.random.default_rng(3 * D + T_f)
    H = 3
    cache = ops.KVCache(H, D, T_f, 1, 6, v_adaptive=True)
    chunks = []
    for nf in frames:
        assert cache.append_schedule(nf) == 4
        k = t4_bits(rng, (H, nf * T_f, D), 1.5)
        v = t4_bits(rng, (H, nf * T_f, D), 2.0)
        cache.append(dev(k), dev(v), nf)
        chunks.append((k, v))
    for c, (k, v) in enumerate(chunks):
        kc, ks, vc, vs, sk, sv = cache.export_chunk(c)
        assert_codec_equal((host(kc), host(ks), host(sk)[0]), quantize_ref(k), f"chunk {c} K")
        want_v = quantize_ref(v, adaptive=True)
        print(f"chunk {c}: {np.count_nonzero(want_v[1] != quantize_ref(v)[1])} V blocks take the 4-scale", flush=True)
        assert_codec_equal((host(vc), host(vs), host(sv)[0]), want_v, f"chunk {c} V")
    cache.close()


def test_append_k_smoothing_extreme_scales(ops):
    """K-smoothing and adaptive V appends of chunks at extreme scales (1e-20, 3e5,
    with per-channel offsets in K), with poll limits 0 (help at once) and 65536:
    codes, scale bytes and tensor scales equal the oracle's."""
    from gpu_util import dev, host
    from oracle import channel_mean_ref
    H, D, T_f = 3, 128, 256
    rng = np.random.default_rng(12)
    chunks = []
    for s in (1.0, 1e-20, 3e5):
        kx = (rng.standard_normal((H, 2 * T_f, D)) + rng.standard_normal((H, 1, D)) * 8) * s
        chunks.append((W.f32_to_bf16_bits(kx.astype(np.float32)), t4_bits(rng, (H, 2 * T_f, D), 1.0 / s)))
    results = []
    for limit in (0, 1 << 16):
        ops.set_wait_limit(limit)
        try:
            cache = ops.KVCache(H, D, T_f, 2, 4, k_smooth=True, v_adaptive=True)
            for k, v in chunks:
                cache.append(dev(k), dev(v), 2)
            results.append([tuple(host(t) for t in cache.export_chunk(c)) for c in range(3)])
        finally:
            ops.set_wait_limit(1 << 16)
    for c, (k, v) in enumerate(chunks):
        wk = quantize_ref(k, mean=channel_mean_ref(k))
        wv = quantize_ref(v, adaptive=True)
        for r in results:
            kc, ks, vc, vs, sk, sv = r[c]
            assert_codec_equal((kc, ks, sk[0]), wk, f"chunk {c} K")
            assert_codec_equal((vc, vs, sv[0]), wv, f"chunk {c} V")


@pytest.mark.parametrize("k_smooth,v_adaptive", [(True, True), (True, False), (False, True)])
def test_append_options_wait_fallback_help(ops, k_smooth, v_adaptive):
    """The single pass with the cache options under poll limits 0, 1, 2 and 65536:
    with a small limit its workgroups help instead of waiting, computing missing
    tiles' maxima, K channel sums, or max |K - mean| (after the means of that tile's
    head) in their owners' place.  Means, codes, scale bytes and tensor scales must
    not change, for a small grid and for the quantize workload's 456 workgroups."""
    from gpu_util import dev, host
    from oracle import channel_mean_ref
    rng = np.random.default_rng(17)
    H, D, T_f = 4, 128, 256         # 2 tiles per head: 8 K and 8 V workgroups
    small = []
    for s in (1.0, 1e-20, 3e5):
        kx = (rng.standard_normal((H, 2 * T_f, D)) + rng.standard_normal((H, 1, D)) * 8) * s
        small.append((W.f32_to_bf16_bits(kx.astype(np.float32)), t4_bits(rng, (H, 2 * T_f, D), 1.0 / s)))
    wl = W.WORKLOADS["quantize"]
    cases = [(H, D, T_f, 2, small),
             (wl.n_heads, wl.head_dim, wl.tokens_per_frame, wl.chunk_frames,
              [W.clean_chunk(wl, c) for c in range(2)])]
    for H, D, T_f, nf, chunks in cases:
        results = []
        for limit in (0, 1, 2, 1 << 16):
            print(f"[options help] ks={k_smooth} va={v_adaptive} H={H} T_f={T_f} wait limit {limit}", flush=True)
            ops.set_wait_limit(limit)
            try:
                cache = ops.KVCache(H, D, T_f, 2, 4 * nf, k_smooth=k_smooth, v_adaptive=v_adaptive)
                assert cache.append_schedule(nf) == 4
                for k, v in chunks:
                    cache.append(dev(k), dev(v), nf)
                r = []
                for c in range(len(chunks)):
                    mu = host(cache.export_k_mean(c)) if k_smooth else None
                    r.append((tuple(host(t) for t in cache.export_chunk(c)), mu))
                results.append(r)
                cache.close()
            finally:
                ops.set_wait_limit(1 << 16)
        for c, (k, v) in enumerate(chunks):
            mu_want = channel_mean_ref(k) if k_smooth else None
            wk = quantize_ref(k, mean=mu_want)
            wv = quantize_ref(v, adaptive=v_adaptive)
            for r in results:
                (kc, ks, vc, vs, sk, sv), mu = r[c]
                if k_smooth:
                    assert np.array_equal(mu.view(np.uint32), mu_want.view(np.uint32)), f"chunk {c} means"
                assert_codec_equal((kc, ks, sk[0]), wk, f"chunk {c} K")
                assert_codec_equal((vc, vs, sv[0]), wv, f"chunk {c} V")
