"""GPU parity of the MXFP4 cache variant: the standalone codec and the cache append
must give the oracle's codes and E8M0 scale bytes bit for bit; attention over an
MXFP4 cache must match the oracle's float64 attention over its own MXFP4 cache
within max-abs 1e-2 and relative-L2 5e-3 (the same bar as NVFP4)."""

import json
import os

import numpy as np
import pytest

from oracle import CacheModel, chunk_attention_ref, mx_quantize_ref
from nvfp4_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_blocks.json")


@pytest.fixture(scope="module")
def ops(gpu):
    from nvfp4_kv_cache_amd import ops as _ops
    return _ops


def codec_gpu(ops, bits):
    from gpu_util import dev, host
    c, s = ops.mxfp4_quantize_kv(dev(bits))
    return host(c), host(s)


def assert_equal(got, want, what):
    gc, gs = got
    wc, ws = want
    print(f"[{what}] shape codes {gc.shape} scales {gs.shape}", flush=True)
    assert np.array_equal(gs, ws), f"{what}: {np.count_nonzero(gs != ws)} scale bytes differ"
    assert np.array_equal(gc, wc), f"{what}: {np.count_nonzero(gc != wc)} code bytes differ"


def test_mx_codec_golden(ops):
    g = json.load(open(GOLDEN))
    rows, D = g["shape"]
    x = np.zeros((1, rows, D), dtype=np.float32)
    for blk in g["blocks"]:
        vals = np.array(blk["x"], dtype=np.float32)
        x[0, blk["row"], 32 * blk["block"]:32 * blk["block"] + len(vals)] = vals
    bits = W.f32_to_bf16_bits(x)
    got = codec_gpu(ops, bits)
    assert_equal(got, mx_quantize_ref(bits), "golden")
    for blk in g["blocks"]:
        assert got[1][0, blk["row"], blk["block"]] == blk["scale_byte"], blk["name"]


@pytest.mark.parametrize("shape,scale", [((3, 50, 64), 1.0), ((2, 37, 128), 3.0), ((1, 1, 32), 1.0),
                                         ((4, 1000, 32), 1.0), ((1, 3, 96), 2.0),
                                         ((5, 129, 128), 1e-3), ((2, 300, 256), 1e4)])
def test_mx_codec_random(ops, shape, scale):
    rng = np.random.default_rng(sum(shape))
    bits = W.f32_to_bf16_bits((rng.standard_t(4, size=shape) * scale).astype(np.float32))
    assert_equal(codec_gpu(ops, bits), mx_quantize_ref(bits), f"t4 {shape} x{scale}")


def test_mx_codec_special_values(ops):
    """Zeros of both signs, bf16 subnormals, blocks whose exponent clamps at -127,
    the largest bf16 magnitudes, and elements on every E2M1 rounding midpoint."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 64, 128)).astype(np.float32)
    x[0, 0, :32] = 0.0
    x[0, 1, :32] = -0.0
    x[0, 2, :] = np.float32(2.0 ** -133) * rng.integers(-120, 120, 128)     # bf16 subnormals
    x[0, 3, :64] = np.float32(2.0 ** -126) * rng.integers(-3, 4, 64)
    x[0, 4, :] = np.float32(3.0e38) * np.sign(rng.standard_normal(128))
    x[1, 5, :32] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0] * 4) * np.float32(2.0 ** -3)
    x[1, 6, 32:64] = np.array([6.0, -0.25, 0.7, 5.5, 4.5, 3.0, 2.0, 1.0] * 4)
    bits = W.f32_to_bf16_bits(x)
    assert_equal(codec_gpu(ops, bits), mx_quantize_ref(bits), "special")


def rand_bits(rng, shape, outliers=True):
    x = rng.standard_normal(shape).astype(np.float32)
    if outliers:
        m = rng.random(shape) < 0.02
        x[m] = rng.standard_t(4, size=int(m.sum())).astype(np.float32)
    return W.f32_to_bf16_bits(x)


def build_both(ops, H, D, T_f, sink, window, chunks, shot=0):
    from gpu_util import dev
    cache = ops.KVCache(H, D, T_f, sink, window, shot_frames=shot, mxfp4=True)
    model = CacheModel(H, D, T_f, sink, window, shot_frames=shot, mxfp4=True)
    for k, v in chunks:
        cache.append(dev(k), dev(v), k.shape[1] // T_f)
        model.append(k, v)
    return cache, model


@pytest.mark.parametrize("D", [64, 128])
def test_mx_append_export_bit_exact(ops, D):
    """Chunks appended into MXFP4 cache slots (K in the codec layout, V transposed)
    come back, through the export hook, equal to the oracle's codec of each chunk."""
    from gpu_util import host
    rng = np.random.default_rng(20 + D)
    H, T_f = 3, 40
    from gpu_util import dev
    chunks = [(rand_bits(rng, (H, nf * T_f, D)), rand_bits(rng, (H, nf * T_f, D))) for nf in (2, 3, 1, 2, 3)]
    cache = ops.KVCache(H, D, T_f, 1, 6, mxfp4=True)
    for cid, (k, v) in enumerate(chunks):
        # exported right after its append (later appends evict the oldest frames, so
        # the window wraps and the chunk lands in recycled slots)
        cache.append(dev(k), dev(v), k.shape[1] // T_f)
        kc, ks, vc, vs, sk, sv = (host(t) for t in cache.export_chunk(cid))
        assert_equal((kc, ks), mx_quantize_ref(k), f"K chunk {cid} D{D}")
        assert_equal((vc, vs), mx_quantize_ref(v), f"V chunk {cid} D{D}")
        assert sk[0] == 1.0 and sv[0] == 1.0


def run_case(ops, cache, model, q, ko, vo, scale, rows=None, what=""):
    from gpu_util import dev, host, check_attention
    print(f"[{what}] n_q={q.shape[1]} cache_tokens={model.n_tokens()}", flush=True)
    out = host(cache.attention(dev(q), dev(ko), dev(vo), scale))
    ck, cv = model.dequantized_kv()
    want = chunk_attention_ref(q, ko, vo, ck, cv, scale, rows=rows)
    got = out if rows is None else out[:, rows]
    return check_attention(got, want, what)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("n_q", [1, 257])
def test_mx_attention_ragged_multi_segment(ops, D, n_q):
    rng = np.random.default_rng(30 + D + n_q)
    H, T_f, sink, window = 3, 40, 2, 5
    chunks = [(rand_bits(rng, (H, nf * T_f, D)), rand_bits(rng, (H, nf * T_f, D))) for nf in (3, 2, 1, 3, 2)]
    cache, model = build_both(ops, H, D, T_f, sink, window, chunks)
    q, ko, vo = (rand_bits(rng, (H, n_q, D)) for _ in range(3))
    run_case(ops, cache, model, q, ko, vo, 1.0 / np.sqrt(D), what=f"mx ragged D{D} nq{n_q}")


def test_mx_attention_wide_range_and_shot_sink(ops):
    """Chunks scaled by very different powers of two (the E8M0 scales of one tile
    span a wide range), an all-zero chunk, and a scene cut with a shot-level sink."""
    rng = np.random.default_rng(41)
    H, D, T_f = 2, 128, 64
    chunks = []
    for i, sc in enumerate((1.0, 2.0 ** -20, 0.0, 2.0 ** 6, 1.0, 3.0)):
        x = (rng.standard_normal((H, T_f, D)) * sc).astype(np.float32)
        x[:, :, :32] *= np.float32(2.0 ** -9)   # a block of each token far below the others
        chunks.append((W.f32_to_bf16_bits(x), rand_bits(rng, (H, T_f, D))))
    cache, model = build_both(ops, H, D, T_f, 1, 3, chunks[:3], shot=2)
    cache.begin_shot()
    model.begin_shot()
    for k, v in chunks[3:]:
        from gpu_util import dev
        cache.append(dev(k), dev(v), 1)
        model.append(k, v)
    q, ko, vo = (rand_bits(rng, (H, 130, D)) for _ in range(3))
    run_case(ops, cache, model, q, ko, vo, 0.0884, what="mx wide range + shot")


def test_mx_attention_wan13b_whole_output(ops):
    """The 1.3B-shaped workload (12 heads, 4680 queries over 18720 cached + 4680 own
    keys) with an MXFP4 cache, in the launch configuration the benchmark times;
    every output of every head against the oracle."""
    wl = W.WORKLOADS["wan13b"]
    from gpu_util import dev, host, check_attention
    cache = ops.KVCache(wl.n_heads, wl.head_dim, wl.tokens_per_frame, wl.sink_frames, wl.window_frames,
                        mxfp4=True)
    model = CacheModel(wl.n_heads, wl.head_dim, wl.tokens_per_frame, wl.sink_frames, wl.window_frames,
                       mxfp4=True)
    for c in range(wl.n_cache_chunks):
        k, v = W.clean_chunk(wl, c)
        cache.append(dev(k), dev(v), wl.chunk_frames)
        model.append(k, v)
    q, ko, vo = W.noisy_chunk(wl, wl.n_cache_chunks)
    print(f"[mx wan13b] cache_tokens={model.n_tokens()}", flush=True)
    out = host(cache.attention(dev(q), dev(ko), dev(vo), wl.softmax_scale))
    ck, cv = model.dequantized_kv()
    want = chunk_attention_ref(q, ko, vo, ck, cv, wl.softmax_scale)
    check_attention(out, want, "mx wan13b")


# ---- MX-scaled QK^T: the cache logits from MXFP8 queries on the MX-scaled matrix cores


def q_mxfp8(q_bits):
    from oracle import mxfp8_dequantize_ref, mxfp8_quantize_ref
    return mxfp8_dequantize_ref(*mxfp8_quantize_ref(q_bits))


def build_scaled(ops, H, D, T_f, sink, window, chunks, shot=0):
    from gpu_util import dev
    cache = ops.KVCache(H, D, T_f, sink, window, shot_frames=shot, mxfp4=True, mx_scaled_qk=True)
    model = CacheModel(H, D, T_f, sink, window, shot_frames=shot, mxfp4=True)
    for k, v in chunks:
        cache.append(dev(k), dev(v), k.shape[1] // T_f)
        model.append(k, v)
    return cache, model


def run_scaled(cache, model, q, ko, vo, scale, rows=None, what=""):
    from gpu_util import dev, host, check_attention
    print(f"[{what}] n_q={q.shape[1]} cache_tokens={model.n_tokens()}", flush=True)
    out = host(cache.attention(dev(q), dev(ko), dev(vo), scale))
    ck, cv = model.dequantized_kv()
    want = chunk_attention_ref(q, ko, vo, ck, cv, scale, rows=rows, q_cache64=q_mxfp8(q))
    got = out if rows is None else out[:, rows]
    return check_attention(got, want, what)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("n_q", [1, 257])
def test_mx_scaled_qk_ragged_multi_segment(ops, D, n_q):
    rng = np.random.default_rng(50 + D + n_q)
    H, T_f, sink, window = 3, 40, 2, 5
    chunks = [(rand_bits(rng, (H, nf * T_f, D)), rand_bits(rng, (H, nf * T_f, D))) for nf in (3, 2, 1, 3, 2)]
    cache, model = build_scaled(ops, H, D, T_f, sink, window, chunks)
    q, ko, vo = (rand_bits(rng, (H, n_q, D)) for _ in range(3))
    run_scaled(cache, model, q, ko, vo, 1.0 / np.sqrt(D), what=f"mx scaled-qk ragged D{D} nq{n_q}")


def test_mx_scaled_qk_special_queries_and_shot_sink(ops):
    """Queries with zero blocks, bf16 subnormals, large and tiny rows (MXFP8 exponent
    clamps and saturation at 448) over chunks of very different scales, across a
    scene cut."""
    from gpu_util import dev
    rng = np.random.default_rng(61)
    H, D, T_f = 2, 128, 64
    chunks = []
    for sc in (1.0, 2.0 ** -20, 0.0, 2.0 ** 6, 1.0):
        x = (rng.standard_normal((H, T_f, D)) * sc).astype(np.float32)
        chunks.append((W.f32_to_bf16_bits(x), rand_bits(rng, (H, T_f, D))))
    cache, model = build_scaled(ops, H, D, T_f, 1, 2, chunks[:3], shot=1)
    cache.begin_shot()
    model.begin_shot()
    for k, v in chunks[3:]:
        cache.append(dev(k), dev(v), 1)
        model.append(k, v)
    qf = rng.standard_normal((H, 100, D)).astype(np.float32)
    qf[0, 0, :32] = 0.0
    qf[0, 1, :] = np.float32(2.0 ** -130) * rng.integers(-100, 100, D)
    qf[0, 2, :] *= 30.0
    qf[1, 3, :] *= 1e-30
    qf[1, 4, :32] = np.array([448, 464, 480, 500, 1, -1, 0.5, 3] * 4, dtype=np.float32)
    q = W.f32_to_bf16_bits(qf)
    ko, vo = rand_bits(rng, (H, 100, D)), rand_bits(rng, (H, 100, D))
    run_scaled(cache, model, q, ko, vo, 0.0884, what="mx scaled-qk special queries + shot")


def test_mx_scaled_qk_wan13b_whole_output(ops):
    """The 1.3B-shaped workload with the MX-scaled QK^T: every output of every head."""
    wl = W.WORKLOADS["wan13b"]
    chunks = [W.clean_chunk(wl, c) for c in range(wl.n_cache_chunks)]
    cache, model = build_scaled(ops, wl.n_heads, wl.head_dim, wl.tokens_per_frame, wl.sink_frames,
                                wl.window_frames, chunks)
    q, ko, vo = W.noisy_chunk(wl, wl.n_cache_chunks)
    run_scaled(cache, model, q, ko, vo, wl.softmax_scale, what="mx scaled-qk wan13b")


def test_mx_scaled_qk_head_dim_64_at_scale(ops):
    """head_dim 64 with the MX-scaled QK^T at a size that cuts most query blocks
    between workgroups (16 heads, 2085 queries over a full 2 + 8-frame cache of
    1024-token frames): every output of every head."""
    rng = np.random.default_rng(78)
    H, D, T_f, sink, window = 16, 64, 1024, 2, 8
    chunks = [(rand_bits(rng, (H, 2 * T_f, D)), rand_bits(rng, (H, 2 * T_f, D))) for _ in range(5)]
    cache, model = build_scaled(ops, H, D, T_f, sink, window, chunks)
    assert model.n_tokens() == (sink + window) * T_f
    q, ko, vo = (rand_bits(rng, (H, 2085, D)) for _ in range(3))
    run_scaled(cache, model, q, ko, vo, 0.125, what="mx scaled-qk D64 at scale")
