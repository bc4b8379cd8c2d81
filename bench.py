#!/usr/bin/env python3
"""Benchmark of the NVFP4 KV-cache chunk-attention hot path on one MI355X.

One step = one chunk of the streaming rollout (12 heads, head_dim 128, 1560
tokens per latent frame, 3-frame chunks, cache of 3 sink + 9 window frames):
four chunk-attention calls of the noisy chunk over the NVFP4 cache plus its
own bf16 K/V (4 denoising steps), then quantize + append of the clean chunk.
`--warmup W` chunks run first (W >= 4 fills the cache, so every timed step
sees the steady-state 18720 cache tokens); `--steps K` chunks are timed.
Inputs are resident on the device before timing starts.

Prints progress on stderr and ONE JSON line on stdout:
  value          chunk-attention TFLOP/s over the timed rollout steps (the time
                 includes the appends);  latent_frames_per_s alongside
  roofline       the attention kernel alone: FLOPs per launch / mean launch time
                 (HIP events on the launch stream) vs the 2516.6 TFLOP/s bf16
                 dense MFMA peak
  quantize       the append (quantize + pack) kernel on the quantize-only
                 workload, cache-cold inputs: algorithmic GB/s vs 8 TB/s HBM
  configs        the other workloads (tiny, 1.3B-shaped, 5B-shaped), and the append and
                 the 1.3B-shaped attention with K-smoothing + adaptive V scales
  rollout_full_loop  the whole 40-chunk streaming rollout from an empty cache
                 (ramp included): latent frames/s = 120 / loop time
  cpu_baseline   the CPU oracle on a bounded sample of every workload
"""

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6     # MI355X dense bf16 (fp16 is the same)
CSRC = os.path.join(ROOT, "nvfp4_kv_cache_amd", "csrc")
# kernel sources whose digest a PMC summary in profiles/ records; a summary taken
# on other sources no longer describes the kernel, and its traffic is not reported
TRAFFIC_SOURCES = {
    "attention": ("attention.hip", "attn_plan.h", "device_common.h", "nvfp4kv_internal.h"),
    "quantize": ("quantize.hip", "device_common.h", "nvfp4kv_internal.h"),
    "quantize_mx": ("quantize.hip", "device_common.h", "nvfp4kv_internal.h"),
}
TRAFFIC_PROFILES = {
    "attention": "chunk_attention_kernel_rollout_steady_pmc.md",
    "quantize": "quantize_append_quantize_workload_pmc.md",
    "quantize_mx": "quantize_mx_append_quantize_workload_pmc.md",
}
HBM_PEAK_GBPS = 8000.0             # MI355X HBM3E
METRIC = "NVFP4-KV chunk attention TFLOP/s + latent frames/s; KV-quantize GB/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=36)
    p.add_argument("--warmup", type=int, default=4)
    p.add_argument("--reps", type=int, default=100, help="launches per attention microbenchmark")
    p.add_argument("--quantize-reps", type=int, default=1000, help="appends timed by the quantize leg")
    p.add_argument("--warm-launches", type=int, default=30,
                   help="untimed attention launches enqueued right before the timed ones")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--skip-configs", action="store_true", help="rollout + roofline legs only")
    p.add_argument("--only", choices=["attention", "quantize", "copy", "stream"],
                   help="run one kernel leg only (for profiler runs): the attention kernel on the "
                        "steady-state rollout cache (the roofline leg), the append of the "
                        "quantize-only workload, or a plain 256 MiB device copy (reference for "
                        "the HBM byte counters), or the same-size streaming reference of the append")
    p.add_argument("--mxfp4", action="store_true",
                   help="with --only attention / quantize: the cache holds MXFP4 instead of NVFP4")
    p.add_argument("--mx-scaled-qk", action="store_true",
                   help="with --only attention --mxfp4: QK^T on the MX-scaled matrix cores (MXFP8 queries)")
    p.add_argument("--k-smooth", action="store_true",
                   help="with --only quantize: the cache applies K-smoothing")
    p.add_argument("--v-adaptive", action="store_true",
                   help="with --only quantize: the cache applies adaptive 4/6 V block scales")
    return p.parse_args()


def source_digest(leg):
    import hashlib
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES[leg]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(leg):
    """HBM bytes per launch from the committed PMC summary of this leg
    (FETCH_SIZE and WRITE_SIZE, each scaled by what it reads for a plain copy),
    or None when the summary is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", TRAFFIC_PROFILES[leg])
    fields = {}
    try:
        for ln in open(path):
            cells = [c.strip() for c in ln.strip().strip("|").split("|")]
            if len(cells) == 2:
                fields[cells[0]] = cells[1]
        if fields.get("sources_sha256") != source_digest(leg):
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def timed(fn, reps, torch, warm=3, host_us_per_call=None, dist=None):
    """Mean ms per call of fn() over `reps` back-to-back calls, HIP events on
    the current stream (the stream the library launches on).  `warm` untimed
    calls are enqueued right before the timed ones, so the GPU is at its working
    clock when timing starts.  For calls shorter than the host's enqueue time,
    `host_us_per_call` queues a device-side sleep first, long enough for the host
    to enqueue every timed call before the first one starts: the events then time
    back-to-back GPU execution, not the Python call rate.  With a dict `dist`, an
    event also separates every two calls, and the median, p10 and p90 of the
    per-call times (µs) are stored in it."""
    def run(per_call):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1 if per_call else 2)]
        fn()
        torch.cuda.synchronize()
        for _ in range(warm):
            fn()
        if host_us_per_call:
            torch.cuda._sleep(int(2.0e3 * host_us_per_call * reps) + 1_000_000)   # ~cycles at >= 2 GHz
        ev[0].record()
        for i in range(reps):
            fn()
            if per_call:
                ev[i + 1].record()
        if not per_call:
            ev[1].record()
        torch.cuda.synchronize()
        return ev

    ev = run(False)
    mean_ms = ev[0].elapsed_time(ev[1]) / reps
    if dist is not None:
        # a second pass with an event between every two calls (each event adds a little
        # to the call it follows, so the mean above is taken without them)
        import numpy as np
        ev = run(True)
        t = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps)])
        dist.update({"median_us": float(np.median(t)), "p10_us": float(np.percentile(t, 10)),
                     "p90_us": float(np.percentile(t, 90)), "reps": reps,
                     "note": "per-call times from a second pass with an event between calls"})
    return mean_ms


def dev_bits(torch, bits, device):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)


def rollout(args, torch, ops, W, device):
    wl = W.WORKLOADS["rollout"]
    n_chunks = args.warmup + args.steps
    S = wl.steps_per_chunk
    log(f"rollout: drawing {n_chunks} chunks x ({S} noisy steps + clean append) on device")
    inputs = []
    for c in range(n_chunks):
        noisy = [tuple(W.draw_device_normal(wl, c, s, t, device) for t in (W.Q_ID, W.K_ID, W.V_ID))
                 for s in range(S)]
        clean = tuple(W.draw_device_normal(wl, c, W.APPEND_STEP, t, device) for t in (W.K_ID, W.V_ID))
        inputs.append((noisy, clean))
    cache = ops.KVCache(wl.n_heads, wl.head_dim, wl.tokens_per_frame, wl.sink_frames,
                        wl.window_frames, device=device)
    out = torch.empty((wl.n_heads, wl.n_q, wl.head_dim), dtype=torch.float32, device=device)
    scale = wl.softmax_scale

    def step(c):
        noisy, (kc, vc) = inputs[c]
        for q, k, v in noisy:
            cache.attention(q, k, v, scale, out=out)
        cache.append(kc, vc, wl.chunk_frames)

    for c in range(args.warmup):
        step(c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for c in range(args.warmup, n_chunks):
        step(c)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1)
    n_k = wl.cache_frames_for_chunk(args.warmup) * wl.tokens_per_frame + wl.n_q
    steady = wl.cache_frames_for_chunk(args.warmup) == wl.sink_frames + wl.window_frames
    flops_step = S * W.attention_flops(wl.n_heads, wl.n_q, n_k, wl.head_dim)
    res = {
        "ms_per_step": ms / args.steps,
        "wall_ms_per_step": 1e3 * wall / args.steps,
        "tflops": flops_step * args.steps / (ms * 1e-3) / 1e12,
        "frames_per_s": wl.chunk_frames * args.steps / (ms * 1e-3),
        "cache_tokens": n_k - wl.n_q,
        "steady_state": steady,
    }
    q, k, v = inputs[-1][0][0]
    res.update(attention_roofline(args, torch, ops, W, cache, (q, k, v), out))
    return res


def rollout_full_loop(torch, ops, W, device):
    """The whole streaming rollout as the workload defines it: 40 chunks from an
    empty cache (the ramp through 0, 3, 6, 9 cached frames included), each 4
    attention calls then the clean chunk's append.  One untimed pass on a fresh
    cache brings the GPU to its working clock; a second pass on another fresh cache
    is timed with HIP events: latent frames/s = 120 / loop time."""
    wl = W.WORKLOADS["rollout"]
    S = wl.steps_per_chunk
    log(f"rollout (full loop): drawing {wl.n_chunks} chunks on device")
    inputs = []
    for c in range(wl.n_chunks):
        noisy = [tuple(W.draw_device_normal(wl, c, s, t, device) for t in (W.Q_ID, W.K_ID, W.V_ID))
                 for s in range(S)]
        clean = tuple(W.draw_device_normal(wl, c, W.APPEND_STEP, t, device) for t in (W.K_ID, W.V_ID))
        inputs.append((noisy, clean))
    out = torch.empty((wl.n_heads, wl.n_q, wl.head_dim), dtype=torch.float32, device=device)

    def loop(cache):
        for noisy, (kc, vc) in inputs:
            for q, k, v in noisy:
                cache.attention(q, k, v, wl.softmax_scale, out=out)
            cache.append(kc, vc, wl.chunk_frames)

    caches = [ops.KVCache(wl.n_heads, wl.head_dim, wl.tokens_per_frame, wl.sink_frames, wl.window_frames,
                          device=device) for _ in range(2)]
    loop(caches[0])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    loop(caches[1])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    flops = sum(S * W.attention_flops(wl.n_heads, wl.n_q, wl.cache_frames_for_chunk(c) * wl.tokens_per_frame
                                      + wl.n_q, wl.head_dim) for c in range(wl.n_chunks))
    elems = wl.n_heads * wl.chunk_tokens * wl.head_dim
    nbytes = wl.n_chunks * 2 * W.quantize_bytes(elems)
    ideal_s = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) + nbytes / (HBM_PEAK_GBPS * 1e9)
    frames = wl.n_chunks * wl.chunk_frames
    for c in caches:
        c.close()
    return {"chunks": wl.n_chunks, "attention_calls": wl.n_chunks * S, "appends": wl.n_chunks,
            "loop_ms": ms, "latent_frames_per_s": frames / (ms * 1e-3),
            "ideal_latent_frames_per_s": frames / ideal_s, "frac_of_ideal": ideal_s / (ms * 1e-3),
            "attention_flops": flops, "append_bytes": nbytes,
            "note": "ideal = attention FLOPs at the dense bf16/fp16 MFMA peak + append bytes at the HBM peak"}


def attention_roofline(args, torch, ops, W, cache, qkv, out):
    """The attention kernel alone on the steady-state rollout cache: mean launch
    time over `reps` back-to-back launches (HIP events on the launch stream)."""
    wl = W.WORKLOADS["rollout"]
    q, k, v = qkv
    dist = {}
    ams = timed(lambda: cache.attention(q, k, v, wl.softmax_scale, out=out), args.reps, torch,
                warm=args.warm_launches, dist=dist)
    flops = W.attention_flops(wl.n_heads, wl.n_q, cache.tokens()[0] + cache.tokens()[1] + wl.n_q,
                              wl.head_dim)
    return {"attn_ms": ams, "attn_flops": flops, "attn_tflops": flops / (ams * 1e-3) / 1e12, "attn_dist": dist}


def roofline_only(args, torch, ops, W, device):
    """--only attention: the same measurement as the roofline leg of a full run,
    with the steady-state cache filled by appends alone, so that a profiler run
    of this command sees only the timed attention launches."""
    wl = W.WORKLOADS["rollout"]
    cache = ops.KVCache(wl.n_heads, wl.head_dim, wl.tokens_per_frame, wl.sink_frames,
                        wl.window_frames, device=device, mxfp4=args.mxfp4,
                        mx_scaled_qk=args.mxfp4 and args.mx_scaled_qk)
    n_fill = (wl.sink_frames + wl.window_frames + wl.chunk_frames - 1) // wl.chunk_frames
    for c in range(n_fill):
        kc, vc = (W.draw_device_normal(wl, c, W.APPEND_STEP, t, device) for t in (W.K_ID, W.V_ID))
        cache.append(kc, vc, wl.chunk_frames)
    qkv = tuple(W.draw_device_normal(wl, n_fill, 0, t, device) for t in (W.Q_ID, W.K_ID, W.V_ID))
    out = torch.empty((wl.n_heads, wl.n_q, wl.head_dim), dtype=torch.float32, device=device)
    r = attention_roofline(args, torch, ops, W, cache, qkv, out)
    return {"launch_us": r["attn_ms"] * 1e3, "flops_per_launch": r["attn_flops"],
            "tflops": r["attn_tflops"], "frac_mfma_peak": r["attn_tflops"] / MFMA_BF16_PEAK_TFLOPS,
            "cache_tokens": sum(cache.tokens()), "per_launch": r["attn_dist"]}


def quantize_leg(args, torch, ops, W, device, k_smooth=False, v_adaptive=False, sets=None, mxfp4=False):
    """Append of one 3-frame chunk of K and V [12, 4680, 128] into a full cache,
    cycling 10 distinct input sets (287.5 MB > the 256 MB Infinity Cache).  With
    k_smooth / v_adaptive the cache applies K-smoothing / adaptive V scales; with
    mxfp4 it holds MXFP4 (single-pass quantizer)."""
    wl = W.WORKLOADS["quantize"]
    n_sets = 10
    if sets is None:
        log(f"quantize: drawing {n_sets} Student-t input sets on the host")
        sets = [tuple(dev_bits(torch, b, device) for b in W.clean_chunk(wl, c)) for c in range(n_sets)]
    cache = ops.KVCache(wl.n_heads, wl.head_dim, wl.tokens_per_frame, wl.sink_frames,
                        wl.window_frames, device=device, k_smooth=k_smooth, v_adaptive=v_adaptive,
                        mxfp4=mxfp4)
    for c in range(4):
        cache.append(*sets[c], wl.chunk_frames)
    it = [0]

    def app():
        k, v = sets[it[0] % n_sets]
        it[0] += 1
        cache.append(k, v, wl.chunk_frames)

    reps = max(args.quantize_reps, 1)
    dist = {}
    ms = timed(app, reps, torch, warm=10, host_us_per_call=60.0, dist=dist)
    elems = wl.n_heads * wl.chunk_tokens * wl.head_dim
    nbytes = 2 * (W.quantize_bytes_mx(elems) if mxfp4 else W.quantize_bytes(elems))
    gbps = nbytes / (ms * 1e-3) / 1e9
    out = {"us_per_append": ms * 1e3, "bytes_per_append": nbytes, "GB_per_s": gbps, "per_append": dist,
           "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": gbps / HBM_PEAK_GBPS,
                        "traffic": None if (k_smooth or v_adaptive) else
                                   measured_traffic("quantize_mx" if mxfp4 else "quantize")}}
    return out, sets


def stream_leg(args, torch, ops, W, device, sets):
    """The same-size streaming reference: the bytes of one K+V append of the quantize
    workload (2 B read, 1/2 + 1/16 B written per element) moved with the quantizer's
    tiling and no exchange between workgroups, cycling the same 10 cache-cold input
    sets: the time this transfer size allows."""
    wl = W.WORKLOADS["quantize"]
    H, T, D = wl.n_heads, wl.chunk_tokens, wl.head_dim
    out = [torch.empty(s, dtype=torch.uint8, device=device)
           for s in ((H, T, D // 2), (H, T, D // 16), (H, T, D // 2), (H, T, D // 16))]
    it = [0]

    def run():
        k, v = sets[it[0] % len(sets)]
        it[0] += 1
        ops.stream_reference(k, v, out)

    reps = max(args.quantize_reps, 1)
    dist = {}
    ms = timed(run, reps, torch, warm=10, host_us_per_call=60.0, dist=dist)
    nbytes = 2 * W.quantize_bytes(H * T * D)
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"us_per_call": ms * 1e3, "bytes_per_call": nbytes, "GB_per_s": gbps, "frac_hbm_peak": gbps / HBM_PEAK_GBPS,
            "per_call": dist}


def attention_config(name, args, torch, ops, W, device, k_smooth=False, v_adaptive=False, mxfp4=False,
                     mx_scaled_qk=False):
    wl = W.WORKLOADS[name]
    log(f"{name}: building the cache from {wl.n_cache_chunks} host-drawn chunks")
    cache = ops.KVCache(wl.n_heads, wl.head_dim, wl.tokens_per_frame, wl.sink_frames,
                        wl.window_frames, device=device, k_smooth=k_smooth, v_adaptive=v_adaptive,
                        mxfp4=mxfp4, mx_scaled_qk=mx_scaled_qk)
    for c in range(wl.n_cache_chunks):
        k, v = W.clean_chunk(wl, c)
        cache.append(dev_bits(torch, k, device), dev_bits(torch, v, device), wl.chunk_frames)
    q, ko, vo = (dev_bits(torch, b, device) for b in W.noisy_chunk(wl, wl.n_cache_chunks))
    out = torch.empty((wl.n_heads, wl.n_q, wl.head_dim), dtype=torch.float32, device=device)
    reps = args.reps if name != "tiny" else 200
    ms = timed(lambda: cache.attention(q, ko, vo, wl.softmax_scale, out=out), reps, torch,
               warm=args.warm_launches if name != "tiny" else 20,
               host_us_per_call=60.0 if name == "tiny" else None)
    s, w = cache.tokens()
    flops = W.attention_flops(wl.n_heads, wl.n_q, s + w + wl.n_q, wl.head_dim)
    tf = flops / (ms * 1e-3) / 1e12
    return {"us": ms * 1e3, "cache_tokens": s + w, "n_q": wl.n_q, "tflops": tf,
            "frac_mfma_peak": tf / MFMA_BF16_PEAK_TFLOPS}


def _median_time(fn, reps):
    import numpy as np
    t = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        t.append(time.perf_counter() - t0)
    return float(np.median(t))


def cpu_baseline(args, W):
    """The oracle, untuned, timed on the host on a bounded sample of every workload:
    tiny and quantize-only x10 (median), one full chunk-attention call of the 1.3B- and
    5B-shaped workloads, and one steady-state chunk of the streaming rollout (one of
    its 4 attention calls and its append) extrapolated to the 40-chunk loop.  Inputs
    are drawn and the oracle caches built before each timed call.  The headline value
    is the 1.3B-shaped call (the steady-state rollout step's attention shape)."""
    from oracle import CacheModel, chunk_attention_ref, quantize_ref

    def cache_of(wl, n_chunks, draw):
        model = CacheModel(wl.n_heads, wl.head_dim, wl.tokens_per_frame, wl.sink_frames, wl.window_frames)
        for c in range(n_chunks):
            model.append(*draw(c))
        return model.dequantized_kv()

    per = {}
    # tiny: quantize the 4-frame chunk (K and V) + attention, x10
    wl = W.WORKLOADS["tiny"]
    k, v = W.clean_chunk(wl, 0)
    q, ko, vo = W.noisy_chunk(wl, 1)

    def tiny():
        model = CacheModel(wl.n_heads, wl.head_dim, wl.tokens_per_frame, wl.sink_frames, wl.window_frames)
        model.append(k, v)
        ck, cv = model.dequantized_kv()
        chunk_attention_ref(q, ko, vo, ck, cv, wl.softmax_scale)
    t = _median_time(tiny, 10)
    f = W.attention_flops(wl.n_heads, wl.n_q, 256 + wl.n_q, wl.head_dim)
    per["tiny"] = {"seconds_median": t, "reps": 10, "GFLOP_per_s": f / t / 1e9,
                   "what": "quantize K and V of the cache chunk, dequantize, attention"}
    # quantize-only: K and V [12, 4680, 128], x10
    wl = W.WORKLOADS["quantize"]
    k, v = W.clean_chunk(wl, 0)
    t = _median_time(lambda: (quantize_ref(k), quantize_ref(v)), 10)
    nbytes = 2 * W.quantize_bytes(k.size)
    per["quantize"] = {"seconds_median": t, "reps": 10, "GB_per_s": nbytes / t / 1e9,
                       "what": "oracle codec of K and V"}
    # 1.3B- and 5B-shaped: one full call each
    for name in ("wan13b", "wan5b"):
        wl = W.WORKLOADS[name]
        ck, cv = cache_of(wl, wl.n_cache_chunks, lambda c, wl=wl: W.clean_chunk(wl, c))
        q, ko, vo = W.noisy_chunk(wl, wl.n_cache_chunks)
        t0 = time.perf_counter()
        chunk_attention_ref(q, ko, vo, ck, cv, wl.softmax_scale)
        t = time.perf_counter() - t0
        f = W.attention_flops(wl.n_heads, wl.n_q, ck.shape[1] + wl.n_q, wl.head_dim)
        per[name] = {"seconds": t, "reps": 1, "TFLOP_per_s": f / t / 1e12, "flops": f}
    # streaming rollout: one steady-state chunk (cache of chunks 0..3 = 3 sink + 9 window
    # frames), one attention call and the append timed, extrapolated to the 40 chunks
    wl = W.WORKLOADS["rollout"]
    rng_draw = lambda c: tuple(W.draw_bf16(wl, c, W.APPEND_STEP, t) for t in (W.K_ID, W.V_ID))
    ck, cv = cache_of(wl, 4, rng_draw)
    q, ko, vo = W.noisy_chunk(wl, 4, step=0)
    t0 = time.perf_counter()
    chunk_attention_ref(q, ko, vo, ck, cv, wl.softmax_scale)
    t_attn = time.perf_counter() - t0
    k, v = rng_draw(4)
    t0 = time.perf_counter()
    quantize_ref(k), quantize_ref(v)
    t_app = time.perf_counter() - t0
    n_full = ck.shape[1] + wl.n_q
    # attention time scales with the key count of each chunk (0, 3, 6, 9, 12, 12, ... frames)
    t_loop = sum(wl.steps_per_chunk * t_attn * (wl.cache_frames_for_chunk(c) * wl.tokens_per_frame + wl.n_q)
                 / n_full + t_app for c in range(wl.n_chunks))
    per["rollout"] = {"seconds_attention_call": t_attn, "seconds_append": t_app,
                      "extrapolated_loop_seconds": t_loop,
                      "latent_frames_per_s": wl.n_chunks * wl.chunk_frames / t_loop,
                      "what": f"1 steady-state attention call + 1 append timed, extrapolated to "
                              f"{wl.n_chunks} chunks x ({wl.steps_per_chunk} calls scaled by key count + 1 append)"}
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    cpu_model = ""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                cpu_model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    h = per["wan13b"]
    return {"value": h["TFLOP_per_s"], "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 oracle: one 1.3B-shaped chunk-attention call (12 heads x 4680 queries x 23400 "
                      f"keys x D128) for the value; per_config: tiny and quantize-only x10 (median), one "
                      f"5B-shaped call, one steady-state rollout chunk extrapolated; numpy BLAS threads={cores}; "
                      f"{cpu_model}",
            "seconds": h["seconds"], "host_cpus": os.cpu_count(), "per_config": per}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this path is single-GPU)", file=sys.stderr)
        sys.exit(2)
    if args.warmup < 4:
        log("note: warmup < 4 chunks, so the timed steps do not all see the full cache")
    import torch
    from nvfp4_kv_cache_amd import ops, workloads as W
    assert torch.cuda.is_available(), "needs a GPU"
    device = torch.device("cuda:0")
    ops.lib()
    log(f"device: {torch.cuda.get_device_name(0)}")
    if args.only == "attention":
        r = roofline_only(args, torch, ops, W, device)
        print(json.dumps({"leg": "attention", "workload": "rollout steady state", "mxfp4": args.mxfp4, **r}),
              flush=True)
        return
    if args.only == "copy":
        src = torch.ones(64 << 20, dtype=torch.float32, device=device)   # 256 MiB
        dst = torch.empty_like(src)
        ms = timed(lambda: dst.copy_(src), 5, torch, warm=2)
        print(json.dumps({"leg": "copy", "bytes_read": src.numel() * 4, "bytes_written": dst.numel() * 4,
                          "ms": ms, "GB_per_s": 2 * src.numel() * 4 / (ms * 1e-3) / 1e9}), flush=True)
        return
    if args.only == "stream":
        wl = W.WORKLOADS["quantize"]
        sets = [tuple(dev_bits(torch, b, device) for b in W.clean_chunk(wl, c)) for c in range(10)]
        r = stream_leg(args, torch, ops, W, device, sets)
        print(json.dumps({"leg": "stream", "workload": "quantize", **r}), flush=True)
        return
    if args.only == "quantize":
        qz, _ = quantize_leg(args, torch, ops, W, device, mxfp4=args.mxfp4, k_smooth=args.k_smooth,
                             v_adaptive=args.v_adaptive)
        print(json.dumps({"leg": "quantize", "workload": "quantize", "mxfp4": args.mxfp4,
                          "k_smooth": args.k_smooth, "v_adaptive": args.v_adaptive, **qz}), flush=True)
        return

    r = rollout(args, torch, ops, W, device)
    log(f"rollout: {r['ms_per_step']:.3f} ms/step, {r['tflops']:.1f} TFLOP/s, "
        f"{r['frames_per_s']:.1f} frames/s; attention kernel {r['attn_ms']*1e3:.1f} us "
        f"= {r['attn_tflops']:.1f} TFLOP/s")
    full = None
    if not args.skip_configs:
        full = rollout_full_loop(torch, ops, W, device)
        log(f"rollout, full 40-chunk loop: {full['loop_ms']:.1f} ms = {full['latent_frames_per_s']:.1f} frames/s "
            f"({100 * full['frac_of_ideal']:.1f}% of the {full['ideal_latent_frames_per_s']:.0f} frames/s ideal)")
    qz, qsets = quantize_leg(args, torch, ops, W, device)
    log(f"quantize: {qz['us_per_append']:.2f} us/append = {qz['GB_per_s']:.1f} GB/s")
    configs = {}
    if not args.skip_configs:
        for name in ("tiny", "wan13b", "wan5b"):
            configs[name] = attention_config(name, args, torch, ops, W, device)
            log(f"{name}: {configs[name]['us']:.1f} us, {configs[name]['tflops']:.1f} TFLOP/s")
        # the cache options (K-smoothing for K, adaptive 4/6 scales for V)
        qo, _ = quantize_leg(args, torch, ops, W, device, k_smooth=True, v_adaptive=True, sets=qsets)
        configs["quantize_k_smooth_v_adaptive"] = {k: qo[k] for k in ("us_per_append", "GB_per_s")}
        log(f"quantize, K-smoothing + adaptive V: {qo['us_per_append']:.2f} us/append")
        qa, _ = quantize_leg(args, torch, ops, W, device, v_adaptive=True, sets=qsets)
        configs["quantize_v_adaptive"] = {k: qa[k] for k in ("us_per_append", "GB_per_s")}
        log(f"quantize, adaptive V: {qa['us_per_append']:.2f} us/append")
        configs["wan13b_k_smooth_v_adaptive"] = attention_config("wan13b", args, torch, ops, W, device,
                                                                 k_smooth=True, v_adaptive=True)
        log(f"wan13b, K-smoothing + adaptive V: {configs['wan13b_k_smooth_v_adaptive']['us']:.1f} us")
        # the MXFP4 cache variant (32-element blocks, E8M0 scales, no tensor scale)
        qm, _ = quantize_leg(args, torch, ops, W, device, mxfp4=True, sets=qsets)
        configs["quantize_mxfp4"] = {k: qm[k] for k in ("us_per_append", "GB_per_s", "bytes_per_append")}
        configs["quantize_mxfp4"]["frac_hbm_peak"] = qm["roofline"]["frac"]
        configs["quantize_mxfp4"]["traffic"] = qm["roofline"]["traffic"]
        log(f"quantize, MXFP4: {qm['us_per_append']:.2f} us/append = {qm['GB_per_s']:.1f} GB/s")
        configs["wan13b_mxfp4"] = attention_config("wan13b", args, torch, ops, W, device, mxfp4=True)
        log(f"wan13b, MXFP4 cache: {configs['wan13b_mxfp4']['us']:.1f} us")
        configs["wan13b_mxfp4_scaled_qk"] = attention_config("wan13b", args, torch, ops, W, device, mxfp4=True,
                                                             mx_scaled_qk=True)
        log(f"wan13b, MXFP4 cache, MX-scaled QK^T with MXFP8 queries: "
            f"{configs['wan13b_mxfp4_scaled_qk']['us']:.1f} us")
    sr = stream_leg(args, torch, ops, W, device, qsets)
    configs["quantize_stream_reference"] = sr
    log(f"stream reference (same bytes, no exchange): {sr['us_per_call']:.2f} us = {sr['GB_per_s']:.1f} GB/s")
    configs["quantize"] = {k: qz[k] for k in ("us_per_append", "GB_per_s", "bytes_per_append")}
    configs["quantize"]["frac_hbm_peak"] = qz["roofline"]["frac"]

    wl = W.WORKLOADS["rollout"]
    result = {
        "metric": METRIC,
        "value": r["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16/bf16 MFMA, fp32 accumulate",
        "data": "synthetic",
        "config": {
            "workload": "streaming rollout, steady state: 12 heads, head_dim 128, 1560 tokens/frame, "
                        "3-frame chunks (4680 queries) over an NVFP4 cache of 3 sink + 9 window frames "
                        "(18720 tokens) + 4680 own bf16 tokens; 4 attention calls + 1 append per step",
            "n_heads": wl.n_heads, "head_dim": wl.head_dim, "tokens_per_frame": wl.tokens_per_frame,
            "chunk_frames": wl.chunk_frames, "sink_frames": wl.sink_frames,
            "window_frames": wl.window_frames, "attention_calls_per_step": wl.steps_per_chunk,
            "cache_tokens": r["cache_tokens"], "steady_state": r["steady_state"],
        },
        "latent_frames_per_s": r["frames_per_s"],
        "rollout_full_loop": full,
        "wall_ms_per_step": r["wall_ms_per_step"],
        "roofline": {"bound": "mfma", "kernel": "chunk_attention_kernel<128, false, false> (NVFP4 cache)",
                     "achieved": r["attn_tflops"], "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": r["attn_tflops"] / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": measured_traffic("attention"),
                     "launch_us": r["attn_ms"] * 1e3, "flops_per_launch": r["attn_flops"],
                     "per_launch": r["attn_dist"]},
        "quantize": qz,
        "configs": configs,
        "cpu_baseline": None,
        "host": platform.node(),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: running the oracle on a bounded sample")
        cb = cpu_baseline(args, W)
        log(f"cpu baseline: {cb['value']*1e3:.2f} GFLOP/s in {cb['seconds']:.1f} s")
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
