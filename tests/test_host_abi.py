"""CPU tests of the C ABI: every declared symbol is exported by the built
library; argument errors return status codes before any device work; and the
cache metadata (slot assignment, FIFO eviction, sink retention, segment lists)
matches the oracle's frame-list model, using a build of the host code whose
kernel launchers only record their arguments (tests/host_stub)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import CacheModel

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4kv.h")
LIB = os.path.join(ROOT, "nvfp4_kv_cache_amd", "libnvfp4kv.so")
STUB = os.path.join(ROOT, "nvfp4_kv_cache_amd", "libnvfp4kv_hoststub.so")
# NVFP4KV_STUB_SANITIZE=1: the stub build of the host code is instrumented with
# AddressSanitizer and UndefinedBehaviorSanitizer (the process must preload the ASan
# runtime; test_metadata_under_sanitizers below does this in a child process)
SANITIZE = os.environ.get("NVFP4KV_STUB_SANITIZE") == "1"
if SANITIZE:
    STUB = STUB.replace(".so", "_asan.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]

OK, EINVAL, ESHAPE, ECAPACITY, ESTATE, EHIP = 0, -1, -2, -3, -4, -5


class Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_heads", "head_dim", "tokens_per_frame", "sink_frames", "window_frames",
                 "shot_frames", "options")]


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    skip = {"if", "defined", "sizeof"}
    return sorted({n for n in names if n not in skip and not n.startswith("_")})


def test_header_declares_the_boundary():
    fns = declared_functions()
    for need in ["nvfp4_quantize_kv", "nvfp4_quantize_workspace_bytes", "kvcache_storage_bytes",
                 "kvcache_create", "kvcache_destroy", "kvcache_append", "kvcache_evict",
                 "kvcache_tokens", "chunk_attention", "kvcache_export_chunk", "nvfp4kv_strerror"]:
        assert need in fns


@pytest.fixture(scope="module")
def real():
    if not os.path.exists(LIB):
        pytest.fail("libnvfp4kv.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_library_exports_every_declared_symbol(real):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\s[TW]\s(\S+)$", out, flags=re.M))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing


def test_error_paths_before_device_work(real):
    P = ctypes.c_void_p
    real.nvfp4_quantize_kv.argtypes = [P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P, P, P, P,
                                       ctypes.c_size_t, P]
    dummy = P(0x10000)
    ws = real.nvfp4_quantize_workspace_bytes()
    assert real.nvfp4_quantize_kv(None, 1, 1, 64, dummy, dummy, dummy, dummy, ws, None) == EINVAL
    assert real.nvfp4_quantize_kv(dummy, 1, 1, 40, dummy, dummy, dummy, dummy, ws, None) == EINVAL
    assert real.nvfp4_quantize_kv(dummy, 0, 1, 64, dummy, dummy, dummy, dummy, ws, None) == EINVAL
    assert real.nvfp4_quantize_kv(dummy, 1, 1, 64, dummy, dummy, dummy, dummy, ws - 1, None) == ECAPACITY
    real.mxfp4_quantize_kv.argtypes = [P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P, P, P]
    assert real.mxfp4_quantize_kv(None, 1, 1, 64, dummy, dummy, None) == EINVAL
    assert real.mxfp4_quantize_kv(dummy, 1, 1, 48, dummy, dummy, None) == EINVAL   # D % 32 != 0
    assert real.mxfp4_quantize_kv(dummy, 1, 0, 64, dummy, dummy, None) == EINVAL
    assert real.mxfp4_quantize_kv(P(0x10008), 1, 1, 64, dummy, dummy, None) == EINVAL
    real.kvcache_storage_bytes.restype = ctypes.c_size_t
    real.kvcache_storage_bytes.argtypes = [ctypes.POINTER(Cfg)]
    for bad in [Cfg(1, 96, 64, 1, 3), Cfg(1, 128, 60, 1, 3), Cfg(0, 128, 64, 1, 3),
                Cfg(1, 128, 64, -1, 3), Cfg(1, 128, 64, 1, 0), Cfg(1, 128, 64, 40, 30),
                Cfg(1, 128, 64, 1, 3, -1), Cfg(1, 128, 64, 30, 30, 5)]:
        assert real.kvcache_storage_bytes(ctypes.byref(bad)) == 0
    h = P()
    real.kvcache_create.argtypes = [ctypes.POINTER(Cfg), P, ctypes.c_size_t, ctypes.POINTER(P)]
    good = Cfg(2, 128, 64, 1, 3)
    n = real.kvcache_storage_bytes(ctypes.byref(good))
    assert real.kvcache_create(ctypes.byref(good), None, n, ctypes.byref(h)) == EINVAL
    assert real.kvcache_create(ctypes.byref(good), P(0x10001), n, ctypes.byref(h)) == EINVAL
    assert real.kvcache_create(ctypes.byref(good), P(0x10000), n - 1, ctypes.byref(h)) == ECAPACITY
    real.chunk_attention.argtypes = [P, P, P, P, ctypes.c_int64, ctypes.c_float, P, P]
    assert real.chunk_attention(None, dummy, dummy, dummy, 4, 0.1, dummy, None) == EINVAL
    real.kvcache_append.argtypes = [P, P, P, ctypes.c_int32, P]
    assert real.kvcache_append(None, dummy, dummy, 1, None) == EINVAL
    real.nvfp4kv_strerror.restype = ctypes.c_char_p
    assert b"invalid" in real.nvfp4kv_strerror(EINVAL)


def test_storage_bytes_budget(real):
    """9/16 byte per cached element for each of K and V (reading note: 9/8 T_c H d
    bytes for K and V), plus scratch of a fixed size that does not grow with the
    cache: the tensor-scale table, the quantizer workspace, and the attention
    load-balancing slots (one partial query-block result, fp32 output plus per-lane
    max and sum, and one 8-byte flag per workgroup of a 256-CU launch)."""
    real.kvcache_storage_bytes.restype = ctypes.c_size_t
    real.kvcache_storage_bytes.argtypes = [ctypes.POINTER(Cfg)]
    for D, queries, threads, wgs in ((128, 256, 512, 256), (64, 128, 256, 512)):
        attn = wgs * (queries * D * 4 + threads * 8 + 8)
        fixed = None
        for sink, window in ((3, 9), (6, 18)):
            cfg = Cfg(12, D, 1560, sink, window)
            n = real.kvcache_storage_bytes(ctypes.byref(cfg))
            elems = 12 * D * 1560 * (sink + window)
            rest = n - 2 * elems * 9 // 16
            assert attn <= rest <= attn + 64 * 1024, (D, sink, window)
            if fixed is not None:
                assert rest == fixed      # independent of the cache length
            fixed = rest
    # K-smoothing adds the fp32 channel means of every scale slot (65 x H x D), the
    # mean reduction's workspace (two buffers of H x D node sums per 256 padded tokens)
    # and the single pass's exchange words (2048 head words, one per 128-byte line, and
    # per 256-token tile of the longest chunk, 3 + 9 frames of 1560 tokens = 74 tiles,
    # H x D tagged channel sums and H x D tagged channel extremes, and 64 words of slack
    # per tile plus 16)
    plain = real.kvcache_storage_bytes(ctypes.byref(Cfg(12, 128, 1560, 3, 9)))
    smooth = real.kvcache_storage_bytes(ctypes.byref(Cfg(12, 128, 1560, 3, 9, 0, 1)))
    adaptive = real.kvcache_storage_bytes(ctypes.byref(Cfg(12, 128, 1560, 3, 9, 0, 2)))
    assert adaptive == plain
    slots = (16 * 2048 + 2 * 12 * 74 * 128 + (74 + 16) * 64) * 8
    assert smooth - plain == 65 * 12 * 128 * 4 + 2 * 12 * (32768 // 256) * 128 * 4 + -(-slots // 256) * 256
    # MXFP4 (option 4): 17/32 byte per cached element (scales per 32 instead of 16);
    # it does not combine with the NVFP4 options; no other option bits exist
    mx = real.kvcache_storage_bytes(ctypes.byref(Cfg(12, 128, 1560, 3, 9, 0, 4)))
    elems = 12 * 128 * 1560 * 12
    assert plain - mx == 2 * (elems // 16 - elems // 32)
    for opts in (5, 6, 7, 8, 9, 10, 16):
        assert real.kvcache_storage_bytes(ctypes.byref(Cfg(12, 128, 1560, 3, 9, 0, opts))) == 0
    # the MX-scaled QK^T needs the MXFP4 cache, whose storage it shares
    assert real.kvcache_storage_bytes(ctypes.byref(Cfg(12, 128, 1560, 3, 9, 0, 12))) == mx


# ------------------------------------------------------------ host stub


@pytest.fixture(scope="module")
def stub():
    src = [os.path.join(ROOT, "nvfp4_kv_cache_amd", "csrc", "api.cpp"),
           os.path.join(ROOT, "tests", "host_stub", "stub_launch.cpp")]
    flags = SAN_FLAGS if SANITIZE else []
    subprocess.run(["g++", "-O1", "-std=c++17", "-fPIC", "-shared", *flags, "-o", STUB] + src, check=True)
    L = ctypes.CDLL(STUB)
    P = ctypes.c_void_p
    L.kvcache_storage_bytes.restype = ctypes.c_size_t
    L.kvcache_storage_bytes.argtypes = [ctypes.POINTER(Cfg)]
    L.kvcache_create.argtypes = [ctypes.POINTER(Cfg), P, ctypes.c_size_t, ctypes.POINTER(P)]
    L.kvcache_append.argtypes = [P, P, P, ctypes.c_int32, P]
    L.kvcache_evict.argtypes = [P, ctypes.c_int32]
    L.kvcache_destroy.argtypes = [P]
    L.chunk_attention.argtypes = [P, P, P, P, ctypes.c_int64, ctypes.c_float, P, P]
    L.kvcache_tokens.argtypes = [P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
    L.kvcache_begin_shot.argtypes = [P]
    L.kvcache_shot_sink.argtypes = [P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32),
                                    ctypes.POINTER(ctypes.c_int64)]
    L.kvcache_export_chunk.argtypes = [P, ctypes.c_int32] + [P] * 7
    L.kvcache_append_schedule.argtypes = [P, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
    L.stub_last_segments.argtypes = [ctypes.POINTER(ctypes.c_int32), ctypes.c_int]
    L.stub_last_quant_slots.argtypes = [ctypes.POINTER(ctypes.c_int32), ctypes.c_int,
                                        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)]
    L.stub_last_scale_ptr.restype = ctypes.c_int64
    L.stub_last_export_slot.argtypes = [ctypes.POINTER(ctypes.c_int32), ctypes.c_int]
    return L


class StubCache:
    BASE = 1 << 32

    def __init__(self, L, cfg):
        self.L, self.cfg = L, cfg
        n = L.kvcache_storage_bytes(ctypes.byref(cfg))
        assert n > 0
        self.base, self.nbytes = self.BASE, n
        self.h = ctypes.c_void_p()
        assert L.kvcache_create(ctypes.byref(cfg), ctypes.c_void_p(self.BASE), n, ctypes.byref(self.h)) == OK

    def append(self, n_frames):
        d = ctypes.c_void_p(0x1000)
        return self.L.kvcache_append(self.h, d, d, n_frames, None)

    def segments(self):
        d = ctypes.c_void_p(0x1000)
        assert self.L.chunk_attention(self.h, d, d, d, 8, 0.125, d, None) == OK
        buf = (ctypes.c_int32 * 192)()
        n = self.L.stub_last_segments(buf, 64)
        return [tuple(buf[3 * i:3 * i + 3]) for i in range(n)]

    def quant_slots(self):
        buf = (ctypes.c_int32 * 64)()
        nt, rows = ctypes.c_int32(), ctypes.c_int64()
        n = self.L.stub_last_quant_slots(buf, 64, ctypes.byref(nt), ctypes.byref(rows))
        return list(buf[:n]), nt.value, rows.value


@pytest.mark.parametrize("seed", range(16))
def test_cache_metadata_matches_frame_list_model(stub, seed):
    """Random append/evict/scene-cut sequences: the tokens the attention kernel would
    read (segment list, in order) are exactly the frames of the oracle's cache model
    (global sink, shot-level sink, window), each frame's slot being where its chunk's
    quantize launch wrote it, and each segment carrying its chunk's tensor-scale
    slot.  Seeds 0-7 run without a shot-level sink."""
    rng = np.random.default_rng(seed)
    sink, window = int(rng.integers(0, 4)), int(rng.integers(1, 8))
    shot = 0 if seed < 8 else int(rng.integers(1, 4))
    T_f = 8 * int(rng.integers(1, 5))
    c = StubCache(stub, Cfg(1, 64, T_f, sink, window, shot))
    model = CacheModel(1, 64, T_f, sink, window, shot_frames=shot)
    where = {}          # (chunk, frame) -> slot
    scale_of = {}       # chunk -> table offset of its K scale
    chunk = 0
    for step in range(60):
        if shot and rng.random() < 0.15:
            assert stub.kvcache_begin_shot(c.h) == OK
            model.begin_shot()
        if rng.random() < 0.2 and len(model.window) > 0:
            e = int(rng.integers(1, len(model.window) + 1))
            assert stub.kvcache_evict(c.h, e) == OK
            model.evict(e)
        nf = int(rng.integers(1, window + 1))
        assert c.append(nf) == OK
        slots, nt, rows = c.quant_slots()
        assert nt == 2 and rows == (sink + window + shot) * T_f and len(slots) == nf
        for f, s in enumerate(slots):
            where[(chunk, f)] = s
        scale_of[chunk] = stub.stub_last_scale_ptr(0) - StubCache.BASE
        assert stub.stub_last_scale_ptr(1) - stub.stub_last_scale_ptr(0) == 4
        zeros = np.zeros((1, nf * T_f, 64), dtype=np.uint16)
        model.append(zeros, zeros)
        chunk += 1
        # expected token runs from the model, in key order
        want_tokens = []
        for fr in model.frames():
            s = where[(fr.chunk_id, fr.frame_in_chunk)]
            want_tokens += [(t, fr.chunk_id) for t in range(s * T_f, (s + 1) * T_f)]
        got_tokens = []
        seg_scale = {}
        for tok0, ntok, sslot in c.segments():
            for t in range(tok0, tok0 + ntok):
                got_tokens.append(t)
            seg_scale.setdefault(sslot, set()).update(range(tok0, tok0 + ntok))
        assert got_tokens == [t for t, _ in want_tokens]
        # all tokens of a segment belong to chunks sharing that scale slot
        tok_chunk = dict(want_tokens)
        for sslot, toks in seg_scale.items():
            chunks = {tok_chunk[t] for t in toks}
            assert len(chunks) == 1
        # slots in use are distinct
        occupied = [where[(fr.chunk_id, fr.frame_in_chunk)] for fr in model.frames()]
        assert len(set(occupied)) == len(occupied)
        # sink frames sit in slots [0, sink)
        for i, fr in enumerate(model.sinks):
            assert where[(fr.chunk_id, fr.frame_in_chunk)] == i
        s_tok, w_tok = ctypes.c_int64(), ctypes.c_int64()
        stub.kvcache_tokens(c.h, ctypes.byref(s_tok), ctypes.byref(w_tok))
        assert s_tok.value == len(model.sinks) * T_f and w_tok.value == len(model.window) * T_f
        st, nsh, extra = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int64()
        assert stub.kvcache_shot_sink(c.h, ctypes.byref(st), ctypes.byref(nsh), ctypes.byref(extra)) == OK
        assert st.value == model.shot_start
        assert nsh.value == min(shot, model.n_frames - model.shot_start)
        assert extra.value == len(model.pinned) * T_f
    stub.kvcache_destroy(c.h)


def test_cache_errors_and_rollback(stub):
    c = StubCache(stub, Cfg(2, 128, 16, 1, 3))
    assert c.append(5) == ECAPACITY          # 4 frames would enter a 3-frame window
    assert c.append(0) == EINVAL
    assert stub.kvcache_evict(c.h, 1) == ESTATE
    assert c.append(4) == OK                 # 1 sink + 3 window
    stub.stub_fail_next(EHIP)
    assert c.append(2) == EHIP               # a failed launch leaves the state unchanged
    assert c.segments() == [(0, 64, 0)]
    assert stub.kvcache_evict(c.h, 4) == ESTATE
    assert stub.kvcache_evict(c.h, 2) == OK
    assert c.segments() == [(0, 16, 0), (48, 16, 0)]
    d = ctypes.c_void_p(0x1000)
    # chunk 0 lost two frames: not fully resident, cannot be exported
    assert stub.kvcache_export_chunk(c.h, 0, d, d, d, d, d, d, None) == ESTATE
    assert stub.kvcache_export_chunk(c.h, 7, d, d, d, d, d, d, None) == ESTATE
    assert c.append(2) == OK
    segs = c.segments()
    assert segs[0] == (0, 16, 0) and segs[1] == (48, 16, 0) and segs[2][1] == 32
    assert segs[2][2] != 0
    buf = (ctypes.c_int32 * 64)()
    assert stub.kvcache_export_chunk(c.h, 1, d, d, d, d, d, d, None) == OK
    assert stub.stub_last_export_slot(buf, 64) == segs[2][2]
    stub.kvcache_destroy(c.h)


def test_cache_options_route_to_their_kernels(stub):
    """Each cache option reaches the launches it changes: K-smoothing runs the mean
    reduction and hands its means to the quantizer and to attention; adaptive V
    scales mark V; appends with either option take the two-pass quantizer (epoch 0),
    plain ones may take the single pass; MXFP4 appends go to the
    single-pass MXFP4 quantizer (never the NVFP4 one), and its attention and export
    launches carry the format; kvcache_append_schedule reports the same routing."""
    stub.stub_last_attn_k_mean.restype = ctypes.c_int64
    stub.stub_last_quant_epoch.restype = ctypes.c_int64
    stub.stub_last_quant_slots_ptr.restype = ctypes.c_int64
    d = ctypes.c_void_p(0x1000)
    for opts in (0, 1, 2, 3, 4, 12):
        before = [stub.stub_calls(k) for k in range(6)]
        c = StubCache(stub, Cfg(2, 128, 16, 1, 3, 0, opts))
        assert c.append(2) == OK
        after = [stub.stub_calls(k) for k in range(6)]
        calls = [a - b for a, b in zip(after, before)]
        assert calls[3] == 0   # the mean levels are the options launcher's fallback, not the host's
        if opts & 4:
            assert calls[0] == 0 and calls[4] == 1 and calls[5] == 0
        elif opts:
            # K-smoothing and adaptive V scales: the options launcher, with an epoch;
            # K-smoothing caches also hand it their exchange slots (zeroed at create,
            # inside the storage)
            assert calls[5] == 1 and calls[0] == 0 and calls[4] == 0
            assert stub.stub_last_quant_options() == opts
            assert stub.stub_last_quant_epoch() > 0
            for which in (0, 1):
                ptr = stub.stub_last_quant_slots_ptr(which)
                assert (ptr != -1) == bool(opts & 1)
                if opts & 1:
                    assert c.base <= ptr < c.base + c.nbytes
        else:
            assert calls[0] == 1 and calls[4] == 0 and calls[5] == 0
            assert stub.stub_last_quant_options() == 0
            assert stub.stub_last_quant_epoch() > 0
        sched = ctypes.c_int32()
        assert stub.kvcache_append_schedule(c.h, 2, ctypes.byref(sched)) == OK
        assert sched.value == (3 if opts & 4 else 4 if opts else 1)
        assert stub.kvcache_append_schedule(c.h, 0, ctypes.byref(sched)) == EINVAL
        assert stub.chunk_attention(c.h, d, d, d, 8, 0.125, d, None) == OK
        assert stub.stub_last_attn_mx() == (2 if opts & 8 else 1 if opts & 4 else 0)
        assert (stub.stub_last_attn_k_mean() != 0) == bool(opts & 1)
        assert stub.kvcache_export_chunk(c.h, 0, d, d, d, d, d, d, None) == OK
        assert stub.stub_last_export_block() == (32 if opts & 4 else 16)
        stub.kvcache_destroy(c.h)


@pytest.mark.skipif(SANITIZE, reason="this test starts the sanitized run itself")
def test_metadata_under_sanitizers():
    """The host code (api.cpp: slot map, FIFO eviction, segment lists, argument checks)
    built with AddressSanitizer and UndefinedBehaviorSanitizer runs every stub test of
    this file in a child process; any report aborts it."""
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("no ASan runtime for g++")
    env = dict(os.environ, NVFP4KV_STUB_SANITIZE="1", LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run(["python", "-m", "pytest", "-q", "-p", "no:cacheprovider", __file__,
                        "-k", "metadata_matches or errors_and_rollback or options_route"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert " passed" in r.stdout, tail
