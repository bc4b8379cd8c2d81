"""Thin ctypes binding of libnvfp4kv (C ABI in include/nvfp4kv.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's gfx950 kernels.
There is no CPU fallback: without the built library every call raises.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4kv.so")

_lib = None


class NVFP4KVError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


class KVCacheConfig(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("tokens_per_frame", ctypes.c_int32), ("sink_frames", ctypes.c_int32),
                ("window_frames", ctypes.c_int32), ("shot_frames", ctypes.c_int32),
                ("options", ctypes.c_int32)]


K_SMOOTH = 1      # NVFP4KV_K_SMOOTH
V_ADAPTIVE = 2    # NVFP4KV_V_ADAPTIVE
MXFP4 = 4         # NVFP4KV_MXFP4
MX_SCALED_QK = 8  # NVFP4KV_MX_SCALED_QK


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m nvfp4_kv_cache_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, SZ, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
        sig = {
            "nvfp4kv_strerror": (ctypes.c_char_p, [I]),
            "nvfp4kv_version": (ctypes.c_char_p, []),
            "nvfp4kv_set_wait_limit": (I, [ctypes.c_int32]),
            "nvfp4_quantize_workspace_bytes": (SZ, []),
            "nvfp4_quantize_kv": (I, [P, I64, I64, I64, P, P, P, P, SZ, P]),
            "nvfp4_quantize_noalloc_scratch_bytes": (SZ, []),
            "nvfp4kv_stream_reference": (I, [P, P, I64, I64, I64, P, P, P, P, P]),
            "nvfp4_quantize_kv_noalloc": (I, [P, I64, I64, I64, P, P, P, P]),
            "mxfp4_quantize_kv": (I, [P, I64, I64, I64, P, P, P]),
            "kvcache_storage_bytes": (SZ, [ctypes.POINTER(KVCacheConfig)]),
            "kvcache_create": (I, [ctypes.POINTER(KVCacheConfig), P, SZ, ctypes.POINTER(P)]),
            "kvcache_destroy": (I, [P]),
            "kvcache_append": (I, [P, P, P, ctypes.c_int32, P]),
            "kvcache_evict": (I, [P, ctypes.c_int32]),
            "kvcache_append_schedule": (I, [P, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]),
            "kvcache_tokens": (I, [P, ctypes.POINTER(I64), ctypes.POINTER(I64)]),
            "kvcache_begin_shot": (I, [P]),
            "kvcache_export_k_mean": (I, [P, ctypes.c_int32, P, P]),
            "kvcache_shot_sink": (I, [P, ctypes.POINTER(I64), ctypes.POINTER(ctypes.c_int32),
                                      ctypes.POINTER(I64)]),
            "kvcache_chunk_count": (I, [P, ctypes.POINTER(ctypes.c_int32)]),
            "kvcache_chunk_frames": (I, [P, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]),
            "chunk_attention": (I, [P, P, P, P, I64, F, P, P]),
            "kvcache_export_chunk": (I, [P, ctypes.c_int32, P, P, P, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def strerror(status):
    return lib().nvfp4kv_strerror(int(status)).decode()


def _check(rc, where):
    if rc != 0:
        raise NVFP4KVError(rc, where)


def set_wait_limit(limit):
    """Testing hook: polls the bounded waits between workgroups make (the append
    quantizer's maxima exchange, the attention's partial-result merge) before taking
    their fallback paths (same results either way)."""
    _check(lib().nvfp4kv_set_wait_limit(int(limit)), "nvfp4kv_set_wait_limit")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _bf16_ptr(t, name, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold bf16 values (bfloat16 or their 16-bit patterns)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def quantize_workspace(device=None):
    """A zero-filled workspace for quantize_kv (reusable across calls)."""
    n = lib().nvfp4_quantize_workspace_bytes()
    return torch.zeros(n, dtype=torch.uint8, device=device or "cuda")


def quantize_kv(x, workspace=None):
    """NVFP4 codec of one bf16 tensor [H, T, D]: returns (codes uint8 [H,T,D/2],
    scales uint8 [H,T,D/16], tensor_scale float32 [1])."""
    H, T, D = x.shape
    dev = x.device
    if workspace is None:
        workspace = quantize_workspace(dev)
    codes = torch.empty((H, T, D // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((H, T, D // 16), dtype=torch.uint8, device=dev)
    ts = torch.empty(1, dtype=torch.float32, device=dev)
    rc = lib().nvfp4_quantize_kv(_bf16_ptr(x, "x"), H, T, D, ctypes.c_void_p(codes.data_ptr()),
                                 ctypes.c_void_p(scales.data_ptr()), ctypes.c_void_p(ts.data_ptr()),
                                 ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream())
    _check(rc, "nvfp4_quantize_kv")
    return codes, scales, ts


def quantize_kv_noalloc(x, out=None):
    """The same codec through the entry point that allocates nothing (its scratch is
    the library's per-device array).  ``out`` optionally gives preallocated (codes,
    scales, tensor_scale) tensors of the shapes quantize_kv returns, so that the call
    itself allocates nothing either; returns them."""
    H, T, D = x.shape
    dev = x.device
    if out is None:
        out = (torch.empty((H, T, D // 2), dtype=torch.uint8, device=dev),
               torch.empty((H, T, D // 16), dtype=torch.uint8, device=dev),
               torch.empty(1, dtype=torch.float32, device=dev))
    codes, scales, ts = out
    for t, shape, dt, name in ((codes, (H, T, D // 2), torch.uint8, "codes"),
                               (scales, (H, T, D // 16), torch.uint8, "scales"),
                               (ts, (1,), torch.float32, "tensor_scale")):
        if tuple(t.shape) != shape or t.dtype != dt or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name}: expected a contiguous {dt} tensor of shape {shape} on {dev}")
    rc = lib().nvfp4_quantize_kv_noalloc(_bf16_ptr(x, "x"), H, T, D, ctypes.c_void_p(codes.data_ptr()),
                                         ctypes.c_void_p(scales.data_ptr()), ctypes.c_void_p(ts.data_ptr()),
                                         _stream())
    _check(rc, "nvfp4_quantize_kv_noalloc")
    return codes, scales, ts


def stream_reference(x0, x1, out):
    """Measurement hook: moves the bytes of a two-tensor codec call with the quantizer's
    tiling and no exchange between workgroups (outputs are not an encoding).  out =
    (codes0, scales0, codes1, scales1), preallocated uint8 tensors."""
    H, T, D = x0.shape
    ptrs = [ctypes.c_void_p(t.data_ptr()) for t in out]
    _check(lib().nvfp4kv_stream_reference(_bf16_ptr(x0, "x0"), _bf16_ptr(x1, "x1", (H, T, D)), H, T, D, *ptrs,
                                          _stream()), "nvfp4kv_stream_reference")


def mxfp4_quantize_kv(x):
    """MXFP4 codec of one bf16 tensor [H, T, D] (D % 32 == 0): returns (codes uint8
    [H,T,D/2], scales uint8 E8M0 [H,T,D/32])."""
    H, T, D = x.shape
    dev = x.device
    codes = torch.empty((H, T, D // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((H, T, D // 32), dtype=torch.uint8, device=dev)
    rc = lib().mxfp4_quantize_kv(_bf16_ptr(x, "x"), H, T, D, ctypes.c_void_p(codes.data_ptr()),
                                 ctypes.c_void_p(scales.data_ptr()), _stream())
    _check(rc, "mxfp4_quantize_kv")
    return codes, scales


class KVCache:
    """Sink + window NVFP4 (or MXFP4) KV cache on one device (see include/nvfp4kv.h)."""

    def __init__(self, n_heads, head_dim, tokens_per_frame, sink_frames, window_frames,
                 device=None, shot_frames=0, k_smooth=False, v_adaptive=False, mxfp4=False,
                 mx_scaled_qk=False):
        opts = (K_SMOOTH if k_smooth else 0) | (V_ADAPTIVE if v_adaptive else 0) | (MXFP4 if mxfp4 else 0)
        opts |= MX_SCALED_QK if mx_scaled_qk else 0
        self.cfg = KVCacheConfig(n_heads, head_dim, tokens_per_frame, sink_frames, window_frames,
                                 shot_frames, opts)
        n = lib().kvcache_storage_bytes(ctypes.byref(self.cfg))
        if n == 0:
            raise ValueError("unsupported cache configuration")
        self.device = torch.device(device or "cuda")
        self.storage = torch.empty(n, dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        rc = lib().kvcache_create(ctypes.byref(self.cfg), ctypes.c_void_p(self.storage.data_ptr()),
                                  n, ctypes.byref(h))
        _check(rc, "kvcache_create")
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            lib().kvcache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def n_heads(self):
        return self.cfg.n_heads

    @property
    def head_dim(self):
        return self.cfg.head_dim

    def append(self, k, v, n_frames):
        shape = (self.cfg.n_heads, n_frames * self.cfg.tokens_per_frame, self.cfg.head_dim)
        rc = lib().kvcache_append(self._h, _bf16_ptr(k, "k", shape), _bf16_ptr(v, "v", shape),
                                  n_frames, _stream())
        _check(rc, "kvcache_append")

    def append_schedule(self, n_frames):
        """1: single-pass quantizer, 2: two passes, 3: MXFP4 quantizer, 4: single pass
        with the cache options (see the header)."""
        r = ctypes.c_int32()
        _check(lib().kvcache_append_schedule(self._h, n_frames, ctypes.byref(r)), "kvcache_append_schedule")
        return r.value

    def evict(self, n_frames):
        _check(lib().kvcache_evict(self._h, n_frames), "kvcache_evict")

    def tokens(self):
        s, w = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().kvcache_tokens(self._h, ctypes.byref(s), ctypes.byref(w)), "kvcache_tokens")
        return s.value, w.value

    def begin_shot(self):
        """Scene cut: the next appended frame starts a new shot."""
        _check(lib().kvcache_begin_shot(self._h), "kvcache_begin_shot")

    def shot_sink(self):
        """(start_frame, n_frames, extra_tokens) of the shot-level sink."""
        st, n, ex = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int64()
        _check(lib().kvcache_shot_sink(self._h, ctypes.byref(st), ctypes.byref(n), ctypes.byref(ex)),
               "kvcache_shot_sink")
        return st.value, n.value, ex.value

    def chunk_count(self):
        n = ctypes.c_int32()
        _check(lib().kvcache_chunk_count(self._h, ctypes.byref(n)), "kvcache_chunk_count")
        return n.value

    def attention(self, q, k_own, v_own, softmax_scale, out=None):
        H, n_q, D = q.shape
        shape = (self.cfg.n_heads, n_q, self.cfg.head_dim)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=q.device)
        if out.dtype != torch.float32 or tuple(out.shape) != shape or not out.is_contiguous():
            raise ValueError("out must be a contiguous float32 tensor [H, n_q, D]")
        rc = lib().chunk_attention(self._h, _bf16_ptr(q, "q", shape), _bf16_ptr(k_own, "k_own", shape),
                                   _bf16_ptr(v_own, "v_own", shape), n_q, float(softmax_scale),
                                   ctypes.c_void_p(out.data_ptr()), _stream())
        _check(rc, "chunk_attention")
        return out

    def chunk_frames(self, chunk_index):
        n = ctypes.c_int32()
        _check(lib().kvcache_chunk_frames(self._h, chunk_index, ctypes.byref(n)), "kvcache_chunk_frames")
        return n.value

    def export_chunk(self, chunk_index):
        """(k_codes, k_scales, v_codes, v_scales, k_scale, v_scale) of a resident
        chunk, in the codec layout."""
        nf = self.chunk_frames(chunk_index)
        H, D, T = self.cfg.n_heads, self.cfg.head_dim, nf * self.cfg.tokens_per_frame
        dev = self.device
        kc = torch.empty((H, T, D // 2), dtype=torch.uint8, device=dev)
        ks = torch.empty((H, T, D // (32 if self.cfg.options & MXFP4 else 16)), dtype=torch.uint8, device=dev)
        vc = torch.empty_like(kc)
        vs = torch.empty_like(ks)
        sk = torch.empty(1, dtype=torch.float32, device=dev)
        sv = torch.empty(1, dtype=torch.float32, device=dev)
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        rc = lib().kvcache_export_chunk(self._h, chunk_index, p(kc), p(ks), p(vc), p(vs), p(sk), p(sv),
                                        _stream())
        _check(rc, "kvcache_export_chunk")
        return kc, ks, vc, vs, sk, sv

    def export_k_mean(self, chunk_index):
        """K-smoothing channel means [H, D] (fp32) of a resident chunk."""
        mu = torch.empty((self.cfg.n_heads, self.cfg.head_dim), dtype=torch.float32, device=self.device)
        _check(lib().kvcache_export_k_mean(self._h, chunk_index, ctypes.c_void_p(mu.data_ptr()), _stream()),
               "kvcache_export_k_mean")
        return mu
