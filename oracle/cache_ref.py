"""Sink + sliding-window KV cache, as an ordered frame list (test infrastructure).

Paper text, section 4.2 "Inference with Multi-Shot Attention Sink": inference
keeps a sliding window of cached chunks (per-step cost O(W * L_c)); the global
sink is the first S_g frames of the video, kept permanently; the effective key
set is the union of the sink and the window with duplicate tokens removed.
Reading note, "The inference infrastructure": each appended frame chunk is
quantized to NVFP4 on its own (one tensor scale per chunk tensor).

Model: the first ``sink_frames`` frames ever appended are sinks; every later
frame joins a FIFO window of at most ``window_frames`` frames; when a frame
arrives at a full window the oldest window frame leaves.  A sink frame is
stored once and never enters the window, so the union is duplicate-free.  The
effective key order is sinks, then window frames oldest first (attention is
invariant to key order, so this order is a convention only).
"""

from collections import deque
from dataclasses import dataclass

import numpy as np

from .nvfp4_ref import quantize_ref, dequantize_ref


@dataclass
class Frame:
    chunk_id: int
    frame_in_chunk: int
    k_codes: np.ndarray   # uint8 [H, T_f, D/2]
    k_scales: np.ndarray  # uint8 [H, T_f, D/16]
    v_codes: np.ndarray
    v_scales: np.ndarray
    s_k: np.float32
    s_v: np.float32


class CacheModel:
    def __init__(self, n_heads, head_dim, tokens_per_frame, sink_frames, window_frames):
        self.H = n_heads
        self.D = head_dim
        self.T_f = tokens_per_frame
        self.S_g = sink_frames
        self.W_f = window_frames
        self.sinks = []
        self.window = deque()
        self.n_chunks = 0
        self.chunk_codes = {}   # chunk id -> (k_codes, k_scales, s_k, v_codes, v_scales, s_v)

    def append(self, k_bits, v_bits):
        """Quantize one chunk's K and V (bf16 bits [H, n*T_f, D]) and push its
        frames.  Returns the chunk id (0, 1, ...)."""
        k_bits = np.asarray(k_bits, dtype=np.uint16)
        v_bits = np.asarray(v_bits, dtype=np.uint16)
        H, T, D = k_bits.shape
        assert (H, D) == (self.H, self.D) and v_bits.shape == k_bits.shape
        assert T % self.T_f == 0
        n_frames = T // self.T_f
        kc, ks, sk = quantize_ref(k_bits)
        vc, vs, sv = quantize_ref(v_bits)
        cid = self.n_chunks
        self.n_chunks += 1
        self.chunk_codes[cid] = (kc, ks, sk, vc, vs, sv)
        for f in range(n_frames):
            sl = slice(f * self.T_f, (f + 1) * self.T_f)
            fr = Frame(cid, f, kc[:, sl], ks[:, sl], vc[:, sl], vs[:, sl], sk, sv)
            if len(self.sinks) < self.S_g:
                self.sinks.append(fr)
            else:
                if len(self.window) == self.W_f:
                    self.window.popleft()
                self.window.append(fr)
        return cid

    def evict(self, n_frames):
        """Drop the oldest ``n_frames`` window frames (never sinks)."""
        assert 0 <= n_frames <= len(self.window)
        for _ in range(n_frames):
            self.window.popleft()

    def frames(self):
        return list(self.sinks) + list(self.window)

    def n_tokens(self):
        return len(self.frames()) * self.T_f

    def dequantized_kv(self):
        """Float64 K and V of the effective key set, [H, n_tokens, D] each."""
        frs = self.frames()
        if not frs:
            z = np.zeros((self.H, 0, self.D))
            return z, z.copy()
        ks = [dequantize_ref(f.k_codes, f.k_scales, f.s_k) for f in frs]
        vs = [dequantize_ref(f.v_codes, f.v_scales, f.s_v) for f in frs]
        return np.concatenate(ks, axis=1), np.concatenate(vs, axis=1)
