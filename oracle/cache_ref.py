"""Sink + sliding-window KV cache with a shot-level sink, as an ordered frame list
(test infrastructure).

Paper text, section 4.2 "Inference with Multi-Shot Attention Sink": inference
keeps a sliding window of cached chunks (per-step cost O(W * L_c)); the global
sink is the first S_g frames of the video, kept permanently; the shot-level sink
is the first S_s frames of the current shot, re-bound at every scene cut, tracked
by a (start, len) pair and kept once the window has rolled past it; the effective
key set is the union of the global sink, the shot-level sink and the window, with
duplicate tokens removed.  Reading note, "The inference infrastructure": each
appended frame chunk is quantized to NVFP4 on its own (one tensor scale per chunk
tensor), optionally with K-smoothing for K and adaptive scale selection for V
(see nvfp4_ref; the smoothing means are added back to the dequantized K).  As the
alternative the paper text's appendix A.2 "FP4 Quantization" sets against NVFP4,
a cache may hold MXFP4 instead (see mxfp4_ref): 32-element blocks with E8M0
scales and no tensor scale.

Model: frames are numbered in append order.  The first ``sink_frames`` frames are
the global sink; every later frame joins a FIFO window of at most
``window_frames`` frames; when a frame arrives at a full window the oldest window
frame leaves the window.  A frame leaving the window stays (is "pinned") if its
number lies in [shot_start, shot_start + shot_frames); ``begin_shot`` drops the
pinned frames and moves shot_start to the next frame.  A global-sink frame is
stored once and never enters the window, and a pinned frame is no longer in the
window, so the union is duplicate-free.  The effective key order is global sink,
pinned frames, window oldest first (attention is invariant to key order, so this
order is a convention only).
"""

from collections import deque
from dataclasses import dataclass

import numpy as np

from .nvfp4_ref import quantize_ref, dequantize_ref, channel_mean_ref
from .mxfp4_ref import mx_quantize_ref, mx_dequantize_ref


@dataclass
class Frame:
    chunk_id: int
    frame_in_chunk: int
    k_codes: np.ndarray   # uint8 [H, T_f, D/2]
    k_scales: np.ndarray  # uint8 [H, T_f, D/16] (MXFP4: E8M0 bytes [H, T_f, D/32])
    v_codes: np.ndarray
    v_scales: np.ndarray
    s_k: np.float32
    s_v: np.float32
    index: int = -1       # number of the frame in append order
    k_mean: np.ndarray = None   # K-smoothing channel means of the frame's chunk [H, D]
    mx: bool = False            # MXFP4 codes and scales (s_k, s_v unused)


class CacheModel:
    def __init__(self, n_heads, head_dim, tokens_per_frame, sink_frames, window_frames,
                 shot_frames=0, k_smooth=False, v_adaptive=False, mxfp4=False):
        self.H = n_heads
        self.D = head_dim
        self.T_f = tokens_per_frame
        self.S_g = sink_frames
        self.W_f = window_frames
        self.S_s = shot_frames
        self.k_smooth = k_smooth      # K quantized after subtracting its chunk's channel means
        self.v_adaptive = v_adaptive  # V blocks take the better of the 6- and 4-scaled encodings
        self.mxfp4 = mxfp4            # MXFP4 instead of NVFP4 (no smoothing, no adaptive scales)
        assert not (mxfp4 and (k_smooth or v_adaptive)), "the options are NVFP4 steps"
        self.chunk_mean = {}          # chunk id -> K channel means [H, D] (K-smoothing only)
        self.sinks = []
        self.window = deque()
        self.pinned = []        # shot-level-sink frames that left the window
        self.n_frames = 0       # frames appended so far
        self.shot_start = 0     # number of the current shot's first frame
        self.n_chunks = 0
        self.chunk_codes = {}   # chunk id -> (k_codes, k_scales, s_k, v_codes, v_scales, s_v)

    def _in_shot_sink(self, fr):
        return self.shot_start <= fr.index < self.shot_start + self.S_s

    def _leave_window(self):
        fr = self.window.popleft()
        if self._in_shot_sink(fr):
            self.pinned.append(fr)

    def begin_shot(self):
        """Scene cut: the next appended frame starts a new shot."""
        self.pinned = []
        self.shot_start = self.n_frames

    def append(self, k_bits, v_bits):
        """Quantize one chunk's K and V (bf16 bits [H, n*T_f, D]) and push its
        frames.  Returns the chunk id (0, 1, ...)."""
        k_bits = np.asarray(k_bits, dtype=np.uint16)
        v_bits = np.asarray(v_bits, dtype=np.uint16)
        H, T, D = k_bits.shape
        assert (H, D) == (self.H, self.D) and v_bits.shape == k_bits.shape
        assert T % self.T_f == 0
        n_frames = T // self.T_f
        mu = channel_mean_ref(k_bits) if self.k_smooth else None
        if self.mxfp4:
            (kc, ks), (vc, vs) = mx_quantize_ref(k_bits), mx_quantize_ref(v_bits)
            sk = sv = np.float32(1.0)
        else:
            kc, ks, sk = quantize_ref(k_bits, mean=mu)
            vc, vs, sv = quantize_ref(v_bits, adaptive=self.v_adaptive)
        cid = self.n_chunks
        self.n_chunks += 1
        self.chunk_codes[cid] = (kc, ks, sk, vc, vs, sv)
        if mu is not None:
            self.chunk_mean[cid] = mu
        for f in range(n_frames):
            sl = slice(f * self.T_f, (f + 1) * self.T_f)
            fr = Frame(cid, f, kc[:, sl], ks[:, sl], vc[:, sl], vs[:, sl], sk, sv, self.n_frames, mu,
                       self.mxfp4)
            self.n_frames += 1
            if len(self.sinks) < self.S_g:
                self.sinks.append(fr)
            else:
                if len(self.window) == self.W_f:
                    self._leave_window()
                self.window.append(fr)
        return cid

    def evict(self, n_frames):
        """Drop the oldest ``n_frames`` window frames (never global sinks; a
        shot-level-sink frame stays, pinned)."""
        assert 0 <= n_frames <= len(self.window)
        for _ in range(n_frames):
            self._leave_window()

    def frames(self):
        return list(self.sinks) + list(self.pinned) + list(self.window)

    def n_tokens(self):
        return len(self.frames()) * self.T_f

    def dequantized_kv(self):
        """Float64 K and V of the effective key set, [H, n_tokens, D] each."""
        frs = self.frames()
        if not frs:
            z = np.zeros((self.H, 0, self.D))
            return z, z.copy()
        def deq(codes, scales, s_t, mx):
            return mx_dequantize_ref(codes, scales) if mx else dequantize_ref(codes, scales, s_t)
        ks = [deq(f.k_codes, f.k_scales, f.s_k, f.mx)
              + (0.0 if f.k_mean is None else f.k_mean.astype(np.float64)[:, None, :]) for f in frs]
        vs = [deq(f.v_codes, f.v_scales, f.s_v, f.mx) for f in frs]
        return np.concatenate(ks, axis=1), np.concatenate(vs, axis=1)
