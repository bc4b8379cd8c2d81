"""Seeded synthetic workloads (shared by the GPU path's tests/bench and the
oracle's tests).  Holds no NVFP4 or attention arithmetic: only the shapes of
the five workloads and seeded draws of their bf16 inputs.

Shapes follow the Wan-style latent token counts the pages' models run at
(paper text, section 4.1: the base model is Wan2.2-TI2V-5B; section 5.3: 720p
generation), stood in by synthetic tensors: no prompts, weights or video data
are used.

Seeds: every tensor comes from
    numpy.random.default_rng(SeedSequence([cfg_seed, chunk, step, tensor_id]))
with tensor_id Q=0, K=1, V=2, outlier-channel choice for K=3 and V=4; a clean
chunk that is appended to the cache uses step=4.  Values are drawn in float32
and rounded to bf16 with round-to-nearest-even; those bf16 bit patterns are
the inputs of both the GPU path and the oracle.
"""

from dataclasses import dataclass, field

import numpy as np

Q_ID, K_ID, V_ID, KCH_ID, VCH_ID = 0, 1, 2, 3, 4
APPEND_STEP = 4


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    n_heads: int
    head_dim: int
    tokens_per_frame: int
    sink_frames: int
    window_frames: int
    chunk_frames: int        # frames per appended chunk
    n_cache_chunks: int      # chunks appended before the measured query chunk
    dist: str                # 'normal', 'normal_t4_2pct', 't4_outlier_channels'
    n_chunks: int = 1        # rollout length (streaming workload)
    steps_per_chunk: int = 1
    description: str = ""
    query_frames: int = 0    # frames of the query chunk (0: chunk_frames)

    @property
    def chunk_tokens(self):
        return self.chunk_frames * self.tokens_per_frame

    @property
    def n_q(self):
        return (self.query_frames or self.chunk_frames) * self.tokens_per_frame

    @property
    def softmax_scale(self):
        return 1.0 / float(np.sqrt(self.head_dim))

    def cache_frames_for_chunk(self, c):
        """Frames resident when chunk c's queries run (all earlier chunks
        appended, sink kept, window FIFO)."""
        total = c * self.chunk_frames
        sinks = min(total, self.sink_frames)
        return sinks + min(total - sinks, self.window_frames)


WORKLOADS = {
    # 1 head, D=64, 64 queries (one 64-token frame) over a 256-token cache (one
    # 4-frame chunk of 64-token frames: 1 sink + 3 window frames) plus their own
    # 64 tokens.
    "tiny": Workload("tiny", 1, 1, 64, 64, 1, 3, 4, 1, "normal", query_frames=1,
                     description="1 head, D64, 64 queries over a 256-token NVFP4 cache + 64 own bf16 tokens"),
    # K, V [12, 4680, 128] appended as one 3-frame chunk into a full 3+9 cache.
    "quantize": Workload("quantize", 2, 12, 128, 1560, 3, 9, 3, 4, "t4_outlier_channels",
                         description="K,V [12,4680,128] Student-t(4) with 4 outlier channels x20 per head, appended to a full 3 sink + 9 window cache"),
    # 1.3B-shaped: 12 heads, 1560 tokens/frame, 3-frame chunk over 3+9 frames.
    "wan13b": Workload("wan13b", 3, 12, 128, 1560, 3, 9, 3, 4, "normal_t4_2pct",
                       description="12 heads, D128, 4680 queries over 18720 NVFP4 cache tokens + 4680 own"),
    # 5B-shaped: 24 heads, 880 tokens/frame, 3-frame chunk over 3+18 frames.
    "wan5b": Workload("wan5b", 4, 24, 128, 880, 3, 18, 3, 7, "normal_t4_2pct",
                      description="24 heads, D128, 2640 queries over 18480 NVFP4 cache tokens + 2640 own"),
    # Streaming rollout: 40 chunks x (4 denoising steps + 1 append).
    "rollout": Workload("rollout", 5, 12, 128, 1560, 3, 9, 3, 0, "normal",
                        n_chunks=40, steps_per_chunk=4,
                        description="12 heads, D128, 1560 tok/frame, 40 chunks x (4 attention steps + append), 3 sink + 9 window frames"),
}


def rng_for(seed, chunk, step, tensor_id):
    return np.random.default_rng(np.random.SeedSequence([seed, chunk, step, tensor_id]))


def f32_to_bf16_bits(x):
    """Round finite float32 values to bf16 (round-to-nearest-even); returns
    uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> 16) & 1
    return ((b + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def draw_f32(wl, chunk, step, tensor_id, shape):
    """Float32 draw of one tensor of workload ``wl``."""
    rng = rng_for(wl.seed, chunk, step, tensor_id)
    if wl.dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if wl.dist == "normal_t4_2pct":
        x = rng.standard_normal(shape, dtype=np.float32)
        mask = rng.random(shape, dtype=np.float32) < 0.02
        x[mask] = rng.standard_t(4, size=int(mask.sum())).astype(np.float32)
        return x
    if wl.dist == "t4_outlier_channels":
        x = rng.standard_t(4, size=shape).astype(np.float32)
        H, D = shape[0], shape[-1]
        ch_id = KCH_ID if tensor_id == K_ID else VCH_ID
        crng = rng_for(wl.seed, chunk, step, ch_id)
        for h in range(H):
            chans = crng.choice(D, 4, replace=False)
            x[h, ..., chans] *= np.float32(20.0)
        return x
    raise ValueError(wl.dist)


def draw_bf16(wl, chunk, step, tensor_id, n_tokens=None):
    """bf16 bit patterns [H, n_tokens, D] (default n_tokens = chunk tokens)."""
    n = wl.chunk_tokens if n_tokens is None else n_tokens
    shape = (wl.n_heads, n, wl.head_dim)
    return f32_to_bf16_bits(draw_f32(wl, chunk, step, tensor_id, shape))


def clean_chunk(wl, chunk):
    """K, V of the clean chunk ``chunk`` that is appended to the cache."""
    return (draw_bf16(wl, chunk, APPEND_STEP, K_ID), draw_bf16(wl, chunk, APPEND_STEP, V_ID))


def noisy_chunk(wl, chunk, step=0):
    """Q, K_own, V_own [H, n_q, D] of the noisy chunk ``chunk`` at denoising ``step``."""
    return (draw_bf16(wl, chunk, step, Q_ID, wl.n_q), draw_bf16(wl, chunk, step, K_ID, wl.n_q),
            draw_bf16(wl, chunk, step, V_ID, wl.n_q))


def attention_flops(n_heads, n_q, n_k, head_dim):
    """QK^T plus PV: 2 flops per multiply-add, 4 * H * Lq * Lk * D."""
    return 4.0 * n_heads * n_q * n_k * head_dim


def quantize_bytes(n_elements):
    """Algorithmic bytes of quantizing one tensor: 2 B read, 1/2 B of codes
    and 1/16 B of scale written per element, plus the 4-byte tensor scale."""
    return n_elements * (2.0 + 0.5 + 1.0 / 16.0) + 4.0


def quantize_bytes_mx(n_elements):
    """Algorithmic bytes of quantizing one tensor to MXFP4: 2 B read, 1/2 B of codes
    and 1/32 B of E8M0 scale written per element (no tensor scale)."""
    return n_elements * (2.0 + 0.5 + 1.0 / 32.0)


def device_seed(seed, chunk, step, tensor_id):
    """64-bit seed for a device-side generator, derived from the same
    (cfg_seed, chunk, step, tensor_id) key as the host draws."""
    return int(np.random.SeedSequence([seed, chunk, step, tensor_id]).generate_state(1, np.uint64)[0]
               & np.uint64(0x7FFFFFFFFFFFFFFF))


def draw_device_normal(wl, chunk, step, tensor_id, device, n_tokens=None):
    """N(0,1) bf16 draw made on the device with torch's seeded generator (used
    for the long streaming workload, whose hundreds of tensors would take
    minutes to draw on the host).  Returns an int16 tensor of bf16 bits."""
    import torch
    n = wl.chunk_tokens if n_tokens is None else n_tokens
    g = torch.Generator(device=device)
    g.manual_seed(device_seed(wl.seed, chunk, step, tensor_id))
    x = torch.randn((wl.n_heads, n, wl.head_dim), generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16).view(torch.int16)
