"""Chunk attention oracle in float64 (test infrastructure).

Paper text, section 2.1 "Sequence-Parallel AR Training": a noisy chunk attends
to the clean history before it and to its own noisy tokens.  Paper text,
section 4.2: at inference the history is the sink + window cache.  Paper text,
section 1 and reading note "The inference infrastructure": the NVFP4 cache is
dequantized for the attention computation.

Definition used: for each head h,
    K = [dequant(cache K) ; K_own],  V = [dequant(cache V) ; V_own]
    O = softmax(Q K^T * softmax_scale) V
with no mask (every query sees every cache key and every key of its own
chunk).  Everything is float64; the bf16 inputs and the dequantized cache are
exact in float64.  The row maximum is subtracted before exp, which leaves the
softmax unchanged.
"""

import numpy as np

from .nvfp4_ref import bf16_bits_to_f32


def attention_from_kv(q64, k64, v64, softmax_scale, rows=None, block=1024):
    """softmax(q k^T s) v per head, float64.  q64 [H, Lq, D], k64/v64
    [H, Lk, D].  ``rows`` (optional int array) restricts the query rows.
    Returns [H, len(rows) or Lq, D]."""
    H = q64.shape[0]
    if rows is not None:
        q64 = q64[:, rows]
    Lq, D = q64.shape[1], q64.shape[2]
    out = np.empty((H, Lq, D), dtype=np.float64)
    for h in range(H):
        kt = np.ascontiguousarray(k64[h].T)
        for r0 in range(0, Lq, block):
            s = (q64[h, r0:r0 + block] @ kt) * float(softmax_scale)
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[h, r0:r0 + block] = p @ v64[h]
    return out


def chunk_attention_ref(q_bits, k_own_bits, v_own_bits, cache_k64, cache_v64,
                        softmax_scale, rows=None, q_cache64=None):
    """Noisy-chunk attention over the dequantized cache plus the chunk's own
    bf16 K/V.  q/k_own/v_own: uint16 bf16 bits [H, n_q, D].  cache_k64 /
    cache_v64: float64 [H, n_cache, D] (e.g. ``CacheModel.dequantized_kv()``).
    q_cache64 (optional, float64 [H, n_q, D]): the queries the cache logits are
    computed from (e.g. dequantized MXFP8 queries), the own-key logits keeping the
    bf16 queries; one softmax over both.
    Returns float64 [H, n_q or len(rows), D]."""
    q64 = bf16_bits_to_f32(q_bits).astype(np.float64)
    ko = bf16_bits_to_f32(k_own_bits).astype(np.float64)
    vo = bf16_bits_to_f32(v_own_bits).astype(np.float64)
    if q_cache64 is None:
        k64 = np.concatenate([cache_k64, ko], axis=1)
        v64 = np.concatenate([cache_v64, vo], axis=1)
        return attention_from_kv(q64, k64, v64, softmax_scale, rows=rows)
    qc = np.asarray(q_cache64, dtype=np.float64)
    if rows is not None:
        q64, qc = q64[:, rows], qc[:, rows]
    H, Lq, D = q64.shape
    out = np.empty((H, Lq, D), dtype=np.float64)
    for h in range(H):
        s = np.concatenate([qc[h] @ cache_k64[h].T, q64[h] @ ko[h].T], axis=1) * float(softmax_scale)
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[h] = p @ np.concatenate([cache_v64[h], vo[h]], axis=0)
    return out
