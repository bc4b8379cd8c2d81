"""Helpers for the GPU parity tests (host <-> device copies, tolerance checks)."""

import numpy as np
import torch

MAX_ABS = 1e-2      # attention tolerance: max |gpu - oracle| over the compared outputs
REL_L2 = 5e-3       # and ||gpu - oracle||_2 / ||oracle||_2


def dev(bits):
    """numpy uint16 bf16 bits -> device int16 tensor holding the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")


def host(t):
    return t.detach().cpu().numpy()


def f32_bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def check_attention(got, want, what="", max_abs_bar=MAX_ABS):
    """The parity bar: max-abs <= max_abs_bar (1e-2 unless a test derives another, see
    bf16_p_bar) and relative L2 <= 5e-3, over every compared output."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    max_abs = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    print(f"[{what}] max_abs={max_abs:.3e} rel_l2={rel:.3e} (bar {max_abs_bar:.3e})", flush=True)
    assert max_abs <= max_abs_bar, f"{what}: max abs error {max_abs} (bar {max_abs_bar:.3e})"
    assert rel <= REL_L2, f"{what}: relative L2 error {rel}"
    return max_abs, rel


def bf16_round(x):
    """float64 -> the nearest bf16 value (8 significant bits, ties to even), as float64
    (normal range; no double rounding through float32)."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.round(m * 256.0) / 256.0, e)


def bf16_p_bar(q_bits, ko_bits, vo_bits, cache_k64, cache_v64, scale, want, q_cache64=None):
    """Max-abs bar for attention whose probabilities enter the PV product as bf16
    (the MXFP4 cache's tiles and the own segment): max(1e-2, 1.05 x the max-abs error
    of a float64 simulation in which P = exp(S - rowmax) is rounded to bf16 (nearest
    even) and the row sums are taken from the rounded P, everything else exact)."""
    from oracle.nvfp4_ref import bf16_bits_to_f32
    q = bf16_bits_to_f32(q_bits).astype(np.float64)
    qc = q if q_cache64 is None else np.asarray(q_cache64, dtype=np.float64)
    ko = bf16_bits_to_f32(ko_bits).astype(np.float64)
    vo = bf16_bits_to_f32(vo_bits).astype(np.float64)
    sim = np.empty_like(np.asarray(want, dtype=np.float64))
    for h in range(q.shape[0]):
        s = np.concatenate([qc[h] @ cache_k64[h].T, q[h] @ ko[h].T], axis=1) * float(scale)
        p = bf16_round(np.exp(s - s.max(axis=1, keepdims=True)))
        sim[h] = (p @ np.concatenate([cache_v64[h], vo[h]], axis=0)) / p.sum(axis=1, keepdims=True)
    sim_err = float(np.abs(sim - want).max()) if sim.size else 0.0
    return max(MAX_ABS, 1.05 * sim_err)
