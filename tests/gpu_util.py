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


def check_attention(got, want, what="", v_scale=1.0):
    """The parity bar.  `v_scale` (>= 1 counts) is the RMS of the V values for draws
    that are not unit-scale: the output is linear in V, so its rounding errors scale
    with V and the max-abs bar is applied to the output in units of v_scale."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    max_abs = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    print(f"[{what}] max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)
    bar = MAX_ABS * max(1.0, float(v_scale))
    assert max_abs <= bar, f"{what}: max abs error {max_abs} (bar {bar:.3e})"
    assert rel <= REL_L2, f"{what}: relative L2 error {rel}"
    return max_abs, rel
