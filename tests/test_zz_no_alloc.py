"""The allocation-free codec entry point (nvfp4_quantize_kv_noalloc, for callers that
cannot allocate): its output must be bit-identical to nvfp4_quantize_kv's (codes,
scale bytes, tensor scale) on consecutive calls that share the library's scratch
array, the later ones smaller, and equal to the oracle codec."""

import numpy as np
import pytest

from oracle import quantize_ref
from nvfp4_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops(gpu):
    from nvfp4_kv_cache_amd import ops as _ops
    return _ops


def test_noalloc_matches_workspace_entry_point(ops):
    import torch
    from gpu_util import dev, host
    assert ops.lib().nvfp4_quantize_noalloc_scratch_bytes() == 32768
    wl = W.WORKLOADS["quantize"]
    k, _ = W.clean_chunk(wl, 0)
    rng = np.random.default_rng(90)
    small = W.f32_to_bf16_bits((rng.standard_t(4, size=(3, 77, 64)) * 1e-3).astype(np.float32))
    odd = W.f32_to_bf16_bits(rng.standard_normal((1, 5, 16)).astype(np.float32) * 1e30)
    # two calls in a row, the second smaller; then a tiny one and the large one again
    for i, x in enumerate((k, small, odd, k)):
        print(f"[noalloc] call {i} shape {x.shape}", flush=True)
        xd = dev(x)
        want = ops.quantize_kv(xd)
        got = ops.quantize_kv_noalloc(xd)
        torch.cuda.synchronize()
        for g, w, what in zip(got, want, ("codes", "scales", "tensor scale")):
            assert np.array_equal(host(g), host(w)), f"call {i} {x.shape}: {what} differ"
        rc, rs, rt = quantize_ref(x)
        assert np.array_equal(host(got[0]), rc) and np.array_equal(host(got[1]), rs)
        assert host(got[2])[0] == rt


def test_noalloc_preallocated_outputs_and_errors(ops):
    import ctypes
    import torch
    from gpu_util import dev, host
    rng = np.random.default_rng(91)
    x = W.f32_to_bf16_bits(rng.standard_normal((2, 40, 128)).astype(np.float32))
    xd = dev(x)
    out = (torch.empty((2, 40, 64), dtype=torch.uint8, device="cuda"),
           torch.empty((2, 40, 8), dtype=torch.uint8, device="cuda"),
           torch.empty(1, dtype=torch.float32, device="cuda"))
    got = ops.quantize_kv_noalloc(xd, out=out)
    assert all(a is b for a, b in zip(got, out))
    rc, rs, rt = quantize_ref(x)
    assert np.array_equal(host(out[0]), rc) and np.array_equal(host(out[1]), rs) and host(out[2])[0] == rt
    L = ops.lib()
    p = ctypes.c_void_p(xd.data_ptr())
    o = ctypes.c_void_p(out[0].data_ptr())
    assert L.nvfp4_quantize_kv_noalloc(None, 2, 40, 128, o, o, o, None) == -1
    assert L.nvfp4_quantize_kv_noalloc(p, 2, 40, 120, o, o, o, None) == -1
