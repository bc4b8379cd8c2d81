"""NVFP4 against MXFP4 on the workload's value distributions, in the oracle: the
paper text's appendix A.2 credits NVFP4's finer 16-element blocks, E4M3 scales and
tensor scale with tracking local dynamic range better than MXFP4.  Both the
reconstruction error of K/V and the error of the chunk attention computed from the
dequantized cache (against the same attention over the unquantized bf16 K/V) must be
smaller with NVFP4.  The MXFP4 variant whose cache logits come from MXFP8 queries
(on the MX-scaled matrix cores) is compared too.  Run with -s to see the numbers."""

import numpy as np

from oracle import (chunk_attention_ref, dequantize_ref, mx_dequantize_ref, mx_quantize_ref, mxfp8_dequantize_ref,
                    mxfp8_quantize_ref, quantize_ref)
from oracle.nvfp4_ref import bf16_bits_to_f32
from nvfp4_kv_cache_amd import workloads as W


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def normal_with_outliers(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    m = rng.random(shape) < 0.02
    x[m] = rng.standard_t(4, size=int(m.sum())).astype(np.float32)
    return W.f32_to_bf16_bits(x)


def student_t_outlier_channels(rng, shape):
    H, T, D = shape
    x = rng.standard_t(4, size=shape).astype(np.float32)
    for h in range(H):
        x[h, :, rng.choice(D, 4, replace=False)] *= 20.0
    return W.f32_to_bf16_bits(x)


def test_nvfp4_tracks_range_better_than_mxfp4():
    rng = np.random.default_rng(7)
    H, T, D, n_q = 2, 768, 128, 96
    for name, draw in (("normal + 2% t(4) outliers", normal_with_outliers),
                       ("Student-t, 4 outlier channels x20", student_t_outlier_channels)):
        k, v = draw(rng, (H, T, D)), draw(rng, (H, T, D))
        q, ko, vo = (normal_with_outliers(rng, (H, n_q, D)) for _ in range(3))
        kf, vf = (bf16_bits_to_f32(t).astype(np.float64) for t in (k, v))
        k_nv, v_nv = dequantize_ref(*quantize_ref(k)), dequantize_ref(*quantize_ref(v))
        k_mx, v_mx = mx_dequantize_ref(*mx_quantize_ref(k)), mx_dequantize_ref(*mx_quantize_ref(v))
        exact = chunk_attention_ref(q, ko, vo, kf, vf, 1.0 / np.sqrt(D))
        o_nv = chunk_attention_ref(q, ko, vo, k_nv, v_nv, 1.0 / np.sqrt(D))
        o_mx = chunk_attention_ref(q, ko, vo, k_mx, v_mx, 1.0 / np.sqrt(D))
        # the MX-scaled-matrix-core variant: the cache logits from MXFP8 queries
        o_mxs = chunk_attention_ref(q, ko, vo, k_mx, v_mx, 1.0 / np.sqrt(D),
                                    q_cache64=mxfp8_dequantize_ref(*mxfp8_quantize_ref(q)))
        e = {"K nvfp4": rel_l2(k_nv, kf), "K mxfp4": rel_l2(k_mx, kf),
             "V nvfp4": rel_l2(v_nv, vf), "V mxfp4": rel_l2(v_mx, vf),
             "attention nvfp4": rel_l2(o_nv, exact), "attention mxfp4": rel_l2(o_mx, exact),
             "attention mxfp4 + MXFP8 queries": rel_l2(o_mxs, exact)}
        print(f"\n[{name}] relative L2 errors: " + ", ".join(f"{a} {b:.4f}" for a, b in e.items()))
        assert e["K nvfp4"] < e["K mxfp4"] and e["V nvfp4"] < e["V mxfp4"], name
        assert e["attention nvfp4"] < e["attention mxfp4"], name
        # quantizing the queries adds little to the cache format's own error
        assert e["attention mxfp4 + MXFP8 queries"] < 1.1 * e["attention mxfp4"], name
