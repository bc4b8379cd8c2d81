"""CPU oracle for NVFP4 KV-cache chunk attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product package (``nvfp4_kv_cache_amd``) never imports it and shares no code,
tables or constants with it: the two meet only on the seeded inputs.

Contents (each function cites the passage of the pages it follows):

* ``nvfp4_ref``     -- E2M1 / E4M3 codecs, the NVFP4 quantizer and dequantizer,
  with the optional K-smoothing and adaptive 4/6 block scales.
* ``mxfp4_ref``     -- the MXFP4 quantizer and dequantizer (32-element blocks,
  E8M0 scales), the format the paper's appendix A.2 sets against NVFP4, and the
  MXFP8 (E4M3) query quantizer of the MX-scaled matrix-core variant.
* ``cache_ref``     -- sink + sliding-window frame list (the effective key set).
* ``attention_ref`` -- softmax attention of a noisy chunk over the dequantized
  cache plus its own bf16 K/V, in float64.

Pages cited: "LongLive-2.0: An NVFP4 Parallel Infrastructure for Long Video
Generation" -- the paper text (sections 2.1, 2.2, 3, 4.2) and the reading note
on it (section II, "The NVFP4 quantization format", "The inference
infrastructure", "Multi-shot attention sinks").
"""

from .nvfp4_ref import (  # noqa: F401
    E2M1_VALUES,
    E4M3_VALUES,
    bf16_bits_to_f32,
    e2m1_encode,
    e4m3_encode,
    quantize_ref,
    dequantize_ref,
    channel_mean_ref,
)
from .mxfp4_ref import mx_quantize_ref, mx_dequantize_ref, mxfp8_quantize_ref, mxfp8_dequantize_ref  # noqa: F401
from .cache_ref import CacheModel  # noqa: F401
from .attention_ref import chunk_attention_ref, attention_from_kv  # noqa: F401
