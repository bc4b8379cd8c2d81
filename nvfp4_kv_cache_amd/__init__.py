"""MI355X-native NVFP4 KV-cache chunk attention.

The compute path is the HIP library ``libnvfp4kv.so`` (C ABI declared in
``include/nvfp4kv.h``); ``nvfp4_kv_cache_amd.ops`` is its thin ctypes binding.
``nvfp4_kv_cache_amd.workloads`` holds the seeded synthetic inputs only.
"""

import importlib

__all__ = ["ops", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
