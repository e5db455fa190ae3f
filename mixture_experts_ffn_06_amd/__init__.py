"""MI355X-native Mixture-of-Experts FFN layer forward (HIP, gfx950).

The layer runs in ``libmoe.so`` (C ABI in ``include/moe.h``); this package
holds its sources (``csrc/``), the build script (``build.py``) and a thin
ctypes binding (``_lib.py``) that passes torch tensors' device pointers and
the current stream.  torch is used for device memory and streams only.
"""
from ._lib import (BF16, F32, FP8_E4M3, GATE_SIGMOID, GATE_SOFTMAX,  # noqa: F401
                   MoeError, MoePlan, lib, strerror)
from .layer import MoeLayer  # noqa: F401
