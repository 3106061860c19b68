"""MI355X-native forward pass of one expert-specialised MoE layer.

The compute lives in ``libmoe.so`` (hand-written HIP kernels for gfx950 behind a C ABI,
declared in ``include/moe.h``).  ``gemm_gate_softmax_amd.ops`` is the thin ctypes binding
over it; importing this package does not load the library, calling an op does, and fails
loudly if it has not been built.
"""
import importlib

from . import workloads  # noqa: F401

__all__ = ["workloads", "ops"]


def __getattr__(name):
    if name == "ops":
        return importlib.import_module(".ops", __name__)
    raise AttributeError(name)
