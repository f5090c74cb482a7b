"""MI355X-native Mixture-of-Experts FFN layer forward.

The computation lives in ``libmoe.so`` (hand-written HIP kernels for gfx950 behind a
C ABI, declared in ``include/moe.h``); ``binding`` marshals torch tensors to it.
Importing this package loads nothing: the library is opened on first use and an error
is raised if it has not been built.
"""
from . import configs, inputs  # noqa: F401

__all__ = ["configs", "inputs"]
