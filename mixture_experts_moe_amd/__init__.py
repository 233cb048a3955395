"""MI355X-native fused Mixture-of-Experts layer.

The compute lives in a HIP/gfx950 shared library (``libmoe.so``, built from
``csrc/``) behind a C ABI; ``binding`` is a thin ctypes layer over it.  The
library is loaded on first use, so importing this package (for example only
for ``synth``) needs no GPU.
"""

import importlib

__all__ = ["binding", "synth"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
