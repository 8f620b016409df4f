"""MI355X-native BitNet b1.58 BitLinear (ternary weights, int8 activations).

The compute path is the HIP library ``libbitnet.so`` built from ``csrc/``
(C ABI declared in ``include/bitnet.h``). ``binding`` wraps its entry points
with the same names; ``layer`` adds the autograd function and the
``QATBitLinear`` module, ``ttq_layer`` the same for the TTQ variant
(``TTQLinear``). Submodules load lazily so that importing the package (e.g.
for ``workloads``) neither imports torch nor loads the library.
"""

import importlib

__all__ = ["binding", "layer", "ttq_layer", "workloads", "build"]


def __getattr__(name):
    if name in ("binding", "layer", "ttq_layer", "workloads", "build"):
        return importlib.import_module(f"{__name__}.{name}")
    if name in ("QATBitLinear", "BitLinearFunction"):
        return getattr(importlib.import_module(f"{__name__}.layer"), name)
    if name in ("TTQLinear", "TTQFunction"):
        return getattr(importlib.import_module(f"{__name__}.ttq_layer"), name)
    raise AttributeError(name)
