"""MI355X-native deterministic MoE layer step (Mixture-of-Kittens hot path).

The GPU work lives in the C-ABI library ``libmok.so`` (hand-written HIP for
gfx950, declared in include/mok.h). ``mixture_experts_layer_stable_amd.mok``
is the thin Python binding with the same entry-point names; it is imported
lazily so that ``mixture_experts_layer_stable_amd.inputs`` (seeded synthetic
workloads) can be used without a GPU.
"""

import importlib

__all__ = ["mok", "inputs"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(__name__ + "." + name)
    raise AttributeError(name)
