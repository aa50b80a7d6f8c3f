"""MI355X-native sparse mixture-of-experts layer: router GEMV, exact top-8 under a total order,
softmax over the selected eight, sigmoid-gated shared expert, SwiGLU experts and the weighted
combine, behind the C-ABI library ``libmoe.so`` (header ``include/moe.h``).

``inputs`` (seeded synthetic workloads) imports without the library; the binding loads
``libmoe.so`` on first use and raises if it is missing.
"""
from . import inputs  # noqa: F401

__all__ = ["inputs", "binding"]


def __getattr__(name):
    if name == "binding":
        from . import binding
        return binding
    raise AttributeError(name)
