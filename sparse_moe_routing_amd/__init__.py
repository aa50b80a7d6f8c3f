"""MI355X-native sparse mixture-of-experts layer: router GEMV, exact top-8 under a total order,
softmax over the selected eight, sigmoid-gated shared expert, SwiGLU experts and the weighted
combine, behind the C-ABI library ``libmoe.so`` (header ``include/moe.h``).

``inputs`` (seeded synthetic workloads) needs only numpy; ``binding`` loads ``libmoe.so`` on
first use and raises if it has not been built.
"""
from . import binding, inputs  # noqa: F401

__all__ = ["binding", "inputs"]
