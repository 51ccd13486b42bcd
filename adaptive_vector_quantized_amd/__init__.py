"""AVQ-Attention forward pass on AMD MI355X (gfx950).

``assign_aggregate`` and ``attention_fwd`` are thin bindings of the two
entry points of libavq (include/avq.h); ``forward`` chains them.  ``gen``
draws seeded synthetic workloads.  Importing the bindings requires the built
library (``adaptive_vector_quantized_amd/libavq.so``); there is no fallback.
"""
from . import gen  # noqa: F401


def __getattr__(name):
    # the HIP binding is imported on first use so that ``gen`` works without it
    if name in ("assign_aggregate", "attention_fwd", "forward", "AvqError", "lib", "declared_symbols"):
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
