"""DCNv4 spatial-aggregation forward for AMD Instinct MI355X (gfx950).

The operator runs in hand-written HIP kernels behind the C ABI declared in
include/dcnv4.h (libdcnv4.so); this package is the thin Python binding
(argument marshalling only, torch for device memory and streams).
"""
__version__ = "0.1.0"


def forward(*args, **kwargs):
    from .binding import forward as _forward
    return _forward(*args, **kwargs)
