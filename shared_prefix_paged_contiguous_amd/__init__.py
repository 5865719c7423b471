"""Shared-prefix decode attention for MI355X (gfx950): HOT contiguous prefix
pool, token-level COLD suffix pool, cascade / dense MFMA prefix kernels, a
gather suffix kernel and a log-sum-exp merge behind a per-step dispatcher.

The product is libgkv.so (C ABI in include/gkv.h, HIP kernels in csrc/);
``binding`` is its thin ctypes binding.
"""

from .binding import (  # noqa: F401
    BACKEND_AUTO,
    BACKEND_CASCADE,
    BACKEND_DENSE,
    BACKEND_NAMES,
    Context,
    GkvError,
    NoSpace,
    NotFound,
    default_m_sat,
    load_library,
)
