"""MI355X-native forward path of the Hyena operator (1D) and its 3D variant.

The compute lives in libhyena.so (hand-written HIP kernels for gfx950 behind a C
ABI, declared in include/hyena.h); this package is a thin ctypes binding.
"""
from .hyena import (  # noqa: F401
    CAUSAL,
    NONCAUSAL,
    HYENA_BF16,
    HYENA_F32,
    HyenaError,
    HyenaLayer,
    HyenaNDFilm,
    HyenaNDLayer,
    LIB_PATH,
    ND_CIRCULAR,
    ND_ZERO_PAD,
    SIGNATURES,
    hyena_cache_bytes,
    hyena_filter_gen,
    hyena_filter_workspace_bytes,
    hyena_filter_workspace_bytes_ex,
    hyena_fwd,
    hyena_fwd_profiled,
    hyena_nd_cache_bytes,
    hyena_nd_cache_bytes_ex,
    hyena_nd_film_fwd,
    hyena_nd_film_fwd_profiled,
    hyena_nd_film_workspace_bytes,
    hyena_nd_filter_gen,
    hyena_nd_filter_workspace_bytes,
    hyena_nd_filter_workspace_bytes_ex,
    hyena_nd_fwd,
    hyena_nd_fwd_profiled,
    hyena_nd_workspace_bytes,
    hyena_nd_workspace_bytes_ex,
    hyena_workspace_bytes,
    lib,
)
