"""Plain, slow, fp64 CPU oracle for the Hyena forward operator and its 3D variant.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or run anything in this package. The product path
(subquadratic_sequence_amd) never imports it and shares no code with it.
"""
from .hyena_oracle import (  # noqa: F401
    fft_radix2,
    causal_conv_direct,
    causal_conv_fft,
    noncausal_conv_direct,
    noncausal_conv_fft,
    posenc,
    posenc_at,
    implicit_filter,
    implicit_filter_noncausal,
    short_conv,
    hyena_fwd,
    hyena_fwd_sampled,
)
from .hyena_nd_oracle import (  # noqa: F401
    fftn3_radix2,
    nd_offsets,
    nd_filter,
    nd_gate,
    conv3d_direct,
    conv3d_fft,
    conv3d_circular_direct,
    conv3d_circular_fft,
    hyena_nd_fwd,
    hyena_nd_fwd_sampled,
)
from .hyena_nd_film_oracle import (  # noqa: F401
    film_control,
    film_modulation,
    nd_filter_film,
    film_kernels,
    hyena_nd_film_fwd,
    hyena_nd_film_fwd_sampled,
)
from .hyena_bwd_oracle import (  # noqa: F401
    causal_corr_direct,
    causal_corr_fft,
    causal_xcorr_direct,
    causal_xcorr_fft,
    noncausal_corr_direct,
    noncausal_corr_fft,
    noncausal_xcorr_direct,
    noncausal_xcorr_fft,
    short_conv_bwd,
    hyena_bwd,
    implicit_filter_bwd,
    implicit_filter_noncausal_bwd,
)
