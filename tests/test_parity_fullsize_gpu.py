"""Every output of the full-length and full-grid workloads, at the narrowest
width the library takes (64 channels).

The kernels that only the long and large workloads launch (the bf16 four-step
passes at L = 64k, the 8192-point rows at L = 1M, the persistent plane and
pencil passes of zero-padded 64^3 grids, the periodic 128^3 grids, the
conditioned pencil pass at 64^3) depend on the length or the grid and the
storage type, not on the width; here they run at those lengths and grids and
the whole output is compared with the fp64 oracle, computed in a process pool
over channel shards.

Bar: max |y - y_ref| / max |y_ref| <= 2e-2 (bf16 storage) or <= 1e-4 (fp32)."""
import numpy as np
import pytest

from synth import make_config
from tests.gpu_util import TOL, gpu_1d, gpu_nd, gpu_nd_film, rel_err, say

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


def _workers():
    from oracle._pool import default_workers
    return default_workers()


@pytest.mark.parametrize("name", ["order2_bf16_L64k_D64", "order2_bf16_L64k_D64_noncausal",
                                  "order2_bf16_L1M_D64_dna"])
def test_full_length_1d_every_output(name):
    import oracle
    inp = make_config(name)
    say(f"full-length {name}: B={inp.B} L={inp.L} D={inp.D} causal={inp.causal} (oracle on {_workers()} procs)")
    if inp.causal:
        h = oracle.implicit_filter(inp.filter_params, inp.L, inp.N, inp.D)
    else:
        h = oracle.implicit_filter_noncausal(inp.filter_params, inp.L, inp.N, inp.D)
    ref = oracle.hyena_fwd(inp.u, inp.w_in, inp.short_w, inp.dskip, inp.w_out, h, conv="fft",
                           causal=inp.causal, workers=_workers())
    del h
    say("  oracle done; running the library")
    y = gpu_1d(inp)
    assert np.all(np.isfinite(y))
    err = rel_err(y, ref)
    say(f"  rel err over all {y.size} outputs: {err:.3e}")
    assert err <= TOL[inp.dtype], err


@pytest.mark.parametrize("name", ["nd3d_f32_B2_C64_64cube", "nd3d_f32_B1_C64_64cube", "nd3d_circ_f32_B1_C64_128cube"])
def test_full_grid_nd_every_output(name):
    import oracle
    inp = make_config(name)
    say(f"full-grid {name}: B={inp.B} {inp.X}x{inp.Y}x{inp.Z} C={inp.C} circular={inp.circular} "
        f"(oracle on {_workers()} procs)")
    K = oracle.nd_filter(inp.filter_params, inp.X, inp.Y, inp.Z, inp.N, inp.C, circular=inp.circular)
    ref = oracle.hyena_nd_fwd(inp.u, inp.w_in, inp.dskip, inp.gate_a, inp.gate_b, inp.w_out, K,
                              circular=inp.circular, workers=_workers())
    del K
    say("  oracle done; running the library")
    y = gpu_nd(inp)
    assert np.all(np.isfinite(y))
    err = rel_err(y, ref)
    say(f"  rel err over all {y.size} outputs: {err:.3e}")
    assert err <= TOL["f32"], err


@pytest.mark.parametrize("name", ["nd3d_film_f32_B1_C64_64cube", "nd3d_film_f32_B2_C64_64cube"])
def test_full_grid_film_every_output(name):
    import oracle
    inp = make_config(name)
    say(f"full-grid {name}: B={inp.B} {inp.X}^3 C={inp.C} (oracle on {_workers()} procs)")
    Ks = oracle.film_kernels(inp.film_filter_params, inp.reg, inp.q, inp.film_w, inp.film_b, inp.X, inp.Y,
                             inp.Z, inp.N, inp.C, inp.circular)
    ref = oracle.hyena_nd_film_fwd(inp.u, inp.w_in, inp.dskip, inp.w_out, Ks, circular=inp.circular,
                                   workers=_workers())
    del Ks
    say("  oracle done; running the library")
    y = gpu_nd_film(inp)
    assert np.all(np.isfinite(y))
    err = rel_err(y, ref)
    say(f"  rel err over all {y.size} outputs: {err:.3e}")
    assert err <= TOL["f32"], err
