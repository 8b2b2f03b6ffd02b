"""hyena_fwd_noalloc (workspace inside the library) against hyena_fwd (caller
workspace) on the same inputs, through the C ABI: three calls in a row on one
GPU, the first at the largest documented size, the later ones smaller, so the
later calls run over the contents the earlier ones left in the array.

Bar: max |y - y_ref| / max |y_ref| <= 1e-4 (fp32) or <= 2e-2 (bf16 storage)."""
import numpy as np
import pytest

from synth import make_1d, make_config
from tests.gpu_util import TOL, rel_err, say, to_dev

pytestmark = pytest.mark.gpu


def _both(inp):
    import torch
    import subquadratic_sequence_amd as hs
    dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    layer = hs.HyenaLayer(inp.L, inp.D, inp.N)
    hs.hyena_filter_gen(layer, to_dev(inp.w1), to_dev(inp.b1), to_dev(inp.w2), to_dev(inp.b2), to_dev(inp.w3),
                        to_dev(inp.b3), to_dev(inp.decay), inp.K)
    args = (to_dev(inp.u, dt), to_dev(inp.w_in, dt), to_dev(inp.short_w), to_dev(inp.dskip), to_dev(inp.w_out, dt))
    y_ref = hs.hyena_fwd(layer, *args)
    y = hs.hyena_fwd_noalloc(layer, *args)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), y_ref.float().cpu().numpy().astype(np.float64)


def test_noalloc_matches_hyena_fwd_on_calls_of_decreasing_size():
    cases = [make_config("order2_bf16_B8_L2k_D768"),                    # largest documented: LDS regime
             make_1d(91, 2, 16384, 128, N=2, K=16, dtype="bf16", u_scale=0.1),  # four-step regime, smaller
             make_1d(92, 1, 1024, 64, N=3, K=8, dtype="f32")]           # smallest, fp32
    for inp in cases:
        say(f"noalloc B={inp.B} L={inp.L} D={inp.D} N={inp.N} {inp.dtype}")
        y, y_ref = _both(inp)
        assert np.all(np.isfinite(y))
        err = rel_err(y, y_ref)
        say(f"  rel diff to hyena_fwd {err:.3e} (bit-identical: {np.array_equal(y, y_ref)})")
        assert err <= TOL[inp.dtype], err
