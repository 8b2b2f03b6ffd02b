"""The stage-event entry points (hyena_fwd_profiled, hyena_nd_fwd_profiled,
hyena_nd_film_fwd_profiled) run the same launches as the plain ones: identical
outputs, and events (four; five for the register-conditioned layer) that bracket
the stages in order."""
import numpy as np
import pytest

from tests.gpu_util import say, to_dev
from synth import make_1d, make_nd

pytestmark = pytest.mark.gpu


def _events(torch):
    return [torch.cuda.Event(enable_timing=True) for _ in range(4)]


def _check_events(evs):
    t = [evs[0].elapsed_time(evs[i]) for i in range(1, 4)]
    assert all(x >= 0 for x in t) and t[0] <= t[1] <= t[2], t


@pytest.mark.parametrize("L,dt", [(1024, "f32"), (16384, "bf16")])
def test_fwd_profiled_matches_fwd(L, dt):
    import torch
    import subquadratic_sequence_amd as hs
    inp = make_1d(41 + L, 2, L, 64, N=2, K=8, dtype=dt)
    say(f"case profiled 1D B=2 L={L} D=64 dtype={dt}")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    layer = hs.HyenaLayer(inp.L, inp.D, inp.N)
    hs.hyena_filter_gen(layer, to_dev(inp.w1), to_dev(inp.b1), to_dev(inp.w2), to_dev(inp.b2), to_dev(inp.w3),
                        to_dev(inp.b3), to_dev(inp.decay), inp.K)
    u, w_in, w_out = to_dev(inp.u, tdt), to_dev(inp.w_in, tdt), to_dev(inp.w_out, tdt)
    short_w, dskip = to_dev(inp.short_w), to_dev(inp.dskip)
    y0 = hs.hyena_fwd(layer, u, w_in, short_w, dskip, w_out)
    y1 = torch.empty_like(y0)
    ws = torch.empty(hs.hyena_workspace_bytes(inp.B, inp.L, inp.D, inp.N, hs.HYENA_BF16 if dt == "bf16" else
                                              hs.HYENA_F32), dtype=torch.uint8, device="cuda")
    evs = _events(torch)
    hs.hyena_fwd_profiled(layer, u, w_in, short_w, dskip, w_out, y1, ws, evs)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    _check_events(evs)


@pytest.mark.parametrize("X,Y,circ", [(8, 8, False), (16, 16, True), (1, 32, False), (1, 32, True)])
def test_nd_fwd_profiled_matches_nd_fwd(X, Y, circ):
    import torch
    import subquadratic_sequence_amd as hs
    inp = make_nd(43 + X + Y, 2, X, Y, Y, 64, N=2, circular=circ)
    say(f"case profiled ND B=2 grid {X}x{Y}x{Y} C=64 circular={circ}")
    bd = hs.ND_CIRCULAR if circ else hs.ND_ZERO_PAD
    layer = hs.HyenaNDLayer(inp.X, inp.Y, inp.Z, inp.C, inp.N, boundary=bd)
    hs.hyena_nd_filter_gen(layer, to_dev(inp.w1), to_dev(inp.b1), to_dev(inp.w2), to_dev(inp.b2), to_dev(inp.w3),
                           to_dev(inp.b3), to_dev(inp.decay))
    u, w_in, dskip, ga, gb, w_out = (to_dev(a) for a in (inp.u, inp.w_in, inp.dskip, inp.gate_a, inp.gate_b,
                                                          inp.w_out))
    y0 = hs.hyena_nd_fwd(layer, u, w_in, dskip, ga, gb, w_out)
    y1 = torch.empty_like(y0)
    ws = torch.empty(hs.hyena_nd_workspace_bytes_ex(inp.B, inp.X, inp.Y, inp.Z, inp.C, inp.N, bd), dtype=torch.uint8,
                     device="cuda")
    evs = _events(torch)
    hs.hyena_nd_fwd_profiled(layer, u, w_in, dskip, ga, gb, w_out, y1, ws, evs)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    assert np.isfinite(y1.cpu().numpy()).all()
    _check_events(evs)


@pytest.mark.parametrize("X,circ", [(8, False), (1, True)])
def test_nd_film_fwd_profiled_matches_film_fwd(X, circ):
    import torch
    import subquadratic_sequence_amd as hs
    from synth import make_nd_film
    inp = make_nd_film(47 + X, 3, X, 16, 16, 64, N=2, W=64, circular=circ)
    say(f"case profiled film B=3 grid {X}x16x16 C=64 circular={circ}")
    bd = hs.ND_CIRCULAR if circ else hs.ND_ZERO_PAD
    m = hs.HyenaNDFilm(inp.X, inp.Y, inp.Z, inp.C, inp.N, bd, *(to_dev(a) for a in (
        inp.w1, inp.b1, inp.w2, inp.b2, inp.w3, inp.b3, inp.window, inp.q, inp.film_w, inp.film_b, inp.omega0)))
    u, reg, w_in, dskip, w_out = (to_dev(a) for a in (inp.u, inp.reg, inp.w_in, inp.dskip, inp.w_out))
    y0 = hs.hyena_nd_film_fwd(m, u, reg, w_in, dskip, w_out)
    y1 = torch.empty_like(y0)
    ws = torch.empty(hs.hyena_nd_film_workspace_bytes(inp.B, inp.X, inp.Y, inp.Z, inp.C, inp.N, inp.W, bd),
                     dtype=torch.uint8, device="cuda")
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    hs.hyena_nd_film_fwd_profiled(m, u, reg, w_in, dskip, w_out, y1, ws, evs)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    t = [evs[0].elapsed_time(evs[i]) for i in range(1, 5)]
    assert all(x >= 0 for x in t) and t[0] <= t[1] <= t[2] <= t[3], t
