"""Backward pass at lengths past the 64k four-step layout (N1 = 256 columns:
L = 2^17 with 1024-point rows, L = 2^20 with the 8192-point sequential row
pass), where the fp64 backward oracle takes minutes per case: a property that
holds at any size instead of element-wise parity.

For every input and parameter P of the layer, the gradient g_P that hyena_bwd
(and, for the filter generator's parameters, hyena_filter_bwd on its dh)
returns must give the directional derivative of phi = sum(dy * y) along a
random direction V:  <g_P, V> = d/de phi(P + e V) at e = 0, which the test
takes as a central difference of two hyena_fwd calls (through the C ABI).
phi is a polynomial of degree at most three in each P but the generator's
hidden weights w2 (the operator is a product of projections, linear in each
filter and in the generator's last layer; w2 enters through sines), so the
central difference of step e is exact up to e^2 |phi'''| / 6, far below the
bar at e = 1e-2 of P's scale; fp32 storage keeps the rounding noise of the two
forwards small. A kernel that computes the wrong thing gives an error of order
one.

Bar: |FD - <g_P, V>| <= 5e-3 max(|<g_P, V>|, |FD|) (measured: at most 6.2e-4)."""
import numpy as np
import pytest

from synth import make_1d
from tests.gpu_util import say, to_dev

pytestmark = pytest.mark.gpu

BAR = 5e-3
EPS = 1e-2


def _phi(hs, torch, layer, t, dy, fp, K):
    hs.hyena_filter_gen(layer, *fp, K)
    y = hs.hyena_fwd(layer, t["u"], t["w_in"], t["short_w"], t["dskip"], t["w_out"])
    return float(torch.sum(dy.double() * y.double()))


@pytest.mark.parametrize("L,N,causal", [(1 << 17, 2, True), (1 << 20, 1, True), (1 << 17, 2, False)])
def test_bwd_directional_derivatives(L, N, causal):
    import torch
    import subquadratic_sequence_amd as hs
    inp = make_1d(790 + L // 4096 + N, 1, L, 64, N=N, K=8, dtype="f32", causal=causal)
    say(f"bwd adjoint case B=1 L={L} D=64 N={N} f32 causal={causal} seed={inp.meta['seed']}")
    rng = np.random.default_rng(17)
    layer = hs.HyenaLayer(inp.L, inp.D, inp.N, direction=hs.CAUSAL if causal else hs.NONCAUSAL)
    t = {k: to_dev(getattr(inp, k)) for k in ("u", "w_in", "short_w", "dskip", "w_out")}
    fnames = ("w1", "b1", "w2", "b2", "w3", "b3", "decay")
    fp = [to_dev(getattr(inp, k)) for k in fnames]
    dy = to_dev(rng.standard_normal((1, L, 64)).astype(np.float32))
    hs.hyena_filter_gen(layer, *fp, inp.K)
    g = hs.hyena_bwd(layer, t["u"], t["w_in"], t["short_w"], t["dskip"], t["w_out"], dy)
    gf = hs.hyena_filter_bwd(layer, *fp, inp.K, g["dh"])
    torch.cuda.synchronize()
    grads = {"u": g["du"], "w_in": g["dw_in"], "short_w": g["dshort_w"], "dskip": g["ddskip"],
             "w_out": g["dw_out"], "w3": gf["w3"], "w2": gf["w2"]}
    for name, grad in grads.items():
        base = t[name] if name in t else fp[fnames.index(name)]
        v = to_dev(rng.standard_normal(tuple(base.shape)).astype(np.float32))
        step = EPS * float(base.float().pow(2).mean().sqrt())
        ad = float(torch.sum(grad.double() * v.double())) * step

        def at(e):
            pt = dict(t)
            pf = list(fp)
            if name in t:
                pt[name] = (base.double() + e * v.double()).float()
            else:
                pf[fnames.index(name)] = (base.double() + e * v.double()).float()
            return _phi(hs, torch, layer, pt, dy, pf, inp.K)

        fd = (at(step) - at(-step)) / 2.0
        err = abs(fd - ad) / max(abs(ad), abs(fd), 1e-30)
        say(f"  {name:8s} <g, V> step {ad:+.6e}  central difference {fd:+.6e}  rel {err:.2e}")
        assert err <= BAR, (name, ad, fd, err)
    hs.hyena_filter_gen(layer, *fp, inp.K)  # leave the layer as generated from the drawn parameters
