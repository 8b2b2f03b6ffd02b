"""Pins of the backward oracle (oracle/hyena_bwd_oracle.py) against things
other than itself: numpy.correlate for the transposed convolutions, the
adjoint identities that tie them to the pinned forward convolutions, and
central finite differences of the pinned forward oracle for every gradient
(the backward is the derivative of the operator whose training cost the pages
discuss: Hyena Hierarchy and HyenaDNA abstracts)."""
import numpy as np
import pytest

import oracle
import oracle.hyena_bwd_oracle as bwd_mod
from synth import make_1d

RNG = np.random.default_rng(97531)


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ------------------------------------------------------------ correlations

@pytest.mark.parametrize("L", [1, 2, 7, 64])
def test_causal_correlations_match_numpy_correlate(L):
    h, g, z = RNG.standard_normal((3, L))
    full_gh = np.correlate(g, h, "full")            # c[k'] = sum_n g[n + k] h[n], k = k' - (L - 1)
    assert rel(oracle.causal_corr_direct(h, g), full_gh[L - 1:]) < 1e-13
    full_gz = np.correlate(g, z, "full")
    assert rel(oracle.causal_xcorr_direct(g, z), full_gz[L - 1:]) < 1e-13


@pytest.mark.parametrize("L", [1, 2, 5, 33])
def test_noncausal_correlations_match_numpy_correlate(L):
    h2 = RNG.standard_normal(2 * L - 1)
    g, z = RNG.standard_normal((2, L))
    assert rel(oracle.noncausal_corr_direct(h2, g), np.correlate(g, h2, "full")[L - 1:2 * L - 1]) < 1e-13
    assert rel(oracle.noncausal_xcorr_direct(g, z), np.correlate(g, z, "full")) < 1e-13


@pytest.mark.parametrize("L", [1, 2, 16, 128, 1024])
def test_correlation_fft_paths_equal_direct(L):
    h = RNG.standard_normal((2, L))
    h2 = RNG.standard_normal((2, 2 * L - 1))
    g, z = RNG.standard_normal((2, 3, 2, L))
    assert rel(oracle.causal_corr_fft(h, g), oracle.causal_corr_direct(h, g)) < 1e-11
    assert rel(oracle.causal_xcorr_fft(g, z), oracle.causal_xcorr_direct(g, z)) < 1e-11
    assert rel(oracle.noncausal_corr_fft(h2, g), oracle.noncausal_corr_direct(h2, g)) < 1e-11
    assert rel(oracle.noncausal_xcorr_fft(g, z), oracle.noncausal_xcorr_direct(g, z)) < 1e-11


@pytest.mark.parametrize("L", [3, 40])
def test_adjoint_identities_with_the_forward_convolution(L):
    # <corr(h, g), z> = <g, conv(h, z)> and <xcorr(g, z), h> = <g, conv(h, z)>
    h, g, z = RNG.standard_normal((3, L))
    fwd = np.dot(g, oracle.causal_conv_direct(h, z))
    assert abs(np.dot(oracle.causal_corr_direct(h, g), z) - fwd) < 1e-11 * (1 + abs(fwd))
    assert abs(np.dot(oracle.causal_xcorr_direct(g, z), h) - fwd) < 1e-11 * (1 + abs(fwd))
    h2 = RNG.standard_normal(2 * L - 1)
    fwd2 = np.dot(g, oracle.noncausal_conv_direct(h2, z))
    assert abs(np.dot(oracle.noncausal_corr_direct(h2, g), z) - fwd2) < 1e-11 * (1 + abs(fwd2))
    assert abs(np.dot(oracle.noncausal_xcorr_direct(g, z), h2) - fwd2) < 1e-11 * (1 + abs(fwd2))


# ------------------------------------------------------- finite differences

def _loss(inp, h0, dy, causal, **over):
    a = dict(u=inp.u, w_in=inp.w_in, short_w=inp.short_w, dskip=inp.dskip, w_out=inp.w_out, h=h0)
    a.update(over)
    y = oracle.hyena_fwd(a["u"], a["w_in"], a["short_w"], a["dskip"], a["w_out"], a["h"], conv="direct",
                         causal=causal)
    return float(np.sum(dy * y))


def _check_fd(inp, h, causal, eps=1e-6):
    dy = RNG.standard_normal((inp.B, inp.L, inp.D))
    gr = oracle.hyena_bwd(inp.u, inp.w_in, inp.short_w, inp.dskip, inp.w_out, h, dy, conv="direct", causal=causal)
    base = dict(u=inp.u, w_in=inp.w_in, short_w=inp.short_w, dskip=inp.dskip, w_out=inp.w_out, h=h)
    for key, gkey in [("u", "du"), ("w_in", "dw_in"), ("short_w", "dshort_w"), ("dskip", "ddskip"),
                      ("w_out", "dw_out"), ("h", "dh")]:
        x0 = np.asarray(base[key], np.float64)
        d = RNG.standard_normal(x0.shape)
        fp = _loss(inp, h, dy, causal, **{key: x0 + eps * d})
        fm = _loss(inp, h, dy, causal, **{key: x0 - eps * d})
        want = (fp - fm) / (2 * eps)
        got = float(np.sum(gr[gkey] * d))
        assert gr[gkey].shape == x0.shape, key
        assert abs(got - want) <= 1e-6 * (1 + abs(want)), (key, got, want)
    return gr


@pytest.mark.parametrize("N", [1, 2, 3])
def test_hyena_bwd_matches_finite_differences_causal(N):
    inp = make_1d(60 + N, 2, 24, 4, N=N, K=4, W=8)
    h = oracle.implicit_filter(inp.filter_params, inp.L, N, inp.D)
    _check_fd(inp, h, True)


def test_hyena_bwd_matches_finite_differences_noncausal():
    inp = make_1d(64, 2, 20, 4, N=2, K=4, W=8, causal=False)
    h2 = oracle.implicit_filter_noncausal(inp.filter_params, inp.L, 2, inp.D)
    _check_fd(inp, h2, False)


def test_hyena_bwd_single_entry_finite_difference():
    # one entry of du and of dh by a coordinate perturbation
    inp = make_1d(65, 1, 16, 4, N=2, K=4, W=8)
    h = oracle.implicit_filter(inp.filter_params, inp.L, 2, inp.D)
    dy = RNG.standard_normal((1, 16, 4))
    gr = oracle.hyena_bwd(inp.u, inp.w_in, inp.short_w, inp.dskip, inp.w_out, h, dy)
    eps = 1e-6
    u = inp.u.astype(np.float64)
    e = np.zeros_like(u)
    e[0, 5, 2] = eps
    fd = (_loss(inp, h, dy, True, u=u + e) - _loss(inp, h, dy, True, u=u - e)) / (2 * eps)
    assert abs(gr["du"][0, 5, 2] - fd) < 1e-7 * (1 + abs(fd))
    e = np.zeros_like(h)
    e[1, 3, 7] = eps
    fd = (_loss(inp, h, dy, True, h=h + e) - _loss(inp, h, dy, True, h=h - e)) / (2 * eps)
    assert abs(gr["dh"][1, 3, 7] - fd) < 1e-7 * (1 + abs(fd))


def test_hyena_bwd_fft_equals_direct_and_causal_structure():
    inp = make_1d(66, 2, 64, 8, N=2, K=4, W=8)
    h = oracle.implicit_filter(inp.filter_params, inp.L, 2, inp.D)
    dy = RNG.standard_normal((2, 64, 8))
    a = oracle.hyena_bwd(inp.u, inp.w_in, inp.short_w, inp.dskip, inp.w_out, h, dy, conv="direct")
    b = oracle.hyena_bwd(inp.u, inp.w_in, inp.short_w, inp.dskip, inp.w_out, h, dy, conv="fft")
    for k in a:
        assert rel(b[k], a[k]) < 1e-10, k
    # causality, transposed: y_t reads u_{<= t}, so du_s collects dy_{>= s} only;
    # with dy zero from t = 40 on, du is exactly zero there
    dy2 = dy.copy()
    dy2[:, 40:] = 0.0
    c = oracle.hyena_bwd(inp.u, inp.w_in, inp.short_w, inp.dskip, inp.w_out, h, dy2, conv="direct")
    assert np.all(c["du"][:, 40:] == 0.0)


def test_hyena_bwd_is_linear_in_dy():
    inp = make_1d(67, 2, 32, 4, N=2, K=4, W=8)
    h = oracle.implicit_filter(inp.filter_params, inp.L, 2, inp.D)
    d1, d2 = RNG.standard_normal((2, 2, 32, 4))
    g1 = oracle.hyena_bwd(inp.u, inp.w_in, inp.short_w, inp.dskip, inp.w_out, h, d1)
    g2 = oracle.hyena_bwd(inp.u, inp.w_in, inp.short_w, inp.dskip, inp.w_out, h, d2)
    g3 = oracle.hyena_bwd(inp.u, inp.w_in, inp.short_w, inp.dskip, inp.w_out, h, d1 - 2.5 * d2)
    for k in g1:
        assert rel(g3[k], g1[k] - 2.5 * g2[k]) < 1e-11, k


@pytest.mark.parametrize("causal", [True, False])
def test_filter_bwd_matches_finite_differences(causal):
    L, N, D = 24, 2, 4
    inp = make_1d(68, 1, L, D, N=N, K=4, W=8)
    p = {k: np.asarray(v, np.float64) if k != "K" else v for k, v in inp.filter_params.items()}
    gen = oracle.implicit_filter if causal else oracle.implicit_filter_noncausal
    bwd = oracle.implicit_filter_bwd if causal else oracle.implicit_filter_noncausal_bwd
    dh = RNG.standard_normal(gen(p, L, N, D).shape)
    gr = bwd(p, L, N, D, dh)
    eps = 1e-6
    for key in ["w1", "b1", "w2", "b2", "w3", "b3", "decay"]:
        d = RNG.standard_normal(p[key].shape)
        pp, pm = dict(p), dict(p)
        pp[key] = p[key] + eps * d
        pm[key] = p[key] - eps * d
        want = (np.sum(dh * gen(pp, L, N, D)) - np.sum(dh * gen(pm, L, N, D))) / (2 * eps)
        got = float(np.sum(gr[key] * d))
        assert gr[key].shape == p[key].shape, key
        assert abs(got - want) <= 1e-6 * (1 + abs(want)), (key, got, want)


def test_planted_transpose_mistakes_fail_the_finite_difference_pin(monkeypatch):
    # the forward convolution in place of its transpose, or a cross-correlation
    # with its operands swapped, each fails
    inp = make_1d(69, 1, 12, 4, N=2, K=4, W=8)
    h = oracle.implicit_filter(inp.filter_params, inp.L, 2, inp.D)
    for name, wrong in [("causal_corr_direct", oracle.causal_conv_direct),
                        ("causal_xcorr_direct", lambda g, z: oracle.causal_xcorr_direct(z, g))]:
        with monkeypatch.context() as m:
            m.setattr(bwd_mod, name, wrong)
            with pytest.raises(AssertionError):
                _check_fd(inp, h, True)
