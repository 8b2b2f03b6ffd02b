"""Closed-form pins of the filter networks' hidden layers.

The implicit filters are MLPs of the position (TWIML #690, 4:29) and the 3D
kernels coordinate MLPs with sine activations (HyenaND explainer, "Kernel
Synthesis", "Kernel Parameterization"). With weights that route a few named
features through a few named hidden units, every hidden activation reaches the
output, and the expected filter is evaluated scalar by scalar with math.sin,
math.cos and math.exp in pure Python: a dropped, doubled or swapped activation
in either hidden layer changes it.

The last tests plant such mistakes in the oracle's own module (its numpy handle
is swapped for one whose k-th sine call is wrong) and check that a pin fails.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.hyena_nd_film_oracle as film_mod
import oracle.hyena_nd_oracle as nd_mod
import oracle.hyena_oracle as od_mod

RNG = np.random.default_rng(2468)


# --------------------------------------------------------------------------- 1D

def _params_1d(K, W, N, D):
    """Weights with two live hidden units in each layer.

    Layer 1: unit 0 reads the cos_2 feature, unit 1 the sin_3 feature, unit 2
    the tau feature.  Layer 2: unit 0 reads units 0, 1, 2 of layer 1, unit 1
    reads unit 1 only.  Output j reads units 0 and 1 of layer 2.  Every other
    weight is zero; every bias is live.
    """
    F = 1 + 2 * K
    w1 = np.zeros((F, W))
    w1[2, 0] = 2.3            # cos(2 pi 2 tau)
    w1[K + 3, 1] = -1.9       # sin(2 pi 3 tau)
    w1[0, 2] = 3.1            # tau
    b1 = RNG.uniform(-1, 1, W)
    w2 = np.zeros((W, W))
    w2[0, 0], w2[1, 0], w2[2, 0] = 1.7, 0.8, -1.2
    w2[1, 1] = 2.6
    b2 = RNG.uniform(-1, 1, W)
    w3 = np.zeros((W, N * D))
    w3[0] = RNG.uniform(-1, 1, N * D)
    w3[1] = RNG.uniform(-1, 1, N * D)
    b3 = RNG.uniform(-0.5, 0.5, N * D)
    decay = np.linspace(0.7, 5.0, D)
    return dict(K=K, w1=w1, b1=b1, w2=w2, b2=b2, w3=w3, b3=b3, decay=decay)


def _filter_1d_scalar(p, tau, n, c, D):
    """exp(-a_c |tau|) * o(tau)[n D + c], evaluated unit by unit."""
    K = p["K"]
    b1, b2, w3, b3 = p["b1"], p["b2"], p["w3"], p["b3"]
    a10 = math.sin(2.3 * math.cos(2 * math.pi * 2 * tau) + b1[0])
    a11 = math.sin(-1.9 * math.sin(2 * math.pi * 3 * tau) + b1[1])
    a12 = math.sin(3.1 * tau + b1[2])
    a20 = math.sin(1.7 * a10 + 0.8 * a11 - 1.2 * a12 + b2[0])
    a21 = math.sin(2.6 * a11 + b2[1])
    # units >= 3 of layer 1 and >= 2 of layer 2 see only their biases and feed nothing
    j = n * D + c
    o = w3[0, j] * a20 + w3[1, j] * a21 + b3[j]
    assert K >= 3
    return math.exp(-p["decay"][c] * abs(tau)) * o


def _check_causal():
    L, K, W, N, D = 32, 4, 8, 2, 4
    p = _params_1d(K, W, N, D)
    h = oracle.implicit_filter(p, L, N, D)
    assert h.shape == (N, D, L)
    for n in range(N):
        for c in range(D):
            for t in range(L):
                want = _filter_1d_scalar(p, t / L, n, c, D)
                assert abs(h[n, c, t] - want) <= 1e-12 * (1 + abs(want)), (n, c, t)


def _check_noncausal():
    L, K, W, N, D = 16, 4, 8, 2, 4
    p = _params_1d(K, W, N, D)
    h2 = oracle.implicit_filter_noncausal(p, L, N, D)
    assert h2.shape == (N, D, 2 * L - 1)
    for n in range(N):
        for c in range(D):
            for i in range(2 * L - 1):
                tau = (i - (L - 1)) / L          # negative lags first
                want = _filter_1d_scalar(p, tau, n, c, D)
                assert abs(h2[n, c, i] - want) <= 1e-12 * (1 + abs(want)), (n, c, i)


def test_implicit_filter_hidden_layers_closed_form():
    _check_causal()


def test_implicit_filter_noncausal_hidden_layers_at_negative_lags():
    _check_noncausal()


# --------------------------------------------------------------------------- 3D

def _params_nd(W, N, C):
    """Layer 1: unit k reads coordinate axis k (x, y, z) with its own weight and
    bias.  Layer 2: unit 0 reads all three, unit 1 reads unit 2 only.  Output j
    reads units 0 and 1."""
    w1 = np.zeros((3, W))
    w1[0, 0], w1[1, 1], w1[2, 2] = 2.1, -1.4, 2.9
    b1 = RNG.uniform(-1, 1, W)
    w2 = np.zeros((W, W))
    w2[0, 0], w2[1, 0], w2[2, 0] = 1.3, -0.9, 0.7
    w2[2, 1] = 2.2
    b2 = RNG.uniform(-1, 1, W)
    w3 = np.zeros((W, N * C))
    w3[0] = RNG.uniform(-1, 1, N * C)
    w3[1] = RNG.uniform(-1, 1, N * C)
    b3 = RNG.uniform(-0.5, 0.5, N * C)
    decay = np.linspace(0.5, 4.0, C)
    return dict(w1=w1, b1=b1, w2=w2, b2=b2, w3=w3, b3=b3, decay=decay)


def _coord(i, M, G, circular):
    """Coordinate of index i on an axis of transform length M (offset i - M/2)."""
    h = G // 2 if circular else G
    return (i - M // 2) / h if h else 0.0


def _nd_unit_outputs(p, cx, cy, cz, mod=None, omega0=None):
    """(a2_0, a2_1) of the coordinate MLP at one point; with mod = (g1, be1, g2, be2)
    the FiLM form sin(omega g1 (pre) + be1), sin(g2 (pre) + be2)."""
    b1, b2 = p["b1"], p["b2"]
    pre1 = [2.1 * cx + b1[0], -1.4 * cy + b1[1], 2.9 * cz + b1[2]]
    if mod is None:
        a1 = [math.sin(v) for v in pre1]
        a20 = math.sin(1.3 * a1[0] - 0.9 * a1[1] + 0.7 * a1[2] + b2[0])
        a21 = math.sin(2.2 * a1[2] + b2[1])
    else:
        g1, be1, g2, be2 = mod
        a1 = [math.sin(omega0[k] * g1[k] * pre1[k] + be1[k]) for k in range(3)]
        a20 = math.sin(g2[0] * (1.3 * a1[0] - 0.9 * a1[1] + 0.7 * a1[2] + b2[0]) + be2[0])
        a21 = math.sin(g2[1] * (2.2 * a1[2] + b2[1]) + be2[1])
    return a20, a21


def _check_nd(circular, X=4, Y=2, Z=4):
    W, N, C = 8, 2, 3
    p = _params_nd(W, N, C)
    K = oracle.nd_filter(p, X, Y, Z, N, C, circular=circular)
    f = 1 if circular else 2
    MX, MY, MZ = f * X, f * Y, f * Z
    assert K.shape == (N, C, MX, MY, MZ)
    for i in range(MX):
        for j in range(MY):
            for k in range(MZ):
                cx, cy, cz = _coord(i, MX, X, circular), _coord(j, MY, Y, circular), _coord(k, MZ, Z, circular)
                a20, a21 = _nd_unit_outputs(p, cx, cy, cz)
                r = math.sqrt(cx * cx + cy * cy + cz * cz)
                for n in range(N):
                    for c in range(C):
                        jj = n * C + c
                        want = math.exp(-p["decay"][c] * r) * (p["w3"][0, jj] * a20 + p["w3"][1, jj] * a21
                                                               + p["b3"][jj])
                        assert abs(K[n, c, i, j, k] - want) <= 1e-12 * (1 + abs(want)), (i, j, k, n, c)


@pytest.mark.parametrize("circular", [False, True])
def test_nd_filter_hidden_layers_closed_form(circular):
    _check_nd(circular)


def _check_film(circular, X=4, Y=4, Z=2):
    W, N, C = 8, 2, 3
    p = _params_nd(W, N, C)
    window = np.linspace(0.3, 3.0, C)
    omega0 = RNG.uniform(0.5, 12.0, W)
    mod = np.stack([RNG.uniform(0.5, 1.5, W), RNG.uniform(-1, 1, W), RNG.uniform(0.5, 1.5, W),
                    RNG.uniform(-1, 1, W)])
    fp = dict(w1=p["w1"], b1=p["b1"], w2=p["w2"], b2=p["b2"], w3=p["w3"], b3=p["b3"], omega0=omega0,
              window=window)
    K = oracle.nd_filter_film(fp, mod, X, Y, Z, N, C, circular=circular)
    f = 1 if circular else 2
    MX, MY, MZ = f * X, f * Y, f * Z
    for i in range(MX):
        for j in range(MY):
            for k in range(MZ):
                cx, cy, cz = _coord(i, MX, X, circular), _coord(j, MY, Y, circular), _coord(k, MZ, Z, circular)
                a20, a21 = _nd_unit_outputs(p, cx, cy, cz, mod=mod, omega0=omega0)
                r2 = cx * cx + cy * cy + cz * cz
                for n in range(N):
                    for c in range(C):
                        jj = n * C + c
                        want = math.exp(-window[c] * r2) * (p["w3"][0, jj] * a20 + p["w3"][1, jj] * a21
                                                            + p["b3"][jj])
                        assert abs(K[n, c, i, j, k] - want) <= 1e-12 * (1 + abs(want)), (i, j, k, n, c)


@pytest.mark.parametrize("circular", [False, True])
def test_nd_filter_film_hidden_layers_closed_form(circular):
    _check_film(circular)


def test_nd_filter_2d_grid_hidden_layers_closed_form():
    # X = 1: the x coordinate is 0 in both boundaries, so unit 0 sees only its bias
    _check_nd(False, X=1, Y=4, Z=4)
    _check_nd(True, X=1, Y=4, Z=4)


# ------------------------------------------------------------ planted mistakes

class _WrongSine:
    """Stands in for numpy inside one oracle module; its `which`-th call of sin
    (counting from 1) returns a wrong activation, every other call is numpy's."""

    KINDS = {
        "cos": np.cos,                                    # cos for sin
        "missing": lambda a: np.asarray(a, np.float64),   # activation dropped
        "extra": lambda a: np.sin(np.sin(a)),             # activation applied twice
        "2pi": lambda a: np.sin(2 * np.pi * np.asarray(a)),
    }

    def __init__(self, which, kind):
        self.which, self.kind, self.calls = which, kind, 0

    def __getattr__(self, name):
        return getattr(np, name)

    def sin(self, a, *args, **kw):
        self.calls += 1
        if self.calls == self.which:
            return self.KINDS[self.kind](a)
        return np.sin(a, *args, **kw)


def _fails(check, module, which, kind, monkeypatch):
    with monkeypatch.context() as m:
        m.setattr(module, "np", _WrongSine(which, kind))
        try:
            check()
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("kind", sorted(_WrongSine.KINDS))
@pytest.mark.parametrize("which", [1, 2, 3])     # sin calls: positional-encoding sines, layer 1, layer 2
def test_planted_1d_activation_mistakes_fail_a_pin(kind, which, monkeypatch):
    assert _fails(_check_causal, od_mod, which, kind, monkeypatch)
    assert _fails(_check_noncausal, od_mod, which, kind, monkeypatch)


@pytest.mark.parametrize("kind", sorted(_WrongSine.KINDS))
@pytest.mark.parametrize("which", [1, 2])        # sin calls: layer 1, layer 2
def test_planted_nd_activation_mistakes_fail_a_pin(kind, which, monkeypatch):
    assert _fails(lambda: _check_nd(False), nd_mod, which, kind, monkeypatch)
    assert _fails(lambda: _check_nd(True), nd_mod, which, kind, monkeypatch)
    assert _fails(lambda: _check_film(False), film_mod, which, kind, monkeypatch)
    assert _fails(lambda: _check_film(True), film_mod, which, kind, monkeypatch)


def test_unplanted_pins_pass_through_the_stand_in(monkeypatch):
    # the stand-in itself changes nothing when no call is planted
    for check, module in ((_check_causal, od_mod), (lambda: _check_nd(False), nd_mod),
                          (lambda: _check_film(True), film_mod)):
        assert not _fails(check, module, 0, "cos", monkeypatch)
