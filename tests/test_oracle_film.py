"""Pins of the register/FiLM-conditioned HyenaND oracle against things other than
itself: library reductions (numpy mean), the pinned plain-SIREN kernel
(oracle.nd_filter, itself pinned in test_oracle.py) under exact reparametrisations,
closed forms of the Gaussian window, and invariants (permutations, batch
independence, the pinned gated operator when every sample shares one kernel)."""
import numpy as np
import pytest

import oracle
from synth import make_nd_film

RNG = np.random.default_rng(4321)


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ------------------------------------------------------------- control vector

def test_control_with_equal_scores_is_the_register_mean():
    reg = RNG.standard_normal((3, 5, 16))
    z = oracle.film_control(reg, np.zeros(16))
    assert np.allclose(z, reg.mean(axis=1), rtol=0, atol=1e-14)


def test_control_of_one_register_is_that_register():
    reg = RNG.standard_normal((2, 1, 16))
    assert np.allclose(oracle.film_control(reg, RNG.standard_normal(16)), reg[:, 0], rtol=0, atol=1e-14)


def test_control_is_a_convex_combination_and_permutation_invariant():
    reg = RNG.standard_normal((2, 6, 32))
    q = RNG.standard_normal(32)
    z = oracle.film_control(reg, q)
    assert np.all(z <= reg.max(axis=1) + 1e-12) and np.all(z >= reg.min(axis=1) - 1e-12)
    perm = RNG.permutation(6)
    assert np.allclose(oracle.film_control(reg[:, perm], q), z, rtol=0, atol=1e-13)


def test_control_follows_a_dominant_score():
    # register 2 of sample 0 scores far above the others: the weights select it
    q = np.zeros(8)
    q[0] = 1.0
    reg = RNG.standard_normal((1, 4, 8))
    reg[0, 2, 0] = 80.0
    assert np.allclose(oracle.film_control(reg, q)[0], reg[0, 2], rtol=0, atol=1e-12)


# ------------------------------------------------------------- kernel synthesis

def _plain_params(inp, w1, b1, w2, b2):
    return dict(w1=w1, b1=b1, w2=w2, b2=b2, w3=inp.w3, b3=inp.b3, decay=np.zeros(inp.C))


def test_identity_film_is_the_plain_siren_kernel():
    inp = make_nd_film(11, 1, 4, 4, 4, 8, N=2, W=16)
    p = dict(inp.film_filter_params, omega0=np.ones(16), window=np.zeros(8))
    mod = np.stack([np.ones(16), np.zeros(16), np.ones(16), np.zeros(16)])
    K = oracle.nd_filter_film(p, mod, 4, 4, 4, 2, 8)
    want = oracle.nd_filter(_plain_params(inp, inp.w1, inp.b1, inp.w2, inp.b2), 4, 4, 4, 2, 8)
    assert rel(K, want) < 1e-13


@pytest.mark.parametrize("circular", [False, True])
def test_film_terms_are_exact_reparametrisations_of_the_plain_kernel(circular):
    # gamma scales a layer's pre-activation columns, beta shifts its phase, and
    # omega0 multiplies the first layer's: the plain kernel with rescaled weights
    W, C = 16, 8
    inp = make_nd_film(12, 1, 8, 8, 8, C, N=1, W=W, circular=circular)
    g1, be1, g2, be2 = RNG.uniform(0.5, 1.5, W), RNG.uniform(-1, 1, W), RNG.uniform(0.5, 1.5, W), RNG.uniform(-1, 1, W)
    om = RNG.uniform(1, 20, W)
    p = dict(inp.film_filter_params, omega0=om, window=np.zeros(C))
    K = oracle.nd_filter_film(p, np.stack([g1, be1, g2, be2]), 8, 8, 8, 1, C, circular)
    s1 = om * g1
    w1 = inp.w1.astype(np.float64) * s1[None, :]
    b1 = inp.b1 * s1 + be1
    w2 = inp.w2.astype(np.float64) * g2[None, :]
    b2 = inp.b2 * g2 + be2
    want = oracle.nd_filter(_plain_params(inp, w1, b1, w2, b2), 8, 8, 8, 1, C, circular)
    assert rel(K, want) < 1e-12


def test_gaussian_window_closed_form():
    X = Y = Z = 8
    C = 4
    inp = make_nd_film(13, 1, X, Y, Z, C, N=2, W=16)
    p = dict(inp.film_filter_params, w3=np.zeros_like(inp.w3), b3=np.ones_like(inp.b3))
    mod = oracle.film_modulation(oracle.film_control(inp.reg, inp.q), inp.film_w, inp.film_b)[0]
    K = oracle.nd_filter_film(p, mod, X, Y, Z, 2, C)
    a = inp.window.astype(np.float64)
    assert np.allclose(K[:, :, X, Y, Z], 1.0)                                 # offset 0
    assert np.allclose(K[0, :, X + X // 2, Y, Z], np.exp(-a * 0.25))          # c = (1/2, 0, 0)
    assert np.allclose(K[1, :, X, Y - 3, Z + 2], np.exp(-a * (9 + 4) / 64))    # c = (0, -3/8, 2/8)
    inner = K[..., 1:, 1:, 1:]
    assert np.allclose(inner, inner[..., ::-1, ::-1, ::-1])
    assert np.allclose(inner, np.swapaxes(inner, -1, -2))


def test_control_reaches_the_kernel_through_gamma():
    # one register (z = that register, pinned above) and gamma_1 depending on
    # feature c0 only: gamma_1 = film_b[0] + reg[c0] * v, a column scaling of W1
    W, C, c0 = 16, 8, 3
    inp = make_nd_film(14, 1, 4, 4, 4, C, N=1, W=W, R=1)
    v = RNG.uniform(-0.5, 0.5, W)
    fw = np.zeros((4, C, W))
    fw[0, c0] = v
    fb = np.stack([np.full(W, 1.0), np.zeros(W), np.ones(W), np.zeros(W)])
    mod = oracle.film_modulation(oracle.film_control(inp.reg, inp.q), fw, fb)[0]
    p = dict(inp.film_filter_params, omega0=np.ones(W), window=np.zeros(C))
    K = oracle.nd_filter_film(p, mod, 4, 4, 4, 1, C)
    s1 = 1.0 + float(inp.reg[0, 0, c0]) * v
    want = oracle.nd_filter(_plain_params(inp, inp.w1 * s1[None, :], inp.b1 * s1, inp.w2, inp.b2), 4, 4, 4, 1, C)
    assert rel(K, want) < 1e-12


def test_samples_with_equal_registers_share_their_kernel():
    inp = make_nd_film(15, 3, 4, 4, 4, 8, N=2, W=16)
    reg = inp.reg.copy()
    reg[2] = reg[0]
    Ks = oracle.film_kernels(inp.film_filter_params, reg, inp.q, inp.film_w, inp.film_b, 4, 4, 4, 2, 8)
    assert np.array_equal(Ks[2], Ks[0])
    assert rel(Ks[1], Ks[0]) > 1e-3


# ------------------------------------------------------------- operator

def test_shared_kernel_equals_the_ungated_pinned_operator():
    inp = make_nd_film(16, 2, 4, 4, 4, 8, N=2, W=16)
    K = oracle.nd_filter(inp.base.filter_params, 4, 4, 4, 2, 8)
    y = oracle.hyena_nd_film_fwd(inp.u, inp.w_in, inp.dskip, inp.w_out, np.stack([K, K]))
    ones = (np.zeros((2, 8)), np.full((2, 8), 60.0))   # sigmoid(60) = 1 - 9e-27
    want = oracle.hyena_nd_fwd(inp.u, inp.w_in, inp.dskip, *ones, inp.w_out, K)
    assert rel(y, want) < 1e-13


@pytest.mark.parametrize("circular", [False, True])
def test_batch_is_independent_samples(circular):
    inp = make_nd_film(17, 3, 4, 4, 4, 8, N=2, W=16, circular=circular)
    Ks = oracle.film_kernels(inp.film_filter_params, inp.reg, inp.q, inp.film_w, inp.film_b, 4, 4, 4, 2, 8,
                             circular)
    y = oracle.hyena_nd_film_fwd(inp.u, inp.w_in, inp.dskip, inp.w_out, Ks, circular=circular)
    for b in range(3):
        yb = oracle.hyena_nd_film_fwd(inp.u[b:b + 1], inp.w_in, inp.dskip, inp.w_out, Ks[b:b + 1],
                                      circular=circular)
        assert rel(y[b], yb[0]) < 1e-13


@pytest.mark.parametrize("circular", [False, True])
def test_fft_equals_direct_and_sampled_equals_full(circular):
    X, C = 4, 8
    inp = make_nd_film(18, 2, X, X, X, C, N=2, W=16, circular=circular)
    Ks = oracle.film_kernels(inp.film_filter_params, inp.reg, inp.q, inp.film_w, inp.film_b, X, X, X, 2, C,
                             circular)
    y = oracle.hyena_nd_film_fwd(inp.u, inp.w_in, inp.dskip, inp.w_out, Ks, circular=circular)
    yd = oracle.hyena_nd_film_fwd(inp.u, inp.w_in, inp.dskip, inp.w_out, Ks, conv="direct", circular=circular)
    assert rel(y, yd) < 1e-11
    pts = np.array([[0, 0, 0], [3, 1, 2], [1, 3, 3]])
    ys = oracle.hyena_nd_film_fwd_sampled(inp.u, inp.w_in, inp.dskip, inp.w_out, Ks, pts, chunk=3,
                                          circular=circular)
    assert rel(ys, y[:, pts[:, 0], pts[:, 1], pts[:, 2]]) < 1e-11


def test_pooled_equals_single_process():
    inp = make_nd_film(19, 2, 4, 4, 4, 6, N=2, W=16)
    Ks = oracle.film_kernels(inp.film_filter_params, inp.reg, inp.q, inp.film_w, inp.film_b, 4, 4, 4, 2, 6)
    args = (inp.u, inp.w_in, inp.dskip, inp.w_out, Ks)
    assert np.array_equal(oracle.hyena_nd_film_fwd(*args, workers=4), oracle.hyena_nd_film_fwd(*args))
