"""Pins of the fp64 oracle against things other than itself.

Each test checks the oracle against a library routine (numpy.fft, numpy.convolve,
numpy.cumsum, scipy.special.expit), a closed form, a brute-force sum, or an
invariant the pages state (causality; zero padding to twice the length makes the
FFT convolution non-circular; the convolution theorem).
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle
from synth import make_1d, make_nd

RNG = np.random.default_rng(1234)


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------------- FFT

@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 64, 256, 1024, 4096])
def test_fft_matches_numpy(n):
    x = RNG.standard_normal((3, n)) + 1j * RNG.standard_normal((3, n))
    assert rel(oracle.fft_radix2(x), np.fft.fft(x, axis=-1)) < 1e-12
    assert rel(oracle.fft_radix2(x, inverse=True), np.fft.ifft(x, axis=-1)) < 1e-12


def test_fft_parseval_and_hermitian():
    x = RNG.standard_normal((2, 512))
    X = oracle.fft_radix2(x)
    n = x.shape[-1]
    assert np.allclose(np.sum(np.abs(x) ** 2, -1), np.sum(np.abs(X) ** 2, -1) / n, rtol=1e-12)
    k = np.arange(1, n)
    assert np.allclose(X[:, n - k], np.conj(X[:, k]), rtol=0, atol=1e-10)


def test_fft_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.fft_radix2(np.ones(12))


def test_fftn3_matches_numpy():
    x = RNG.standard_normal((2, 4, 8, 16)) + 1j * RNG.standard_normal((2, 4, 8, 16))
    assert rel(oracle.fftn3_radix2(x), np.fft.fftn(x, axes=(-3, -2, -1))) < 1e-12
    assert rel(oracle.fftn3_radix2(x, inverse=True), np.fft.ifftn(x, axes=(-3, -2, -1))) < 1e-12


# ------------------------------------------------------------------ convolution

@pytest.mark.parametrize("L", [1, 2, 5, 37, 128])
def test_direct_conv_is_truncated_np_convolve(L):
    h = RNG.standard_normal((4, L))
    z = RNG.standard_normal((4, L))
    got = oracle.causal_conv_direct(h, z)
    want = np.stack([np.convolve(h[i], z[i])[:L] for i in range(4)])
    assert rel(got, want) < 1e-13


@pytest.mark.parametrize("L", [1, 2, 4, 16, 128, 1024, 4096])
def test_fft_conv_equals_direct_conv(L):
    h = RNG.standard_normal((3, L))
    z = RNG.standard_normal((2, 3, L))
    assert rel(oracle.causal_conv_fft(h, z), oracle.causal_conv_direct(h, z)) < 1e-11


def test_without_padding_the_fft_conv_wraps():
    # Circular convolution of length L (no padding) = causal conv + wrapped tail.
    L = 64
    h = RNG.standard_normal(L)
    z = RNG.standard_normal(L)
    circ = oracle.fft_radix2(oracle.fft_radix2(h) * oracle.fft_radix2(z), inverse=True).real
    full = np.convolve(h, z)
    assert np.allclose(circ, full[:L] + np.concatenate([full[L:], [0.0]]), atol=1e-10)
    assert not np.allclose(circ, oracle.causal_conv_direct(h, z), atol=1e-3)


def test_constant_filter_is_prefix_sum():
    z = RNG.standard_normal((2, 100))
    assert rel(oracle.causal_conv_direct(np.ones(100), z), np.cumsum(z, axis=-1)) < 1e-13


def test_geometric_filter_is_first_order_scan():
    L, r = 256, 0.97
    z = RNG.standard_normal(L)
    c = np.zeros(L)
    acc = 0.0
    for t in range(L):
        acc = r * acc + z[t]
        c[t] = acc
    h = r ** np.arange(L)
    assert rel(oracle.causal_conv_fft(h, z), c) < 1e-11


# ---------------------------------------------------------------- filter / PosEnc

def test_posenc_frequencies_and_order():
    L, K = 64, 5
    e = oracle.posenc(L, K)
    assert e.shape == (L, 1 + 2 * K)
    assert np.allclose(e[:, 0], np.arange(L) / L)
    for k in range(1, K + 1):
        Fc = np.fft.fft(e[:, k])
        Fs = np.fft.fft(e[:, K + k])
        expect_c = np.zeros(L, complex)
        expect_c[k] = expect_c[L - k] = L / 2
        expect_s = np.zeros(L, complex)
        expect_s[k], expect_s[L - k] = -1j * L / 2, 1j * L / 2
        assert np.allclose(Fc, expect_c, atol=1e-9)
        assert np.allclose(Fs, expect_s, atol=1e-9)


def _filter_params(K, W, N, D, seed=0):
    inp = make_1d(seed, 1, 8, D, N=N, K=K, W=W)
    return dict(inp.filter_params)


def test_window_decays_and_unit_start():
    L, N, D = 256, 2, 8
    p = _filter_params(4, 16, N, D)
    p["w3"] = np.zeros_like(p["w3"])
    p["b3"] = np.ones_like(p["b3"])
    h = oracle.implicit_filter(p, L, N, D)
    assert np.allclose(h[:, :, 0], 1.0)
    ratio = h[:, :, 1:] / h[:, :, :-1]
    assert np.allclose(ratio, ratio[:, :, :1])          # geometric in t
    a = -np.log(ratio[0, :, 0]) * L
    # decays spread from |ln 1e-2|/1.5 (first channel) to |ln 1e-2|/0.3 (last)
    assert math.isclose(a[0] * 1.5, math.log(100), rel_tol=1e-6)
    assert math.isclose(a[-1] * 0.3, math.log(100), rel_tol=1e-6)
    assert np.all(np.diff(a) > 0)


def test_filter_ffn_structure():
    # w1 = 0, b1 = pi/2 -> first activation is 1; w2 = 0, b2 = beta -> second is sin(beta);
    # output = sin(beta) * sum_j w3[j, :] + b3, times the window.
    L, N, D, W = 32, 2, 4, 8
    p = _filter_params(3, W, N, D)
    p["w1"] = np.zeros_like(p["w1"])
    p["b1"] = np.full_like(p["b1"], np.pi / 2)
    p["w2"] = np.zeros_like(p["w2"])
    p["b2"] = np.full_like(p["b2"], 0.3)
    p["decay"] = np.zeros_like(p["decay"])
    h = oracle.implicit_filter(p, L, N, D)
    o = math.sin(0.3) * p["w3"].astype(np.float64).sum(0) + p["b3"]
    assert np.allclose(h, o.reshape(N, D)[:, :, None] * np.ones(L), atol=1e-6)


def test_filter_periodic_when_only_one_frequency_is_fed():
    # Only the cos_2 and sin_2 features reach the FFN -> filter periodic with period L/2
    # (window off); only cos_2 -> even around t = 0 (h(t) = h(L - t)).
    L, K, N, D = 64, 4, 1, 4
    p = _filter_params(K, 8, N, D)
    p["decay"] = np.zeros_like(p["decay"])
    keep = np.zeros_like(p["w1"])
    keep[2] = p["w1"][2]
    keep[K + 2] = p["w1"][K + 2]
    p["w1"] = keep
    h = oracle.implicit_filter(p, L, N, D)
    assert np.allclose(h[..., : L // 2], h[..., L // 2:], atol=1e-12)
    only_cos = np.zeros_like(keep)
    only_cos[2] = keep[2]
    p["w1"] = only_cos
    h = oracle.implicit_filter(p, L, N, D)
    t = np.arange(1, L)
    assert np.allclose(h[..., t], h[..., L - t], atol=1e-12)


# ---------------------------------------------------------------------- operator

def _small(seed=7, B=2, L=64, D=8, N=2, K=4):
    return make_1d(seed, B, L, D, N=N, K=K, W=16)


def _proj_blocks(inp):
    """Projected and short-convolved blocks computed with numpy.convolve."""
    p = inp.u.astype(np.float64) @ inp.w_in.astype(np.float64)
    B, L, J = p.shape
    s = np.empty_like(p)
    for b in range(B):
        for j in range(J):
            s[b, :, j] = np.convolve(p[b, :, j], inp.short_w[j].astype(np.float64))[:L]
    D = inp.D
    return [s[..., i * D:(i + 1) * D] for i in range(inp.N + 1)]


def _run(inp, h, dskip=None, conv="direct", w_in=None):
    return oracle.hyena_fwd(inp.u, inp.w_in if w_in is None else w_in, inp.short_w,
                            inp.dskip if dskip is None else dskip, inp.w_out, h, conv=conv)


def test_delta_filter_reduces_to_products():
    inp = _small()
    h = np.zeros((inp.N, inp.D, inp.L))
    h[:, :, 0] = 1.0
    y = _run(inp, h, dskip=np.zeros((inp.N, inp.D)))
    v, x1, x2 = _proj_blocks(inp)
    assert rel(y, (v * x1 * x2) @ inp.w_out.astype(np.float64)) < 1e-12


def test_block_order_first_gate_is_block_one():
    inp = _small()
    h = np.zeros((inp.N, inp.D, inp.L))
    h[0, :, 0] = 1.0
    dskip = np.zeros((inp.N, inp.D))
    dskip[1] = 1.0
    y = _run(inp, h, dskip=dskip)
    v, x1, _ = _proj_blocks(inp)
    assert rel(y, (v * x1) @ inp.w_out.astype(np.float64)) < 1e-12


def test_skip_only():
    inp = _small()
    y = _run(inp, np.zeros((inp.N, inp.D, inp.L)))
    v = _proj_blocks(inp)[0]
    d = inp.dskip.astype(np.float64)
    assert rel(y, (d[0] * d[1] * v) @ inp.w_out.astype(np.float64)) < 1e-12


def test_order_one_constant_filter_is_gated_prefix_sum():
    inp = _small(N=1)
    h = np.ones((1, inp.D, inp.L))
    y = _run(inp, h, dskip=np.zeros((1, inp.D)))
    v, x1 = _proj_blocks(inp)
    assert rel(y, (x1 * np.cumsum(v, axis=1)) @ inp.w_out.astype(np.float64)) < 1e-12


def test_causality():
    inp = _small(L=48)
    h = oracle.implicit_filter(inp.filter_params, inp.L, inp.N, inp.D)
    y0 = _run(inp, h)
    t0 = 20
    u2 = inp.u.copy()
    u2[:, t0] += 3.0
    y1 = oracle.hyena_fwd(u2, inp.w_in, inp.short_w, inp.dskip, inp.w_out, h, conv="direct")
    assert np.array_equal(y0[:, :t0], y1[:, :t0])
    assert not np.allclose(y0[:, t0], y1[:, t0])


def test_linear_in_v_block_for_fixed_gates():
    inp = _small()
    h = oracle.implicit_filter(inp.filter_params, inp.L, inp.N, inp.D)
    D = inp.D
    wa = inp.w_in.astype(np.float64).copy()
    wb = wa.copy()
    split = RNG.standard_normal((D, D))
    wa[:, :D] = split
    wb[:, :D] = inp.w_in[:, :D] - split
    ysum = _run(inp, h, w_in=wa) + _run(inp, h, w_in=wb)
    assert rel(ysum, _run(inp, h)) < 1e-11
    w3 = inp.w_in.astype(np.float64).copy()
    w3[:, :D] *= -2.5
    assert rel(_run(inp, h, w_in=w3), -2.5 * _run(inp, h)) < 1e-12


def test_fft_and_direct_paths_agree_on_operator():
    inp = _small(L=256, D=16, N=3)
    h = oracle.implicit_filter(inp.filter_params, inp.L, inp.N, inp.D)
    assert rel(_run(inp, h, conv="fft"), _run(inp, h, conv="direct")) < 1e-11


def test_sampled_equals_full():
    inp = _small(L=128, D=8, N=2)
    h = oracle.implicit_filter(inp.filter_params, inp.L, inp.N, inp.D)
    full = _run(inp, h)
    ts = np.array([0, 1, 2, 63, 100, 127])
    samp = oracle.hyena_fwd_sampled(inp.u, inp.w_in, inp.short_w, inp.dskip, inp.w_out, h, ts, chunk=3)
    assert rel(samp, full[:, ts]) < 1e-11


# ---------------------------------------------------------------------------- ND

def test_conv3d_fft_equals_direct_8cube():
    K = RNG.standard_normal((2, 16, 16, 16))
    z = RNG.standard_normal((2, 8, 8, 8))
    assert rel(oracle.conv3d_fft(K, z), oracle.conv3d_direct(K, z)) < 1e-11


def test_conv3d_non_cubic_grid():
    K = RNG.standard_normal((8, 4, 16))
    z = RNG.standard_normal((4, 2, 8))
    assert rel(oracle.conv3d_fft(K, z), oracle.conv3d_direct(K, z)) < 1e-11


def test_conv3d_delta_kernel_is_identity():
    X = Y = Z = 8
    K = np.zeros((2 * X, 2 * Y, 2 * Z))
    K[X, Y, Z] = 1.0
    z = RNG.standard_normal((X, Y, Z))
    assert np.allclose(oracle.conv3d_direct(K, z), z, atol=0)
    assert rel(oracle.conv3d_fft(K, z), z) < 1e-12


def test_conv3d_separable_is_product_of_1d_convs():
    X, Y, Z = 8, 4, 8
    a, b, c = RNG.standard_normal(2 * X), RNG.standard_normal(2 * Y), RNG.standard_normal(2 * Z)
    f, g, k = RNG.standard_normal(X), RNG.standard_normal(Y), RNG.standard_normal(Z)
    K = a[:, None, None] * b[None, :, None] * c[None, None, :]
    z = f[:, None, None] * g[None, :, None] * k[None, None, :]
    ox = np.convolve(a, f)[X:2 * X]
    oy = np.convolve(b, g)[Y:2 * Y]
    oz = np.convolve(c, k)[Z:2 * Z]
    want = ox[:, None, None] * oy[None, :, None] * oz[None, None, :]
    assert rel(oracle.conv3d_direct(K, z), want) < 1e-12
    assert rel(oracle.conv3d_fft(K, z), want) < 1e-11


def test_nd_filter_radial_window():
    X = Y = Z = 8
    N, C = 2, 4
    inp = make_nd(3, 1, X, Y, Z, C, N=N, W=8)
    p = dict(inp.filter_params)
    p["w3"] = np.zeros_like(p["w3"])
    p["b3"] = np.ones_like(p["b3"])
    K = oracle.nd_filter(p, X, Y, Z, N, C)
    a = inp.decay.astype(np.float64)
    assert np.allclose(K[:, :, X, Y, Z], 1.0)                      # offset 0
    assert np.allclose(K[0, :, X + X // 2, Y, Z], np.exp(-a * 0.5))  # offset (G/2, 0, 0)
    assert np.allclose(K[0, :, X, Y, Z + 3], np.exp(-a * 3 / Z))
    # radial: symmetric under sign flips and axis permutations
    inner = K[..., 1:, 1:, 1:]
    assert np.allclose(inner, inner[..., ::-1, ::-1, ::-1])
    assert np.allclose(inner, np.swapaxes(inner, -1, -3))


def test_nd_gate_closed_form():
    B, C, N = 2, 5, 2
    m = RNG.standard_normal((B, C))
    u = np.broadcast_to(m[:, None, None, None, :], (B, 4, 4, 4, C))
    a = RNG.standard_normal((N, C))
    b = RNG.standard_normal((N, C))
    g = oracle.nd_gate(u, a, b)
    want = scipy.special.expit(a[None] * m[:, None, :] + b[None])
    assert rel(g, want) < 1e-14


def _nd_blocks(inp):
    p = inp.u.astype(np.float64) @ inp.w_in.astype(np.float64)
    C = inp.C
    return [p[..., i * C:(i + 1) * C] for i in range(inp.N + 1)]


def test_nd_delta_kernel_closed_form():
    X = Y = Z = 4
    inp = make_nd(4, 2, X, Y, Z, 3, N=2, W=8, u_mean_spread=0.7)
    K = np.zeros((2, 3, 2 * X, 2 * Y, 2 * Z))
    K[:, :, X, Y, Z] = 1.0
    y = oracle.hyena_nd_fwd(inp.u, inp.w_in, np.zeros((2, 3)), inp.gate_a, inp.gate_b,
                            inp.w_out, K, conv="direct")
    v, x1, x2 = _nd_blocks(inp)
    m = inp.u.astype(np.float64).mean(axis=(1, 2, 3))
    g1 = scipy.special.expit(inp.gate_a[0] * m + inp.gate_b[0])[:, None, None, None, :]
    g2 = scipy.special.expit(inp.gate_a[1] * m + inp.gate_b[1])[:, None, None, None, :]
    want = (x2 * g2 * x1 * g1 * v) @ inp.w_out.astype(np.float64)
    assert rel(y, want) < 1e-12


def test_nd_fft_equals_direct_and_sampled_equals_full():
    X = Y = Z = 4
    inp = make_nd(5, 2, X, Y, Z, 4, N=2, W=8, u_mean_spread=0.5)
    K = oracle.nd_filter(inp.filter_params, X, Y, Z, 2, 4)
    args = (inp.u, inp.w_in, inp.dskip, inp.gate_a, inp.gate_b, inp.w_out, K)
    yd = oracle.hyena_nd_fwd(*args, conv="direct")
    yf = oracle.hyena_nd_fwd(*args, conv="fft")
    assert rel(yf, yd) < 1e-11
    pts = np.array([[0, 0, 0], [3, 3, 3], [1, 2, 3], [3, 0, 2]])
    ys = oracle.hyena_nd_fwd_sampled(*args, pts, chunk=3)
    assert rel(ys, yd[:, pts[:, 0], pts[:, 1], pts[:, 2]]) < 1e-11


def test_nd_causality_free_but_translation_equivariant_interior():
    # A kernel supported near offset 0 and an input supported in the middle: shifting
    # the input by one voxel shifts the output by one voxel (away from the borders).
    X = Y = Z = 8
    K = np.zeros((16, 16, 16))
    K[X - 1:X + 2, Y - 1:Y + 2, Z - 1:Z + 2] = RNG.standard_normal((3, 3, 3))
    z = np.zeros((X, Y, Z))
    z[3, 3, 3] = 1.0
    z[3, 4, 3] = -2.0
    o1 = oracle.conv3d_fft(K, z)
    o2 = oracle.conv3d_fft(K, np.roll(z, 1, axis=0))
    assert np.allclose(np.roll(o1, 1, axis=0)[1:-1], o2[1:-1], atol=1e-12)


# ------------------------------------------------------------- ND, circular
# Periodic grids (HyenaND explainer, "Handling Boundaries": circular convolution
# for periodic physical systems). Offset-indexed kernels hold offset d at index
# d + G/2, d in [-G/2, G/2).

def _circ_conv_numpy(K, z):
    """Circular convolution through numpy's FFT (a library routine, not the oracle's)."""
    X, Y, Z = z.shape[-3:]
    Kw = np.roll(K, shift=(-(X // 2), -(Y // 2), -(Z // 2)), axis=(-3, -2, -1))
    return np.fft.ifftn(np.fft.fftn(Kw, axes=(-3, -2, -1)) * np.fft.fftn(z, axes=(-3, -2, -1)),
                        axes=(-3, -2, -1)).real


def test_conv3d_circular_fft_equals_direct():
    K = RNG.standard_normal((2, 8, 8, 8))
    z = RNG.standard_normal((2, 8, 8, 8))
    assert rel(oracle.conv3d_circular_fft(K, z), oracle.conv3d_circular_direct(K, z)) < 1e-11
    K = RNG.standard_normal((8, 4, 4))
    z = RNG.standard_normal((8, 4, 4))
    assert rel(oracle.conv3d_circular_fft(K, z), oracle.conv3d_circular_direct(K, z)) < 1e-11


def test_conv3d_circular_matches_library_fft():
    # an asymmetric kernel: a flipped offset or a wrong wrap direction fails here
    K = RNG.standard_normal((3, 8, 4, 4))
    z = RNG.standard_normal((3, 8, 4, 4))
    assert rel(oracle.conv3d_circular_direct(K, z), _circ_conv_numpy(K, z)) < 1e-12


def test_conv3d_circular_single_offset_is_a_roll():
    # K = delta at offset d: out[p] = z[p - d] for every p (wrapping)
    X, Y, Z = 8, 4, 4
    z = RNG.standard_normal((X, Y, Z))
    for d in [(0, 0, 0), (1, 0, 0), (-4, 1, -2), (3, -2, 1)]:
        K = np.zeros((X, Y, Z))
        K[d[0] + X // 2, d[1] + Y // 2, d[2] + Z // 2] = 1.0
        want = np.roll(z, shift=d, axis=(0, 1, 2))
        assert np.array_equal(oracle.conv3d_circular_direct(K, z), want)
        assert rel(oracle.conv3d_circular_fft(K, z), want) < 1e-12


def test_conv3d_circular_shift_equivariant_everywhere():
    K = RNG.standard_normal((8, 8, 8))
    z = RNG.standard_normal((8, 8, 8))
    o = oracle.conv3d_circular_fft(K, z)
    for s in [(1, 0, 0), (0, 3, 5), (7, 7, 1)]:
        o2 = oracle.conv3d_circular_fft(K, np.roll(z, s, axis=(0, 1, 2)))
        assert rel(o2, np.roll(o, s, axis=(0, 1, 2))) < 1e-12


def test_conv3d_circular_separable_is_product_of_1d_circular_convs():
    X, Y, Z = 8, 4, 8
    a, b, c = RNG.standard_normal(X), RNG.standard_normal(Y), RNG.standard_normal(Z)
    f, g, k = RNG.standard_normal(X), RNG.standard_normal(Y), RNG.standard_normal(Z)
    K = a[:, None, None] * b[None, :, None] * c[None, None, :]
    z = f[:, None, None] * g[None, :, None] * k[None, None, :]

    def circ1(h, x):
        G = len(x)
        # out[p] = sum_q h[offset (p - q) mod G] x[q], offset index (p - q + G/2) mod G
        return np.array([sum(h[(p - q + G // 2) % G] * x[q] for q in range(G)) for p in range(G)])

    want = circ1(a, f)[:, None, None] * circ1(b, g)[None, :, None] * circ1(c, k)[None, None, :]
    assert rel(oracle.conv3d_circular_direct(K, z), want) < 1e-12
    assert rel(oracle.conv3d_circular_fft(K, z), want) < 1e-11


def test_conv3d_circular_equals_linear_when_nothing_wraps():
    # kernel within |d| <= 1 and input within [2, 6)^3 of an 8^3 grid: no sum
    # crosses the boundary, so the periodic and the zero-padded results agree
    G = 8
    Kc = np.zeros((G, G, G))
    Kc[G // 2 - 1:G // 2 + 2, G // 2 - 1:G // 2 + 2, G // 2 - 1:G // 2 + 2] = RNG.standard_normal((3, 3, 3))
    Kp = np.zeros((2 * G, 2 * G, 2 * G))
    Kp[G - 1:G + 2, G - 1:G + 2, G - 1:G + 2] = Kc[G // 2 - 1:G // 2 + 2, G // 2 - 1:G // 2 + 2, G // 2 - 1:G // 2 + 2]
    z = np.zeros((G, G, G))
    z[2:6, 2:6, 2:6] = RNG.standard_normal((4, 4, 4))
    assert rel(oracle.conv3d_circular_direct(Kc, z), oracle.conv3d_direct(Kp, z)) < 1e-12


def test_nd_offsets_circular_span_one_period():
    X, Y, Z = 8, 4, 4
    c = oracle.nd_offsets(X, Y, Z, circular=True)
    assert c.shape == (X, Y, Z, 3)
    assert np.array_equal(c[:, 0, 0, 0], np.arange(-4, 4) / 4.0)
    assert np.array_equal(c[0, :, 0, 1], np.arange(-2, 2) / 2.0)
    assert np.array_equal(c[X // 2, Y // 2, Z // 2], [0.0, 0.0, 0.0])   # offset 0 at index G/2
    # the padded mode keeps its own grid: offsets [-G, G) at c = d / G
    cp = oracle.nd_offsets(X, Y, Z)
    assert cp.shape == (2 * X, 2 * Y, 2 * Z, 3)
    assert np.array_equal(cp[:, 0, 0, 0], np.arange(-X, X) / X)


def test_nd_filter_circular_window():
    X = Y = Z = 8
    N, C = 2, 4
    inp = make_nd(3, 1, X, Y, Z, C, N=N, W=8)
    p = dict(inp.filter_params)
    p["w3"] = np.zeros_like(p["w3"])
    p["b3"] = np.ones_like(p["b3"])
    K = oracle.nd_filter(p, X, Y, Z, N, C, circular=True)
    assert K.shape == (N, C, X, Y, Z)
    a = inp.decay.astype(np.float64)
    assert np.allclose(K[:, :, 4, 4, 4], 1.0)                         # offset 0
    assert np.allclose(K[0, :, 6, 4, 4], np.exp(-a * 0.5))            # offset (2, 0, 0): c = 2/4
    assert np.allclose(K[0, :, 0, 4, 4], np.exp(-a * 1.0))            # offset (-4, 0, 0): c = -1


def test_nd_circular_operator_is_translation_equivariant():
    # the gate sees grid means (unchanged by a roll) and the projections act per
    # voxel, so rolling the input rolls the output of the whole operator exactly
    X = Y = Z = 4
    inp = make_nd(6, 2, X, Y, Z, 4, N=2, W=8, u_mean_spread=0.5)
    K = oracle.nd_filter(inp.filter_params, X, Y, Z, 2, 4, circular=True)
    rest = (inp.w_in, inp.dskip, inp.gate_a, inp.gate_b, inp.w_out, K)
    y = oracle.hyena_nd_fwd(inp.u, *rest, circular=True)
    s = (1, 2, 3)
    y2 = oracle.hyena_nd_fwd(np.roll(inp.u, s, axis=(1, 2, 3)), *rest, circular=True)
    assert rel(y2, np.roll(y, s, axis=(1, 2, 3))) < 1e-12


def test_nd_circular_fft_equals_direct_and_sampled_equals_full():
    X = Y = Z = 4
    inp = make_nd(7, 3, X, Y, Z, 4, N=2, W=8, u_mean_spread=0.5)
    K = oracle.nd_filter(inp.filter_params, X, Y, Z, 2, 4, circular=True)
    args = (inp.u, inp.w_in, inp.dskip, inp.gate_a, inp.gate_b, inp.w_out, K)
    yd = oracle.hyena_nd_fwd(*args, conv="direct", circular=True)
    yf = oracle.hyena_nd_fwd(*args, conv="fft", circular=True)
    assert rel(yf, yd) < 1e-11
    pts = np.array([[0, 0, 0], [3, 3, 3], [1, 2, 3], [3, 0, 2]])
    ys = oracle.hyena_nd_fwd_sampled(*args, pts, chunk=3, circular=True)
    assert rel(ys, yd[:, pts[:, 0], pts[:, 1], pts[:, 2]]) < 1e-11
    # the boundary matters: the zero-padded operator gives a different result
    Kp = oracle.nd_filter(inp.filter_params, X, Y, Z, 2, 4)
    yp = oracle.hyena_nd_fwd(*args[:-1], Kp)
    assert rel(yp, yd) > 1e-3


# ---------------------------------------------------------------- ND, 2D grids
# A 2D grid (image plane) is the 3D operator with X = 1 (HyenaND explainer,
# "Native ND Convolution": grids of any dimension).

def test_conv2d_zero_padded_matches_scipy():
    import scipy.signal
    Y, Z = 8, 4
    K = RNG.standard_normal((2, 2 * Y, 2 * Z))      # x offsets -1, 0
    z = RNG.standard_normal((1, Y, Z))
    # out[p] = sum_q K0[p - q] z[q] with K0 the dx = 0 slice, offset d at index d + G
    full = scipy.signal.convolve2d(K[1], z[0], mode="full")
    want = full[Y:2 * Y, Z:2 * Z]
    assert rel(oracle.conv3d_direct(K, z)[0], want) < 1e-12
    assert rel(oracle.conv3d_fft(K, z)[0], want) < 1e-12


def test_conv2d_circular_matches_library_fft():
    Y, Z = 8, 4
    K = RNG.standard_normal((1, Y, Z))
    z = RNG.standard_normal((1, Y, Z))
    Kw = np.roll(K[0], shift=(-(Y // 2), -(Z // 2)), axis=(0, 1))
    want = np.fft.ifft2(np.fft.fft2(Kw) * np.fft.fft2(z[0])).real
    assert rel(oracle.conv3d_circular_direct(K, z)[0], want) < 1e-12
    assert rel(oracle.conv3d_circular_fft(K, z)[0], want) < 1e-12


def test_nd_filter_2d_uses_x_coordinate_zero():
    # with X = 1 the kernel's x coordinate is 0 (dx = 0 slice): the first MLP row
    # (the x weights) cannot change it, in either boundary
    Y = Z = 8
    inp = make_nd(8, 1, 1, Y, Z, 4, N=2, W=8)
    p = dict(inp.filter_params)
    p2 = dict(p)
    p2["w1"] = p["w1"].copy()
    p2["w1"][0] += 3.0
    for circ, sl in ((False, 1), (True, 0)):
        Ka = oracle.nd_filter(p, 1, Y, Z, 2, 4, circular=circ)
        Kb = oracle.nd_filter(p2, 1, Y, Z, 2, 4, circular=circ)
        assert np.array_equal(Ka[:, :, sl], Kb[:, :, sl])
        c = oracle.nd_offsets(1, Y, Z, circular=circ)
        assert np.all(c[sl, ..., 0] == 0.0)


def test_nd_2d_fft_equals_direct():
    inp = make_nd(9, 2, 1, 8, 8, 4, N=2, W=8, u_mean_spread=0.5)
    for circ in (False, True):
        K = oracle.nd_filter(inp.filter_params, 1, 8, 8, 2, 4, circular=circ)
        args = (inp.u, inp.w_in, inp.dskip, inp.gate_a, inp.gate_b, inp.w_out, K)
        yd = oracle.hyena_nd_fwd(*args, conv="direct", circular=circ)
        yf = oracle.hyena_nd_fwd(*args, conv="fft", circular=circ)
        assert rel(yf, yd) < 1e-11


# --------------------------------------------------------- 1D, non-causal
# Two-sided filters over lags (-L, L), the reading of the bidirectional case
# (the pages name causal use and bidirectional comparators only).

@pytest.mark.parametrize("L", [1, 2, 3, 8, 64, 257])
def test_noncausal_conv_direct_matches_numpy_convolve(L):
    h2 = RNG.standard_normal((3, 2 * L - 1))
    z = RNG.standard_normal((3, L))
    want = np.stack([np.convolve(h2[i], z[i])[L - 1:2 * L - 1] for i in range(3)])
    assert rel(oracle.noncausal_conv_direct(h2, z), want) < 1e-12


@pytest.mark.parametrize("L", [1, 2, 16, 128, 1024])
def test_noncausal_conv_fft_equals_direct(L):
    h2 = RNG.standard_normal((2, 2 * L - 1))
    z = RNG.standard_normal((2, L))
    assert rel(oracle.noncausal_conv_fft(h2, z), oracle.noncausal_conv_direct(h2, z)) < 1e-11


def test_noncausal_with_one_sided_filter_is_causal():
    L = 128
    h = RNG.standard_normal((2, L))
    h2 = np.concatenate([np.zeros((2, L - 1)), h], axis=1)     # negative lags zero
    z = RNG.standard_normal((2, L))
    assert rel(oracle.noncausal_conv_fft(h2, z), oracle.causal_conv_direct(h, z)) < 1e-11


def test_noncausal_conv_time_reversal():
    # reversing the input and the lags reverses the output
    L = 50
    h2 = RNG.standard_normal(2 * L - 1)
    z = RNG.standard_normal(L)
    c = oracle.noncausal_conv_direct(h2, z)
    cr = oracle.noncausal_conv_direct(h2[::-1], z[::-1])
    assert rel(cr, c[::-1]) < 1e-12


def test_noncausal_filter_positive_lags_are_the_causal_filter():
    inp = _small(L=64, D=8, N=2, K=4)
    h = oracle.implicit_filter(inp.filter_params, 64, 2, 8)
    h2 = oracle.implicit_filter_noncausal(inp.filter_params, 64, 2, 8)
    assert h2.shape == (2, 8, 127)
    assert np.array_equal(h2[..., 63:], h)


def test_noncausal_filter_negative_lags_flip_the_odd_features():
    # at -tau the features are [-tau, cos, -sin]: negating the weight rows of the
    # odd features makes the causal generator produce h(-t); the window is |tau|
    K = 4
    inp = _small(L=64, D=8, N=2, K=K)
    p = dict(inp.filter_params)
    p["w1"] = np.asarray(p["w1"], np.float64).copy()
    p["w1"][0] *= -1.0
    p["w1"][1 + K:] *= -1.0
    h_flip = oracle.implicit_filter(p, 64, 2, 8)                 # h at -t, t = 0..63
    h2 = oracle.implicit_filter_noncausal(inp.filter_params, 64, 2, 8)
    assert rel(h2[..., 63::-1], h_flip) < 1e-12


def test_noncausal_operator_fft_equals_direct_and_sampled():
    inp = _small(L=128, D=8, N=2)
    h2 = oracle.implicit_filter_noncausal(inp.filter_params, inp.L, inp.N, inp.D)
    args = (inp.u, inp.w_in, inp.short_w, inp.dskip, inp.w_out, h2)
    yd = oracle.hyena_fwd(*args, conv="direct", causal=False)
    yf = oracle.hyena_fwd(*args, conv="fft", causal=False)
    assert rel(yf, yd) < 1e-11
    ts = np.array([0, 1, 63, 100, 127])
    ys = oracle.hyena_fwd_sampled(*args, ts, chunk=3, causal=False)
    assert rel(ys, yd[:, ts]) < 1e-11
    # the future reaches the past: unlike the causal operator
    u2 = inp.u.copy()
    u2[:, 100] += 1.0
    y2 = oracle.hyena_fwd(u2, *args[1:], conv="direct", causal=False)
    assert np.max(np.abs(y2[:, :99] - yd[:, :99])) > 1e-6


# ------------------------------------------------------- channel-shard pools
# The recurrence is depthwise, so running channel shards in separate processes
# must give exactly the single-process result.

def test_pooled_1d_equals_single_process():
    inp = _small(L=128, D=10, N=2)
    h = oracle.implicit_filter(inp.filter_params, inp.L, inp.N, inp.D)
    args = (inp.u, inp.w_in, inp.short_w, inp.dskip, inp.w_out, h)
    assert np.array_equal(oracle.hyena_fwd(*args, conv="fft", workers=3), oracle.hyena_fwd(*args, conv="fft"))


def test_pooled_nd_equals_single_process():
    inp = make_nd(19, 2, 4, 4, 4, 5, N=2, W=8, u_mean_spread=0.5)
    K = oracle.nd_filter(inp.filter_params, 4, 4, 4, 2, 5)
    args = (inp.u, inp.w_in, inp.dskip, inp.gate_a, inp.gate_b, inp.w_out, K)
    assert np.array_equal(oracle.hyena_nd_fwd(*args, workers=2), oracle.hyena_nd_fwd(*args))
