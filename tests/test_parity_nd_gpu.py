"""Parity of the 3D (HyenaND) HIP path (through the C ABI) with the fp64 oracle.

Bar (fp32 storage): max |y - y_ref| / max |y_ref| <= 1e-4 over the whole output."""
import numpy as np
import pytest

from synth import make_nd
from tests.gpu_util import gpu_nd, oracle_nd, rel_err, say

pytestmark = pytest.mark.gpu


def _check(inp, tol=1e-4):
    say(f"nd case B={inp.B} grid={inp.X}x{inp.Y}x{inp.Z} C={inp.C} N={inp.N} seed={inp.meta['seed']}")
    y = gpu_nd(inp)
    ref, _ = oracle_nd(inp)
    err = rel_err(y, ref)
    say(f"  rel err {err:.3e}")
    assert np.all(np.isfinite(y))
    assert err <= tol, err


def test_nd_filter_matches_oracle():
    inp = make_nd(41, 1, 8, 8, 8, 64, N=2, W=64)
    say("nd filter 8^3 C=64 N=2")
    _, k = gpu_nd(inp, with_k=True)
    _, kref = oracle_nd(inp)
    assert rel_err(k, kref) < 1e-5


@pytest.mark.parametrize("B,X,Y,C,N,spread", [
    (2, 4, 4, 64, 2, 0.5),     # smallest grid, gate exercised by mean offsets
    (2, 8, 8, 64, 2, 0.5),
    (1, 8, 8, 64, 2, 0.5),     # odd batch: the second half of the packed field is empty
    (3, 8, 8, 64, 1, 0.0),
    (2, 16, 8, 64, 2, 0.5),    # X != Y
    (2, 8, 16, 128, 3, 0.5),
    (2, 16, 16, 64, 2, 0.5),
    (2, 32, 32, 64, 1, 0.5),
    (2, 8, 8, 192, 2, 0.5),    # C not dividing 256: the general mean / gate kernels
])
def test_nd_sweep(B, X, Y, C, N, spread):
    _check(make_nd(200 + B + X + Y + C + N, B, X, Y, Y, C, N=N, W=64, u_mean_spread=spread))


def test_nd_delta_kernel_closed_form():
    # constant MLP output and a very fast radial window: K ~ delta at offset 0, D = 0
    inp = make_nd(42, 2, 8, 8, 8, 64, N=2, W=32, u_mean_spread=0.7)
    inp.w3 = np.zeros_like(inp.w3)
    inp.b3 = np.ones_like(inp.b3)
    inp.decay = np.full_like(inp.decay, 1.0e4)
    inp.dskip = np.zeros_like(inp.dskip)
    y = gpu_nd(inp)
    import scipy.special
    p = inp.u.astype(np.float64) @ inp.w_in.astype(np.float64)
    C = inp.C
    v, x1, x2 = p[..., :C], p[..., C:2 * C], p[..., 2 * C:]
    m = inp.u.astype(np.float64).mean(axis=(1, 2, 3))
    g1 = scipy.special.expit(inp.gate_a[0] * m + inp.gate_b[0])[:, None, None, None, :]
    g2 = scipy.special.expit(inp.gate_a[1] * m + inp.gate_b[1])[:, None, None, None, :]
    want = (x2 * g2 * x1 * g1 * v) @ inp.w_out.astype(np.float64)
    assert rel_err(y, want) < 1e-4


# ------------------------------------------------------------- circular boundary

def test_nd_circular_filter_matches_oracle():
    inp = make_nd(43, 1, 8, 8, 8, 64, N=2, W=64, circular=True)
    say("nd circular filter 8^3 C=64 N=2")
    _, k = gpu_nd(inp, with_k=True)
    _, kref = oracle_nd(inp)
    assert k.shape == kref.shape == (2, 64, 8, 8, 8)
    assert rel_err(k, kref) < 1e-5


@pytest.mark.parametrize("B,X,Y,C,N,spread", [
    (2, 8, 8, 64, 2, 0.5),     # smallest circular grid (8-point transforms)
    (1, 8, 8, 64, 2, 0.5),     # odd batch
    (3, 8, 8, 64, 1, 0.0),
    (2, 16, 8, 64, 2, 0.5),    # X != Y
    (2, 8, 16, 128, 3, 0.5),
    (2, 16, 16, 64, 2, 0.5),
    (2, 32, 32, 64, 1, 0.5),
    (1, 64, 64, 64, 1, 0.5),   # 64-point planes and pencils
])
def test_nd_circular_sweep(B, X, Y, C, N, spread):
    _check(make_nd(300 + B + X + Y + C + N, B, X, Y, Y, C, N=N, W=64, u_mean_spread=spread, circular=True))


def test_nd_circular_translation_equivariance():
    # periodic grid: rolling the input rolls the output, at every point
    import torch
    inp = make_nd(44, 2, 32, 32, 32, 64, N=2, W=64, u_mean_spread=0.5, circular=True)
    say("nd circular roll 32^3 C=64")
    y = gpu_nd(inp)
    s = (5, 31, 17)
    inp.u = np.ascontiguousarray(np.roll(inp.u, s, axis=(1, 2, 3)))
    y2 = gpu_nd(inp)
    torch.cuda.synchronize()
    err = rel_err(y2, np.roll(y, s, axis=(1, 2, 3)))
    say(f"  roll mismatch {err:.3e}")
    assert err <= 1e-5


# ------------------------------------------------------------- 2D grids (X = 1)

def test_nd_2d_filter_matches_oracle():
    for circ in (False, True):
        inp = make_nd(45, 1, 1, 16, 16, 64, N=2, W=64, circular=circ)
        say(f"nd 2D filter 16^2 C=64 N=2 circular={circ}")
        _, k = gpu_nd(inp, with_k=True)
        _, kref = oracle_nd(inp)
        # zero padded: the oracle also holds the unused dx = -1 slice
        kref = kref[:, :, 1:2] if not circ else kref
        assert k.shape == kref.shape
        assert rel_err(k, kref) < 1e-5


@pytest.mark.parametrize("B,Y,C,N,circ", [
    (2, 4, 64, 2, False),      # smallest zero-padded plane (8-point transforms)
    (2, 8, 64, 2, False),
    (1, 16, 64, 2, False),     # odd batch
    (3, 32, 64, 1, False),
    (2, 64, 128, 3, False),    # 128-point transforms
    (2, 8, 64, 2, True),
    (1, 16, 64, 3, True),
    (2, 32, 64, 2, True),
    (3, 64, 64, 2, True),
    (2, 128, 64, 2, True),     # 128-point circular planes
    (3, 16, 384, 2, False),    # C = 384 (general gate kernels)
])
def test_nd_2d_sweep(B, Y, C, N, circ):
    _check(make_nd(500 + B + Y + C + N + 7 * circ, B, 1, Y, Y, C, N=N, W=64, u_mean_spread=0.5, circular=circ))


@pytest.mark.parametrize("B,Y,Z,C,N,circ", [
    (2, 4, 64, 64, 2, False),     # 8 x 128 planes (the widest and flattest)
    (3, 64, 4, 64, 1, False),     # 128 x 8, odd batch
    (2, 16, 32, 64, 2, False),    # 32 x 64
    (1, 32, 8, 128, 3, False),    # 64 x 16, three orders
    (2, 8, 128, 64, 2, True),     # circular 8 x 128
    (3, 64, 16, 64, 2, True),     # circular 64 x 16, odd batch
    (2, 128, 64, 64, 1, True),    # circular 128 x 64 (1024-line transforms)
])
def test_nd_2d_non_square_sweep(B, Y, Z, C, N, circ):
    # 2D grids take Y and Z independently, like 3D grids
    _check(make_nd(520 + B + 3 * Y + 5 * Z + C + N + 7 * circ, B, 1, Y, Z, C, N=N, W=64, u_mean_spread=0.5,
                   circular=circ))


# ------------------------------------------------------------- reproducibility

@pytest.mark.parametrize("X,Y,circ", [(8, 16, False), (16, 16, False), (8, 16, True)])
def test_nd_filter_spectra_are_bit_reproducible(X, Y, circ):
    # every half-spectrum entry has one writer: two builds of the same layer agree bit for bit
    import torch
    import subquadratic_sequence_amd as hs
    from tests.gpu_util import to_dev
    inp = make_nd(80 + X + Y, 2, X, Y, Y, 64, N=2, W=64, circular=circ)
    say(f"nd spectra reproducibility {X}x{Y}x{Y} circular={circ}")
    bd = hs.ND_CIRCULAR if circ else hs.ND_ZERO_PAD
    fa = [to_dev(a) for a in (inp.w1, inp.b1, inp.w2, inp.b2, inp.w3, inp.b3, inp.decay)]
    caches = []
    for _ in range(2):
        layer = hs.HyenaNDLayer(X, Y, Y, 64, 2, boundary=bd)
        hs.hyena_nd_filter_gen(layer, *fa)
        caches.append(layer.cache)
    torch.cuda.synchronize()
    assert torch.equal(caches[0], caches[1])


# ------------------------------------------------------- non-square grids
# X, Y and Z are independent on 3D grids (HyenaND explainer, "Native ND
# Convolution": the convolution runs on the native grid, any shape).

@pytest.mark.parametrize("B,X,Y,Z,C,N,circ", [
    (2, 8, 16, 32, 64, 2, False),    # 32 x 64 planes
    (2, 16, 32, 8, 64, 2, False),    # 64 x 16 planes
    (1, 8, 4, 16, 64, 2, False),     # odd batch, 8 x 32 planes
    (3, 16, 64, 8, 64, 1, False),    # 128 x 16 planes
    (1, 64, 32, 16, 64, 1, False),   # 128-point x transforms (the persistent pencil pass)
    (1, 64, 16, 64, 64, 1, False),   # 128-point x and z: mirrored pencil blocks in one item, 32-point y
    (3, 64, 8, 64, 64, 2, False),    # the same with an odd batch (second packed field half empty)
    (2, 8, 16, 32, 64, 2, True),     # circular: 16 x 32 planes
    (2, 16, 8, 64, 128, 2, True),
    (1, 8, 128, 16, 64, 1, True),    # circular 128 x 16 planes
])
def test_nd_non_square_sweep(B, X, Y, Z, C, N, circ):
    _check(make_nd(400 + B + X + 3 * Y + 5 * Z + N + 7 * circ, B, X, Y, Z, C, N=N, W=64, u_mean_spread=0.5,
                   circular=circ))


@pytest.mark.parametrize("circ", [False, True])
def test_nd_non_square_filter_matches_oracle(circ):
    inp = make_nd(46, 1, 8, 16, 32, 64, N=2, W=64, circular=circ)
    say(f"nd filter 8x16x32 C=64 N=2 circular={circ}")
    _, k = gpu_nd(inp, with_k=True)
    _, kref = oracle_nd(inp)
    assert k.shape == kref.shape
    assert rel_err(k, kref) < 1e-5


def test_nd_non_square_spectra_are_bit_reproducible():
    import torch
    import subquadratic_sequence_amd as hs
    from tests.gpu_util import to_dev
    inp = make_nd(47, 2, 16, 8, 32, 64, N=2, W=64)
    say("nd spectra reproducibility 16x8x32")
    fa = [to_dev(a) for a in (inp.w1, inp.b1, inp.w2, inp.b2, inp.w3, inp.b3, inp.decay)]
    caches = []
    for _ in range(2):
        layer = hs.HyenaNDLayer(16, 8, 32, 64, 2)
        hs.hyena_nd_filter_gen(layer, *fa)
        caches.append(layer.cache)
    torch.cuda.synchronize()
    assert torch.equal(caches[0], caches[1])
