"""Parity of the register-conditioned HyenaND path (hyena_nd_film_fwd, through the
C ABI) with the fp64 oracle: every sample's kernel, the whole output on small
grids, and sampled outputs of the full-size workload.

Bar (fp32 storage): max |y - y_ref| / max |y_ref| <= 1e-4."""
import os

import numpy as np
import pytest

from synth import make_config, make_nd_film
from tests.gpu_util import gpu_nd_film, oracle_nd_film, rel_err, say

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _check(inp, tol=1e-4):
    say(f"film case B={inp.B} grid={inp.X}x{inp.Y}x{inp.Z} C={inp.C} N={inp.N} W={inp.W} R={inp.reg.shape[1]} "
        f"circular={inp.circular} seed={inp.meta['seed']}")
    y = gpu_nd_film(inp)
    ref, _ = oracle_nd_film(inp)
    err = rel_err(y, ref)
    say(f"  rel err {err:.3e}")
    assert np.all(np.isfinite(y))
    assert err <= tol, err


@pytest.mark.parametrize("W,circ,X", [(16, False, 8), (64, False, 8), (128, True, 8), (64, True, 1)])
def test_film_kernels_match_oracle(W, circ, X):
    # the scalar MLP (W = 16) and the matrix-core MLP (64, 128), 3D and 2D grids
    inp = make_nd_film(61 + W, 2, X, 8, 8, 64, N=2, W=W, circular=circ)
    say(f"film kernels W={W} circular={circ} X={X}")
    _, k = gpu_nd_film(inp, with_k=True)
    _, kref = oracle_nd_film(inp)
    if X == 1 and not circ:
        kref = kref[:, :, :, 1:2]
    assert k.shape == kref.shape
    err = rel_err(k, kref)
    say(f"  kernel rel err {err:.3e}")
    assert err < 1e-5
    # the two samples' registers differ, and so do their kernels
    assert rel_err(k[1], k[0]) > 1e-3


@pytest.mark.parametrize("B,X,Y,C,N,W,R,circ", [
    (1, 4, 4, 64, 2, 16, 4, False),     # smallest padded grid, one sample
    (2, 8, 8, 64, 2, 64, 4, False),
    (3, 8, 8, 64, 1, 16, 1, False),     # one register: z is that register
    (2, 16, 8, 128, 3, 32, 8, False),   # X != Y, three orders
    (2, 16, 16, 64, 2, 64, 4, False),
    (2, 8, 8, 64, 2, 64, 4, True),
    (3, 16, 16, 64, 2, 128, 16, True),
    (2, 1, 16, 64, 2, 64, 4, False),    # 2D grids
    (2, 1, 32, 64, 2, 64, 4, True),
    (3, 1, 32, 64, 2, 64, 4, False),    # 2D, odd batch (a lone sample): 64-point planes
    (3, 1, 64, 64, 2, 64, 4, False),    # 2D, odd batch: 128-point planes (1024-thread kernel)
    (3, 1, 64, 64, 2, 64, 4, True),     # 2D circular, odd batch, 64-point planes
])
def test_film_sweep(B, X, Y, C, N, W, R, circ):
    _check(make_nd_film(600 + B + X + Y + C + N + W + R + 7 * circ, B, X, Y, Y, C, N=N, W=W, R=R, circular=circ))


@pytest.mark.parametrize("B,X,Y,Z,circ", [(2, 8, 16, 32, False), (3, 16, 8, 4, False), (2, 16, 32, 8, True),
                                           (3, 1, 16, 64, False), (2, 1, 64, 8, True)])  # 2D: 32 x 128, 64 x 8
def test_film_non_square(B, X, Y, Z, circ):
    # independent grid axes with per-sample kernels (the (P, Q) pencil pass)
    _check(make_nd_film(640 + B + X + 3 * Y + 5 * Z + 7 * circ, B, X, Y, Z, 64, N=2, W=64, R=4, circular=circ))


def test_film_samples_are_independent():
    # a batch equals its samples run alone (no state shared between samples)
    inp = make_nd_film(71, 3, 8, 8, 8, 64, N=2, W=64)
    y = gpu_nd_film(inp)
    for b in range(3):
        one = make_nd_film(71, 3, 8, 8, 8, 64, N=2, W=64)
        one.base.u = np.ascontiguousarray(inp.u[b:b + 1])
        one.base.B = 1
        one.reg = np.ascontiguousarray(inp.reg[b:b + 1])
        yb = gpu_nd_film(one)
        assert rel_err(yb[0], y[b]) <= 1e-6


def test_full_size_film_sampled():
    name = "nd3d_film_f32_B2_C128_64cube"
    path = os.path.join(GOLDEN, f"sampled_{name}.npz")
    if not os.path.exists(path):
        pytest.fail(f"missing {path}; run tests/golden/make_sampled.py {name}")
    g = np.load(path)
    inp = make_config(name)
    say(f"full-size {name}")
    y = gpu_nd_film(inp)
    assert np.all(np.isfinite(y))
    p = g["points"]
    err = rel_err(y[:, p[:, 0], p[:, 1], p[:, 2], :], g["y"])
    say(f"  rel err at {len(p)} sampled points: {err:.3e}")
    assert err <= 1e-4, err
