"""Full-size workloads on the GPU (the launch configuration bench.py times),
checked at sampled outputs against values the fp64 oracle wrote
(tests/golden/make_sampled.py -> tests/golden/sampled_<workload>.npz).

Bar: max |y - y_ref| / max |y_ref| over the sampled outputs, <= 2e-2 for bf16
storage and <= 1e-4 for fp32."""
import os

import numpy as np
import pytest

from synth import make_config
from tests.gpu_util import TOL, gpu_1d, gpu_nd, rel_err, say

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    path = os.path.join(GOLDEN, f"sampled_{name}.npz")
    if not os.path.exists(path):
        pytest.fail(f"missing {path}; run tests/golden/make_sampled.py {name}")
    return np.load(path, allow_pickle=False)


@pytest.mark.parametrize("name", ["order2_bf16_L64k_D768", "order2_bf16_L1M_D256_dna", "order2_bf16_L256k_D64",
                                  "order2_f32_L512k_D64", "order2_bf16_L64k_D768_noncausal"])
def test_full_size_1d_sampled(name):
    g = _golden(name)
    inp = make_config(name)
    say(f"full-size {name}: B={inp.B} L={inp.L} D={inp.D}")
    y = gpu_1d(inp)
    assert np.all(np.isfinite(y))
    ys = y[:, g["t"], :]
    err = rel_err(ys, g["y"])
    say(f"  rel err at {len(g['t'])} sampled positions: {err:.3e}")
    assert err <= TOL[inp.dtype], err


def test_full_size_nd_sampled():
    name = "nd3d_f32_B2_C128_64cube"
    g = _golden(name)
    inp = make_config(name)
    say(f"full-size {name}")
    y = gpu_nd(inp)
    assert np.all(np.isfinite(y))
    p = g["points"]
    ys = y[:, p[:, 0], p[:, 1], p[:, 2], :]
    err = rel_err(ys, g["y"])
    say(f"  rel err at {len(p)} sampled points: {err:.3e}")
    assert err <= 1e-4, err


@pytest.mark.parametrize("name", ["nd3d_circ_f32_B2_C128_64cube", "nd3d_circ_f32_B1_C64_128cube",
                                  "nd2d_f32_B8_C384_64sq"])
def test_full_size_nd_other_sampled(name):
    """Periodic 3D grids and the 2D image-grid workload."""
    g = _golden(name)
    inp = make_config(name)
    say(f"full-size {name}")
    y = gpu_nd(inp)
    assert np.all(np.isfinite(y))
    p = g["points"]
    ys = y[:, p[:, 0], p[:, 1], p[:, 2], :]
    err = rel_err(ys, g["y"])
    say(f"  rel err at {len(p)} sampled points: {err:.3e}")
    assert err <= 1e-4, err
