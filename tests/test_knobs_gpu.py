"""The tuning knobs (environment variables read once per process) select other
launch paths of the same computation; each setting runs a small parity check in
a child process (one at a time) against the fp64 oracle."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import numpy as np
from synth import make_1d
from tests.gpu_util import TOL, gpu_1d, oracle_1d, rel_err
for (B, L, D, dt) in {cases!r}:
    inp = make_1d(900 + L + B, B, L, D, N=2, K=8, dtype=dt)
    y = gpu_1d(inp)
    ref, _ = oracle_1d(inp, conv="fft")
    err = rel_err(y, ref)
    print(f"B={{B}} L={{L}} D={{D}} {{dt}} rel err {{err:.3e}}", flush=True)
    assert np.all(np.isfinite(y)) and err <= TOL[dt], err
print("ok", flush=True)
"""

FOUR_STEP = [(2, 8192, 128, "bf16"), (1, 16384, 192, "f32")]


@pytest.mark.parametrize("env,cases", [
    ({"HYENA_SPECTRUM_FP32": "1"}, [(2, 8192, 128, "bf16")]),      # fp32 intermediate with bf16 activations
    ({"HYENA_GROUP_PAIRS": "7"}, FOUR_STEP),                       # ragged channel-pair groups
    ({"HYENA_GROUP_MB": "1"}, [(2, 8192, 128, "bf16")]),           # groups sized by a cache bound
    ({"HYENA_ROW_PREFETCH": "0"}, FOUR_STEP),
    ({"HYENA_ROW_PREFETCH": "2"}, FOUR_STEP),
    ({"HYENA_ROW_PREFETCH": "3"}, FOUR_STEP),
    ({"HYENA_LDS_NBUF": "1"}, [(2, 1024, 128, "bf16"), (1, 2048, 64, "f32")]),  # one LDS buffer per transform
])
def test_knob_setting_keeps_parity(env, cases):
    code = CHILD.format(root=ROOT, cases=cases)
    full = dict(os.environ, **env)
    print(f"knobs {env}", flush=True)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=full, capture_output=True, text=True,
                       timeout=240)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok")
