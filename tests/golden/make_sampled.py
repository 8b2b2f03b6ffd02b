"""Writes the expected outputs of the full-size workloads at sampled positions.

    python tests/golden/make_sampled.py [workload ...]

Calls only the fp64 oracle (oracle/) on the seeded inputs of synth/. For the
1D workloads the orders before the last run on the whole sequence with the
FFT path and the last order is summed directly at the sampled times; for the
3D workloads the same holds over the grid (the register-conditioned one with
each sample's own kernel). Output: tests/golden/sampled_<name>.npz
with the sampled indices and y at those indices (float64).
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from synth import CONFIGS, TEST_SHAPES, make_config, sample_positions  # noqa: E402

FULL = ["order2_bf16_L64k_D768", "order2_bf16_L1M_D256_dna", "nd3d_f32_B2_C128_64cube"] + list(TEST_SHAPES)
COUNT = 24


def points_3d(X, Y, Z, count, seed):
    rng = np.random.default_rng(20_000 + seed)
    fixed = np.array([[0, 0, 0], [X - 1, Y - 1, Z - 1], [X // 2, Y // 2, Z // 2], [0, Y - 1, 3]])
    extra = np.stack([rng.integers(0, X, count), rng.integers(0, Y, count), rng.integers(0, Z, count)], 1)
    return np.concatenate([fixed, extra])[:count]


def make(name):
    t0 = time.time()
    cfg = CONFIGS[name] if name in CONFIGS else TEST_SHAPES[name]
    inp = make_config(name)
    out = os.path.join(HERE, f"sampled_{name}.npz")
    if cfg["kind"] == "1d":
        ts = sample_positions(inp.L, COUNT, seed=cfg["seed"])
        if inp.causal:
            h = oracle.implicit_filter(inp.filter_params, inp.L, inp.N, inp.D)
        else:
            h = oracle.implicit_filter_noncausal(inp.filter_params, inp.L, inp.N, inp.D)
        y = oracle.hyena_fwd_sampled(inp.u, inp.w_in, inp.short_w, inp.dskip, inp.w_out, h, ts, chunk=16,
                                     causal=inp.causal)
        np.savez(out, t=ts, y=y)
    elif cfg["kind"] == "nd_film":
        pts = points_3d(inp.X, inp.Y, inp.Z, COUNT, cfg["seed"])
        Ks = oracle.film_kernels(inp.film_filter_params, inp.reg, inp.q, inp.film_w, inp.film_b, inp.X, inp.Y,
                                 inp.Z, inp.N, inp.C, inp.circular)
        y = oracle.hyena_nd_film_fwd_sampled(inp.u, inp.w_in, inp.dskip, inp.w_out, Ks, pts, chunk=4,
                                             circular=inp.circular)
        np.savez(out, points=pts, y=y)
    else:
        pts = points_3d(inp.X, inp.Y, inp.Z, COUNT, cfg["seed"])
        K = oracle.nd_filter(inp.filter_params, inp.X, inp.Y, inp.Z, inp.N, inp.C, circular=inp.circular)
        y = oracle.hyena_nd_fwd_sampled(inp.u, inp.w_in, inp.dskip, inp.gate_a, inp.gate_b, inp.w_out, K, pts,
                                        chunk=4, circular=inp.circular)
        np.savez(out, points=pts, y=y)
    print(f"{name}: wrote {out} in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    for n in (sys.argv[1:] or FULL):
        make(n)
