"""Helpers for the GPU tests: run the HIP path through the C ABI and the oracle
on the same seeded inputs."""
from __future__ import annotations

import os
import sys

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()
    path = os.environ.get("HYENA_TEST_LOG")
    if path:
        with open(path, "a") as f:
            f.write(msg + "\n")


def rel_err(y, ref) -> float:
    return float(np.max(np.abs(np.asarray(y, np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-300))


def to_dev(a, dtype=None, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device=device, dtype=dtype or torch.float32)


def gpu_1d(inp, with_h: bool = False, layer=None):
    """Runs hyena_filter_gen + hyena_fwd on cuda:0; returns y (float64 numpy) [and h]."""
    import torch
    import subquadratic_sequence_amd as hs
    dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    if layer is None:
        layer = hs.HyenaLayer(inp.L, inp.D, inp.N, direction=hs.CAUSAL if inp.causal else hs.NONCAUSAL)
    # non-causal filters come back wrapped: [N][D][2L], lag tau at tau mod 2L
    h_len = inp.L if inp.causal else 2 * inp.L
    h_out = torch.empty(inp.N, inp.D, h_len, device="cuda") if with_h else None
    hs.hyena_filter_gen(layer, to_dev(inp.w1), to_dev(inp.b1), to_dev(inp.w2), to_dev(inp.b2), to_dev(inp.w3),
                        to_dev(inp.b3), to_dev(inp.decay), inp.K, h_out=h_out)
    y = hs.hyena_fwd(layer, to_dev(inp.u, dt), to_dev(inp.w_in, dt), to_dev(inp.short_w), to_dev(inp.dskip),
                     to_dev(inp.w_out, dt))
    torch.cuda.synchronize()
    yn = y.float().cpu().numpy().astype(np.float64)
    if with_h:
        return yn, h_out.cpu().numpy().astype(np.float64)
    return yn


def oracle_1d(inp, conv: str = "auto"):
    """(y, h): h [N, D, L] causal, [N, D, 2L - 1] lag-indexed (lag i - (L-1)) non-causal."""
    import oracle
    if inp.causal:
        h = oracle.implicit_filter(inp.filter_params, inp.L, inp.N, inp.D)
    else:
        h = oracle.implicit_filter_noncausal(inp.filter_params, inp.L, inp.N, inp.D)
    y = oracle.hyena_fwd(inp.u, inp.w_in, inp.short_w, inp.dskip, inp.w_out, h, conv=conv, causal=inp.causal)
    return y, h


def wrap_two_sided(h2):
    """Lag-indexed [..., 2L-1] -> the wrapped [..., 2L] layout of the library's h_out."""
    L = (h2.shape[-1] + 1) // 2
    hw = np.zeros(h2.shape[:-1] + (2 * L,))
    hw[..., :L] = h2[..., L - 1:]
    hw[..., L + 1:] = h2[..., :L - 1]
    return hw


def gpu_nd(inp, with_k: bool = False):
    """Runs hyena_nd_filter_gen + hyena_nd_fwd on cuda:0; returns y (float64 numpy) [and K]."""
    import torch
    import subquadratic_sequence_amd as hs
    bd = hs.ND_CIRCULAR if inp.circular else hs.ND_ZERO_PAD
    layer = hs.HyenaNDLayer(inp.X, inp.Y, inp.Z, inp.C, inp.N, boundary=bd)
    pf = 1 if inp.circular else 2
    mx = 1 if inp.X == 1 else pf * inp.X  # 2D grids: no padding of the one-point x axis
    k_out = None
    if with_k:
        k_out = torch.empty(inp.N, inp.C, mx, pf * inp.Y, pf * inp.Z, device="cuda")
    hs.hyena_nd_filter_gen(layer, to_dev(inp.w1), to_dev(inp.b1), to_dev(inp.w2), to_dev(inp.b2), to_dev(inp.w3),
                           to_dev(inp.b3), to_dev(inp.decay), k_out=k_out)
    y = hs.hyena_nd_fwd(layer, to_dev(inp.u), to_dev(inp.w_in), to_dev(inp.dskip), to_dev(inp.gate_a),
                        to_dev(inp.gate_b), to_dev(inp.w_out))
    torch.cuda.synchronize()
    yn = y.cpu().numpy().astype(np.float64)
    if with_k:
        return yn, k_out.cpu().numpy().astype(np.float64)
    return yn


def _oracle_workers(inp):
    """Channel-shard processes for the oracle on large grids (1 on small ones)."""
    if inp.X * inp.Y * inp.Z * inp.B < (1 << 16):
        return 1
    from oracle._pool import default_workers
    return default_workers()


def oracle_nd(inp, conv: str = "fft"):
    import oracle
    K = oracle.nd_filter(inp.filter_params, inp.X, inp.Y, inp.Z, inp.N, inp.C, circular=inp.circular)
    y = oracle.hyena_nd_fwd(inp.u, inp.w_in, inp.dskip, inp.gate_a, inp.gate_b, inp.w_out, K, conv=conv,
                            circular=inp.circular, workers=_oracle_workers(inp) if conv == "fft" else 1)
    return y, K


def gpu_nd_film(inp, with_k: bool = False):
    """Runs hyena_nd_film_fwd on cuda:0; returns y (float64 numpy) [and the kernels
    [B, N, C, MX, MY, MZ]]."""
    import torch
    import subquadratic_sequence_amd as hs
    bd = hs.ND_CIRCULAR if inp.circular else hs.ND_ZERO_PAD
    pf = 1 if inp.circular else 2
    mx = 1 if inp.X == 1 else pf * inp.X
    m = hs.HyenaNDFilm(inp.X, inp.Y, inp.Z, inp.C, inp.N, bd, to_dev(inp.w1), to_dev(inp.b1), to_dev(inp.w2),
                       to_dev(inp.b2), to_dev(inp.w3), to_dev(inp.b3), to_dev(inp.window), to_dev(inp.q),
                       to_dev(inp.film_w), to_dev(inp.film_b), to_dev(inp.omega0))
    k_out = (torch.empty(inp.B, inp.N, inp.C, mx, pf * inp.Y, pf * inp.Z, device="cuda") if with_k else None)
    y = hs.hyena_nd_film_fwd(m, to_dev(inp.u), to_dev(inp.reg), to_dev(inp.w_in), to_dev(inp.dskip),
                             to_dev(inp.w_out), k_out=k_out)
    torch.cuda.synchronize()
    yn = y.cpu().numpy().astype(np.float64)
    if with_k:
        return yn, k_out.cpu().numpy().astype(np.float64)
    return yn


def oracle_nd_film(inp):
    """(y, Ks) of the register-conditioned oracle on the same inputs."""
    import oracle
    Ks = oracle.film_kernels(inp.film_filter_params, inp.reg, inp.q, inp.film_w, inp.film_b, inp.X, inp.Y, inp.Z,
                             inp.N, inp.C, inp.circular)
    y = oracle.hyena_nd_film_fwd(inp.u, inp.w_in, inp.dskip, inp.w_out, Ks, circular=inp.circular,
                                 workers=_oracle_workers(inp))
    return y, Ks
