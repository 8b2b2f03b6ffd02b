"""fp64 oracle for HyenaND with the page's own input conditioning: register
tokens, a softmax-weighted control vector, a FiLM-modulated SIREN kernel and a
Gaussian window (HyenaND explainer, gist.science, "Methodology: HyenaND":
"Input-Dependent Kernels via Registers and FiLM", "Kernel Synthesis", "Kernel
Parameterization").

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.

The page names the parts and how they connect, not their formulas. Readings
taken here (the plainest ones the page supports):
  * Registers: reg [B, R, C] are the layer's input activations at the R
    register tokens (prepended to the grid, so earlier layers have mixed global
    information into them). The operator reads them; it does not convolve them.
  * Control vector: z_b = sum_r w_{b,r} reg[b, r, :], with softmax weights
    w_{b,r} = softmax_r(reg[b, r, :] . q) over the registers of the sample
    (q [C], a learned score vector).
  * FiLM of the SIREN: for hidden layer l (1, 2), gamma_l = G_{2l-2}^T z + g_{2l-2}
    and beta_l = G_{2l-1}^T z + g_{2l-1} (film_w [4, C, W], film_b [4, W]);
    h_l = sin(omega_l * gamma_l * (W_l^T h_{l-1} + b_l) + beta_l), h_0 = the
    offset coordinates, omega_1 = omega0 [W] (the per-unit frequency factor
    that the block-diagonal multi-frequency initialisation sets), omega_2 = 1.
  * Kernel: o = W3^T h_2 + b3 in R^{N C}; K^n_{b,c}(d) = exp(-a_c |c(d)|^2) *
    o[(n-1) C + c] (Gaussian window, per-channel rate a_c >= 0 in `window`).
  * The per-sample kernel carries the input dependence: there is no separate
    gate, and each sample is convolved with its own kernel.
Offsets, coordinates, boundaries, projections and the recurrence are those of
hyena_nd_oracle.

The pins in tests/test_oracle_film.py tie these functions to the pinned plain
kernel, closed forms and invariants; the conventions above (score form, FiLM
placement, omega0 placement, the Gaussian rate form) are readings no page
fixes: parity unpinned for those conventions.
"""
from __future__ import annotations

import numpy as np

from .hyena_nd_oracle import (_nd_project, conv3d_circular_fft, conv3d_fft, nd_offsets, nd_recurrence)


def film_control(reg, q) -> np.ndarray:
    """z [B, C]: the softmax-weighted average of each sample's register activations."""
    reg = np.asarray(reg, dtype=np.float64)                          # [B, R, C]
    s = reg @ np.asarray(q, dtype=np.float64)                        # [B, R]
    s = s - s.max(axis=1, keepdims=True)
    w = np.exp(s)
    w = w / w.sum(axis=1, keepdims=True)
    return np.einsum("br,brc->bc", w, reg)


def film_modulation(z, film_w, film_b) -> np.ndarray:
    """[B, 4, W]: gamma_1, beta_1, gamma_2, beta_2 of every sample (affine in z)."""
    z = np.asarray(z, dtype=np.float64)
    fw = np.asarray(film_w, dtype=np.float64)                        # [4, C, W]
    return np.einsum("bc,kcw->bkw", z, fw) + np.asarray(film_b, dtype=np.float64)[None]


def nd_filter_film(params: dict, mod, X: int, Y: int, Z: int, N: int, C: int,
                   circular: bool = False) -> np.ndarray:
    """K[n, c, i, j, k] of one sample, offset-indexed like nd_filter.

    params: w1 [3, W], b1, w2 [W, W], b2, w3 [W, N C], b3, omega0 [W], window [C];
    mod [4, W]: that sample's film_modulation.
    """
    f = lambda k: np.asarray(params[k], dtype=np.float64)  # noqa: E731
    mod = np.asarray(mod, dtype=np.float64)
    c = nd_offsets(X, Y, Z, circular)
    h1 = np.sin(f("omega0") * mod[0] * (c @ f("w1") + f("b1")) + mod[1])
    h2 = np.sin(mod[2] * (h1 @ f("w2") + f("b2")) + mod[3])
    o = h2 @ f("w3") + f("b3")                                       # [MX, MY, MZ, N C]
    r2 = np.sum(c * c, axis=-1)
    win = np.exp(-r2[..., None] * f("window"))                      # [MX, MY, MZ, C]
    K = o.reshape(o.shape[:3] + (N, C)) * win[..., None, :]
    return np.ascontiguousarray(np.moveaxis(K, (3, 4), (0, 1)))


def film_kernels(params: dict, reg, q, film_w, film_b, X, Y, Z, N, C, circular=False) -> np.ndarray:
    """[B, N, C, MX, MY, MZ]: every sample's kernel."""
    mod = film_modulation(film_control(reg, q), film_w, film_b)
    return np.stack([nd_filter_film(params, mod[b], X, Y, Z, N, C, circular) for b in range(mod.shape[0])])


def hyena_nd_film_fwd(u, w_in, dskip, w_out, Ks, conv: str = "fft", circular: bool = False,
                      workers: int = 1) -> np.ndarray:
    """y[B, X, Y, Z, C]; Ks [B, N, C, MX, MY, MZ] from film_kernels.

    z^1 = v; z^{n+1} = x^n * (K^n_b conv z^n) + D^n * z^n; y = z^{N+1} W_out.
    workers > 1 runs the recurrence on channel shards in that many processes.
    """
    B, X, Y, Z, C = np.shape(u)
    N = np.shape(dskip)[0]
    dskip = np.asarray(dskip, dtype=np.float64)
    Ks = np.asarray(Ks, dtype=np.float64)
    z, xs = _nd_project(u, w_in, C, N)
    if workers > 1:
        from ._pool import channel_shards
        z = channel_shards(nd_recurrence, C, workers,
                           lambda sl: (z[:, sl], [x[:, sl] for x in xs], dskip[:, sl], Ks[:, :, sl], conv, circular))
    else:
        z = nd_recurrence(z, xs, dskip, Ks, conv, circular)
    return np.moveaxis(z, 1, -1) @ np.asarray(w_out, dtype=np.float64)


def hyena_nd_film_fwd_sampled(u, w_in, dskip, w_out, Ks, points, chunk: int = 8,
                              circular: bool = False) -> np.ndarray:
    """y[:, points] for full-size grids ([B, S, C]): orders 1..N-1 on the whole
    grid by FFT (channel chunks of `chunk`), the last order only at the sampled
    points by the direct sum over the grid."""
    B, X, Y, Z, C = np.shape(u)
    N = np.shape(dskip)[0]
    dskip = np.asarray(dskip, dtype=np.float64)
    z, xs = _nd_project(u, w_in, C, N)
    convf = conv3d_circular_fft if circular else conv3d_fft
    for n in range(N - 1):
        out = np.empty_like(z)
        for b in range(B):
            Kb = np.asarray(Ks[b, n], dtype=np.float64)
            for c0 in range(0, C, chunk):
                out[b, c0:c0 + chunk] = convf(Kb[c0:c0 + chunk], z[b, c0:c0 + chunk])
        z = xs[n] * out + dskip[n][None, :, None, None, None] * z
    n = N - 1
    pts = np.asarray(points, dtype=np.int64)
    res = np.empty((B, len(pts), C))
    for b in range(B):
        Kb = np.asarray(Ks[b, n], dtype=np.float64)
        for i, (px, py, pz) in enumerate(pts):
            if circular:
                ix = (px - np.arange(X) + X // 2) % X
                iy = (py - np.arange(Y) + Y // 2) % Y
                iz = (pz - np.arange(Z) + Z // 2) % Z
                ks = Kb[:, ix[:, None, None], iy[None, :, None], iz[None, None, :]]
            else:
                ks = Kb[:, px + X:px:-1, py + Y:py:-1, pz + Z:pz:-1]
            c = np.einsum("cxyz,cxyz->c", ks, z[b])
            res[b, i, :] = xs[n][b, :, px, py, pz] * c + dskip[n] * z[b, :, px, py, pz]
    return res @ np.asarray(w_out, dtype=np.float64)
