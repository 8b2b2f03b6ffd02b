"""fp64 oracle for the 3D HyenaND operator (channels-last grids).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.

What it computes (HyenaND explainer, gist.science, "Methodology: HyenaND"):
  * a global convolution evaluated natively on the 3D grid (Native ND
    Convolution), non-circular, by zero padding the input to twice the grid
    before the FFT ("Handling Boundaries");
  * a continuous kernel given by a coordinate MLP with sine activations times a
    window ("Kernel Synthesis"; here an exponential radial window);
  * input dependence at the level of the whole sample ("Input-Dependent
    Kernels"; here a sigmoid of a linear map of each channel's grid mean of u
    scales the whole kernel of that channel);
  * the same projection / gating recurrence as the 1D operator, without the
    short convolution.

Geometry, zero-padded boundary (non-circular, the default): the kernel is
defined on signed offsets d in [-G, G) per axis (G the grid size of that axis)
at coordinates c = d / G, and out[p] = sum_{q in grid} g * K[p - q] * z[q] for p
in the grid.  conv3d_fft stores the kernel wrapped (index d mod 2G) in a
(2X, 2Y, 2Z) array, which makes the circular convolution of the zero-padded
input exact on the kept grid.

2D grids (image planes) are the same operator with X = 1: every offset has
dx = 0 (coordinate 0), so only the kernel's dx = 0 slice acts (the zero-padded
array still holds the unused dx = -1 slice).

Geometry, circular boundary (periodic grids; "Handling Boundaries" names both
kinds): the kernel covers one period, signed offsets d in [-G/2, G/2) per axis
at coordinates c = d / (G/2), so that in both modes the coordinates span
[-1, 1) over the kernel's support; out[p] = sum_{q in grid} g * K[(p - q) mod G]
* z[q] for every p, evaluated with an unpadded (X, Y, Z) FFT.  In both modes the
offset-indexed arrays hold offset d at index d + M/2, M the transform length of
the axis (2G padded, G circular).

Window form, MLP width, gate form, coordinate scaling and initialisation are
conventions of this implementation: parity unpinned for those conventions.
"""
from __future__ import annotations

import numpy as np

from .hyena_oracle import fft_radix2


def fftn3_radix2(x, inverse: bool = False) -> np.ndarray:
    """3D DFT over the last three axes, one textbook radix-2 pass per axis."""
    a = np.asarray(x, dtype=np.complex128)
    for ax in (-1, -2, -3):
        a = np.moveaxis(fft_radix2(np.moveaxis(a, ax, -1), inverse=inverse), -1, ax)
    return a


def nd_offsets(X: int, Y: int, Z: int, circular: bool = False) -> np.ndarray:
    """Coordinates of the kernel's signed offsets, [MX, MY, MZ, 3].

    Zero-padded: M = 2G, offsets d in [-G, G), c = d / G.  Circular: M = G,
    offsets d in [-G/2, G/2), c = d / (G/2).  Entry [i, j, k] is the offset
    (i - MX/2, j - MY/2, k - MZ/2) in both modes.
    """
    axes = []
    for G in (X, Y, Z):
        h = G // 2 if circular else G
        # a one-point periodic axis has the single offset 0 (coordinate 0)
        axes.append(np.arange(-h, h, dtype=np.float64) / h if h else np.zeros(1))
    g = np.stack(np.meshgrid(*axes, indexing="ij"), axis=-1)
    return g


def nd_filter(params: dict, X: int, Y: int, Z: int, N: int, C: int, circular: bool = False) -> np.ndarray:
    """K[n, c, i, j, k] at offset (i - X, j - Y, k - Z):
    K = exp(-a_c |coord|_2) * (W3^T sin(W2^T sin(W1^T coord + b1) + b2) + b3)[n*C + c].

    Returns [N, C, MX, MY, MZ] float64 (offset-indexed, not wrapped): (2X, 2Y, 2Z)
    zero-padded, (X, Y, Z) circular.
    """
    f = lambda k: np.asarray(params[k], dtype=np.float64)  # noqa: E731
    c = nd_offsets(X, Y, Z, circular)
    a1 = np.sin(c @ f("w1") + f("b1"))
    a2 = np.sin(a1 @ f("w2") + f("b2"))
    o = a2 @ f("w3") + f("b3")                                       # [MX,MY,MZ,N*C]
    r = np.sqrt(np.sum(c * c, axis=-1))
    win = np.exp(-r[..., None] * f("decay"))                         # [MX,MY,MZ,C]
    K = o.reshape(o.shape[:3] + (N, C)) * win[..., None, :]
    return np.ascontiguousarray(np.moveaxis(K, (3, 4), (0, 1)))


def nd_gate(u, gate_a, gate_b) -> np.ndarray:
    """g[b, n, c] = sigmoid(a[n, c] * mean_grid(u[b, ..., c]) + b[n, c])."""
    u = np.asarray(u, dtype=np.float64)
    m = u.mean(axis=(1, 2, 3))                                       # [B, C]
    s = np.asarray(gate_a, np.float64)[None] * m[:, None, :] + np.asarray(gate_b, np.float64)[None]
    return 1.0 / (1.0 + np.exp(-s))


def conv3d_direct(K, z) -> np.ndarray:
    """out[..., p] = sum_{q in grid} K[..., p - q + G] * z[..., q]  (definition).

    K [..., 2X, 2Y, 2Z] offset-indexed; z [..., X, Y, Z].  O(G^6); for small grids.
    """
    K = np.asarray(K, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    X, Y, Z = z.shape[-3:]
    out = np.zeros(np.broadcast_shapes(K.shape[:-3], z.shape[:-3]) + (X, Y, Z))
    for qx in range(X):
        for qy in range(Y):
            for qz in range(Z):
                # offsets p - q for all p: index (p - q) + G = p + (G - q)
                kslab = K[..., X - qx:2 * X - qx, Y - qy:2 * Y - qy, Z - qz:2 * Z - qz]
                out += kslab * z[..., qx, qy, qz][..., None, None, None]
    return out


def conv3d_fft(K, z) -> np.ndarray:
    """Same result as conv3d_direct via a (2X, 2Y, 2Z) textbook FFT.

    The offset-indexed kernel is wrapped (offset d stored at d mod 2G), the input
    is zero padded to (2X, 2Y, 2Z), and the first X*Y*Z outputs are kept.
    """
    K = np.asarray(K, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    X, Y, Z = z.shape[-3:]
    Kw = np.roll(K, shift=(-X, -Y, -Z), axis=(-3, -2, -1))
    zp = np.zeros(z.shape[:-3] + (2 * X, 2 * Y, 2 * Z))
    zp[..., :X, :Y, :Z] = z
    c = fftn3_radix2(fftn3_radix2(Kw) * fftn3_radix2(zp), inverse=True)
    return c[..., :X, :Y, :Z].real


def conv3d_circular_direct(K, z) -> np.ndarray:
    """out[..., p] = sum_{q in grid} K[..., (p - q) mod G as an offset] * z[..., q]  (definition).

    K [..., X, Y, Z] offset-indexed (offset d at index d + G/2, d in [-G/2, G/2));
    z [..., X, Y, Z].  The offset (p - q) mod G, taken in [-G/2, G/2), sits at
    index (p - q + G/2) mod G.  O(G^6); for small grids.
    """
    K = np.asarray(K, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    X, Y, Z = z.shape[-3:]
    out = np.zeros(np.broadcast_shapes(K.shape[:-3], z.shape[:-3]) + (X, Y, Z))
    for qx in range(X):
        for qy in range(Y):
            for qz in range(Z):
                # slab[p] = K[(p - q + G/2) mod G] = roll(K, q - G/2)[p]
                slab = np.roll(K, shift=(qx - X // 2, qy - Y // 2, qz - Z // 2), axis=(-3, -2, -1))
                out += slab * z[..., qx, qy, qz][..., None, None, None]
    return out


def conv3d_circular_fft(K, z) -> np.ndarray:
    """Same result as conv3d_circular_direct via an (X, Y, Z) textbook FFT.

    The offset-indexed kernel is wrapped (offset d stored at d mod G); no padding,
    no crop: the DFT's own circular convolution is the periodic one.
    """
    K = np.asarray(K, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    X, Y, Z = z.shape[-3:]
    Kw = np.roll(K, shift=(-(X // 2), -(Y // 2), -(Z // 2)), axis=(-3, -2, -1))
    c = fftn3_radix2(fftn3_radix2(Kw) * fftn3_radix2(z), inverse=True)
    return c.real


def _nd_project(u, w_in, C, N):
    u = np.asarray(u, dtype=np.float64)
    p = u @ np.asarray(w_in, dtype=np.float64)                       # [B,X,Y,Z,(N+1)C]
    blocks = [np.ascontiguousarray(np.moveaxis(p[..., i * C:(i + 1) * C], -1, 1))
              for i in range(N + 1)]                                 # [B, C, X, Y, Z]
    return blocks[0], blocks[1:]


def nd_recurrence(z, xs, dskip, Kg, conv: str = "fft", circular: bool = False) -> np.ndarray:
    """z^{N+1} from z^1 = v on channel-major grids: for every sample b,
    z^{n+1}_b = x^n_b * (Kg[b, n] conv z^n_b) + D^n * z^n_b.

    z [B, C, X, Y, Z]; xs: N arrays like z; dskip [N, C]; Kg [B, N, C, MX, MY, MZ]
    (a sample's kernels: the gated kernel g * K, or its own conditioned kernel).
    Channels are independent, so any channel subset can be run alone.
    """
    if circular:
        convf = conv3d_circular_direct if conv == "direct" else conv3d_circular_fft
    else:
        convf = conv3d_direct if conv == "direct" else conv3d_fft
    dskip = np.asarray(dskip, dtype=np.float64)
    for n in range(len(xs)):
        out = np.empty_like(z)
        for b in range(z.shape[0]):
            out[b] = convf(np.asarray(Kg[b][n], dtype=np.float64), z[b])
        z = xs[n] * out + dskip[n][None, :, None, None, None] * z
    return z


def _nd_gated_recurrence(z, xs, dskip, g, K, conv, circular):
    """nd_recurrence with the kernels g[b, n, c] * K[n, c] of the channel-mean gate."""
    K = np.asarray(K, dtype=np.float64)
    Kg = [g[b][:, :, None, None, None] * K for b in range(z.shape[0])]
    return nd_recurrence(z, xs, dskip, Kg, conv, circular)


def hyena_nd_fwd(u, w_in, dskip, gate_a, gate_b, w_out, K, conv: str = "fft",
                 circular: bool = False, workers: int = 1) -> np.ndarray:
    """y[B, X, Y, Z, C] of the 3D operator.

    u [B,X,Y,Z,C]; w_in [C,(N+1)C]; dskip, gate_a, gate_b [N,C]; w_out [C,C];
    K [N, C, MX, MY, MZ] (nd_filter with the same `circular`).  conv: "direct" or
    "fft".  workers > 1 runs the recurrence on channel shards in that many processes.
    """
    B, X, Y, Z, C = np.shape(u)
    N = np.shape(dskip)[0]
    dskip = np.asarray(dskip, dtype=np.float64)
    g = nd_gate(u, gate_a, gate_b)                                   # [B, N, C]
    z, xs = _nd_project(u, w_in, C, N)
    K = np.asarray(K, dtype=np.float64)
    if workers > 1:
        from ._pool import channel_shards
        z = channel_shards(_nd_gated_recurrence, C, workers,
                           lambda sl: (z[:, sl], [x[:, sl] for x in xs], dskip[:, sl], g[:, :, sl], K[:, sl],
                                       conv, circular))
    else:
        z = _nd_gated_recurrence(z, xs, dskip, g, K, conv, circular)
    return np.moveaxis(z, 1, -1) @ np.asarray(w_out, dtype=np.float64)


def hyena_nd_fwd_sampled(u, w_in, dskip, gate_a, gate_b, w_out, K, points, chunk: int = 8,
                         circular: bool = False) -> np.ndarray:
    """y[:, points] for full-size grids.

    Orders 1..N-1 run on the whole grid with conv3d_fft / conv3d_circular_fft
    (channel chunks of `chunk`); the last order is evaluated only at the sampled
    grid points by the direct sum over the grid.  points [S, 3] integer grid
    coordinates.  Returns [B, S, C].
    """
    B, X, Y, Z, C = np.shape(u)
    N = np.shape(dskip)[0]
    dskip = np.asarray(dskip, dtype=np.float64)
    g = nd_gate(u, gate_a, gate_b)
    z, xs = _nd_project(u, w_in, C, N)
    K = np.asarray(K, dtype=np.float64)
    for n in range(N - 1):
        out = np.empty_like(z)
        for b in range(B):
            for c0 in range(0, C, chunk):
                gk = g[b, n, c0:c0 + chunk][:, None, None, None] * K[n, c0:c0 + chunk]
                convf = conv3d_circular_fft if circular else conv3d_fft
                out[b, c0:c0 + chunk] = convf(gk, z[b, c0:c0 + chunk])
        z = xs[n] * out + dskip[n][None, :, None, None, None] * z
    n = N - 1
    pts = np.asarray(points, dtype=np.int64)
    res = np.empty((B, len(pts), C))
    for i, (px, py, pz) in enumerate(pts):
        if circular:
            # offset (p - q) mod G at index (p - q + G/2) mod G, for q over the grid
            ix = (px - np.arange(X) + X // 2) % X
            iy = (py - np.arange(Y) + Y // 2) % Y
            iz = (pz - np.arange(Z) + Z // 2) % Z
            ks = K[n][:, ix[:, None, None], iy[None, :, None], iz[None, None, :]]
        else:
            # K offsets p - q for q over the grid: index (p - q) + G, flipped slab
            ks = K[n][:, px + X:px:-1, py + Y:py:-1, pz + Z:pz:-1]    # [C, X, Y, Z] over q
        c = np.einsum("cxyz,bcxyz->bc", ks, z) * g[:, n, :]
        res[:, i, :] = xs[n][:, :, px, py, pz] * c + dskip[n][None, :] * z[:, :, px, py, pz]
    return res @ np.asarray(w_out, dtype=np.float64)
