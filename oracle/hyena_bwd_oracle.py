"""fp64 oracle for the backward pass of the 1D Hyena operator (its vector-Jacobian
product) and of the implicit filter generator.

TEST INFRASTRUCTURE ONLY: imported by tests/ and bench.py's cpu_baseline leg,
never by the product path.

The pages' speed and compute claims are training claims (Hyena Hierarchy
abstract: less training compute at sequence length 2K; HyenaDNA abstract:
faster training at long contexts), so the operator is differentiated. The pages
give no backward formulas; what follows is the chain rule applied to the
forward steps of hyena_oracle, in reverse order, for a scalar loss whose
gradient with respect to y is dy:

  y = z^{N+1} W_out:          dW_out = sum_b (z^{N+1}_b)^T dy_b,   g = dy W_out^T
  z^{n+1} = x^n c^n + D^n z^n, c^n = h^n conv z^n   (n = N .. 1, g = dz^{n+1}):
      dx^n = g c^n,  dc = g x^n,  dD^n_c = sum_{b,t} g z^n,
      dz^n = D^n g + (h^n conv^T dc),  dh^n = sum_b (dc xcorr z^n)
  where the transpose of the causal convolution is the correlation
      (h conv^T g)(t) = sum_{tau >= 0} h(tau) g(t + tau)          (g zero past L - 1)
  and the filter gradient is the cross-correlation
      (g xcorr z)(tau) = sum_t g(t) z(t - tau)                     (z zero before 0);
  two-sided filters take the same sums over signed lags.
  s = short conv of p:       dp_j(t) = sum_k w[j,k] ds_j(t + k),  dw[j,k] = sum_{b,t} ds_j(t) p_j(t - k)
  p = u W_in:                du = dp W_in^T,  dW_in = sum_b u_b^T dp_b
  with ds = (dz^1, dx^1, .., dx^N) in the block order of W_in's columns.

The correlations are evaluated directly (their definitions) or through the
convolution theorem with the textbook FFT of hyena_oracle: a correlation is a
product with the conjugate spectrum, and the same zero padding to 2L keeps the
circular result equal to the linear one on the kept outputs.

The filter generator h[n, c, t] = exp(-a_c |tau|) o(tau)[n D + c],
o = W3^T sin(W2^T sin(W1^T e + b1) + b2) + b3, is differentiated the same way
(implicit_filter_bwd).
"""
from __future__ import annotations

import numpy as np

from .hyena_oracle import (_project_and_gate_inputs, causal_conv_direct, causal_conv_fft, fft_radix2,
                           noncausal_conv_direct, noncausal_conv_fft, posenc_at)


# ---------------------------------------------------------------------------
# Transposed long convolutions
# ---------------------------------------------------------------------------

def causal_corr_direct(h, g) -> np.ndarray:
    """out[..., t] = sum_{tau=0..L-1-t} h[..., tau] * g[..., t + tau]  (definition)."""
    h = np.asarray(h, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    L = g.shape[-1]
    out = np.zeros(np.broadcast_shapes(h.shape, g.shape), dtype=np.float64)
    for tau in range(L):
        out[..., :L - tau] += h[..., tau:tau + 1] * g[..., tau:]
    return out


def causal_xcorr_direct(g, z) -> np.ndarray:
    """out[..., tau] = sum_{t=tau..L-1} g[..., t] * z[..., t - tau]  (definition)."""
    g = np.asarray(g, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    L = z.shape[-1]
    out = np.zeros(np.broadcast_shapes(g.shape, z.shape), dtype=np.float64)
    for tau in range(L):
        out[..., tau] = np.sum(g[..., tau:] * z[..., :L - tau], axis=-1)
    return out


def noncausal_corr_direct(h2, g) -> np.ndarray:
    """out[..., t] = sum_{tau=-(L-1)..L-1} h2[..., tau + L - 1] * g[..., t + tau], g zero outside [0, L)."""
    h2 = np.asarray(h2, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    L = g.shape[-1]
    out = np.zeros(np.broadcast_shapes(h2.shape[:-1] + (L,), g.shape), dtype=np.float64)
    for tau in range(-(L - 1), L):
        hv = h2[..., tau + L - 1:tau + L]
        if tau >= 0:
            out[..., :L - tau] += hv * g[..., tau:]
        else:
            out[..., -tau:] += hv * g[..., :L + tau]
    return out


def noncausal_xcorr_direct(g, z) -> np.ndarray:
    """out[..., i] = sum_t g[..., t] * z[..., t - tau] at lag tau = i - (L - 1), z zero outside [0, L)."""
    g = np.asarray(g, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    L = z.shape[-1]
    out = np.zeros(np.broadcast_shapes(g.shape, z.shape)[:-1] + (2 * L - 1,), dtype=np.float64)
    for tau in range(-(L - 1), L):
        if tau >= 0:
            out[..., tau + L - 1] = np.sum(g[..., tau:] * z[..., :L - tau], axis=-1)
        else:
            out[..., tau + L - 1] = np.sum(g[..., :L + tau] * z[..., -tau:], axis=-1)
    return out


def _pad2(x) -> np.ndarray:
    return np.concatenate([x, np.zeros(x.shape[:-1] + (x.shape[-1],))], axis=-1)


def _wrap(h2) -> np.ndarray:
    """Lag-indexed [..., 2L - 1] -> [..., 2L] with lag tau at tau mod 2L (entry L zero)."""
    L = (h2.shape[-1] + 1) // 2
    hw = np.zeros(h2.shape[:-1] + (2 * L,))
    hw[..., :L] = h2[..., L - 1:]
    hw[..., L + 1:] = h2[..., :L - 1]
    return hw


def causal_corr_fft(h, g) -> np.ndarray:
    """causal_corr_direct through a 2L-point FFT: inverse of conj(FFT(h)) * FFT(g), first L."""
    h = np.asarray(h, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    L = g.shape[-1]
    c = fft_radix2(np.conj(fft_radix2(_pad2(h))) * fft_radix2(_pad2(g)), inverse=True)
    return c[..., :L].real


def causal_xcorr_fft(g, z) -> np.ndarray:
    """causal_xcorr_direct through a 2L-point FFT: inverse of FFT(g) * conj(FFT(z)), first L."""
    g = np.asarray(g, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    L = z.shape[-1]
    c = fft_radix2(fft_radix2(_pad2(g)) * np.conj(fft_radix2(_pad2(z))), inverse=True)
    return c[..., :L].real


def noncausal_corr_fft(h2, g) -> np.ndarray:
    """noncausal_corr_direct through a 2L-point FFT with the filter wrapped."""
    h2 = np.asarray(h2, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    L = g.shape[-1]
    c = fft_radix2(np.conj(fft_radix2(_wrap(h2))) * fft_radix2(_pad2(g)), inverse=True)
    return c[..., :L].real


def noncausal_xcorr_fft(g, z) -> np.ndarray:
    """noncausal_xcorr_direct through a 2L-point FFT; lag tau read at tau mod 2L."""
    g = np.asarray(g, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    L = z.shape[-1]
    c = fft_radix2(fft_radix2(_pad2(g)) * np.conj(fft_radix2(_pad2(z))), inverse=True).real
    return np.concatenate([c[..., L + 1:], c[..., :L]], axis=-1)   # lags -(L-1) .. L-1


def _corr_fns(conv: str, causal: bool, L: int):
    if conv == "auto":
        conv = "direct" if L <= 1024 else "fft"
    if causal:
        return (causal_corr_direct, causal_xcorr_direct) if conv == "direct" else (causal_corr_fft, causal_xcorr_fft)
    if conv == "direct":
        return noncausal_corr_direct, noncausal_xcorr_direct
    return noncausal_corr_fft, noncausal_xcorr_fft


def _conv_fns(conv: str, causal: bool, L: int):
    if conv == "auto":
        conv = "direct" if L <= 1024 else "fft"
    if causal:
        return causal_conv_direct if conv == "direct" else causal_conv_fft
    return noncausal_conv_direct if conv == "direct" else noncausal_conv_fft


# ---------------------------------------------------------------------------
# Operator backward
# ---------------------------------------------------------------------------

def short_conv_bwd(p, ds, w):
    """(dp, dw) of s = short_conv(p, w) for the upstream gradient ds; p, ds [B, L, J]."""
    p = np.asarray(p, dtype=np.float64)
    ds = np.asarray(ds, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dp = w[:, 0] * ds
    dp[:, :-1] += w[:, 1] * ds[:, 1:]
    dp[:, :-2] += w[:, 2] * ds[:, 2:]
    dw = np.zeros_like(w)
    dw[:, 0] = np.sum(ds * p, axis=(0, 1))
    dw[:, 1] = np.sum(ds[:, 1:] * p[:, :-1], axis=(0, 1))
    dw[:, 2] = np.sum(ds[:, 2:] * p[:, :-2], axis=(0, 1))
    return dp, dw


def hyena_bwd(u, w_in, short_w, dskip, w_out, h, dy, conv: str = "auto", causal: bool = True) -> dict:
    """Gradients of sum(dy * y), y = hyena_fwd(u, w_in, short_w, dskip, w_out, h).

    Returns dict(du [B,L,D], dw_in [D,(N+1)D], dshort_w [(N+1)D,3], ddskip [N,D],
    dw_out [D,D], dh like h: [N,D,L] causal, [N,D,2L-1] lag-indexed two-sided).
    conv: "direct", "fft" or "auto" (direct up to L = 1024).
    """
    B, L, D = np.shape(u)
    N = np.shape(dskip)[0]
    corr, xcorr = _corr_fns(conv, causal, L)
    convf = _conv_fns(conv, causal, L)
    u = np.asarray(u, dtype=np.float64)
    w_in = np.asarray(w_in, dtype=np.float64)
    w_out = np.asarray(w_out, dtype=np.float64)
    dskip = np.asarray(dskip, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)

    # forward, keeping every order's input and convolution
    p = u @ w_in
    z, xs = _project_and_gate_inputs(u, w_in, short_w, D, N)
    zs, cs = [z], []
    for n in range(N):
        c = convf(h[n][None], zs[-1])
        cs.append(c)
        zs.append(xs[n] * c + dskip[n][None, :, None] * zs[-1])

    # backward
    dw_out = np.tensordot(zs[N], dy, axes=([0, 2], [0, 1]))              # sum over b, t
    g = np.ascontiguousarray((dy @ w_out.T).transpose(0, 2, 1))          # dz^{N+1}, [B, D, L]
    dxs = [None] * N
    ddskip = np.zeros((N, D))
    dh = np.zeros_like(h)
    for n in range(N - 1, -1, -1):
        dxs[n] = g * cs[n]
        dc = g * xs[n]
        ddskip[n] = np.sum(g * zs[n], axis=(0, 2))
        dh[n] = np.sum(xcorr(dc, zs[n]), axis=0)
        g = dskip[n][None, :, None] * g + corr(h[n][None], dc)
    ds_cm = np.concatenate([g] + dxs, axis=1)                              # [B, (N+1)D, L]
    dp, dshort = short_conv_bwd(p, ds_cm.transpose(0, 2, 1), short_w)
    du = dp @ w_in.T
    dw_in = np.tensordot(u, dp, axes=([0, 1], [0, 1]))                  # sum over b, t
    return dict(du=du, dw_in=dw_in, dshort_w=dshort, ddskip=ddskip, dw_out=dw_out, dh=dh)


# ---------------------------------------------------------------------------
# Filter generator backward
# ---------------------------------------------------------------------------

def _filter_bwd_at(params: dict, tau, N: int, D: int, dh) -> dict:
    f = lambda k: np.asarray(params[k], dtype=np.float64)  # noqa: E731
    tau = np.asarray(tau, dtype=np.float64)
    dh = np.asarray(dh, dtype=np.float64)                            # [N, D, P]
    P = len(tau)
    e = posenc_at(tau, int(params["K"]))                             # [P, F]
    q1 = e @ f("w1") + f("b1")
    a1 = np.sin(q1)
    q2 = a1 @ f("w2") + f("b2")
    a2 = np.sin(q2)
    o = a2 @ f("w3") + f("b3")                                       # [P, N D]
    win = np.exp(-np.outer(np.abs(tau), f("decay")))                 # [P, D]
    dhp = dh.transpose(2, 0, 1)                                      # [P, N, D]
    do = (dhp * win[:, None, :]).reshape(P, N * D)                   # dL/do
    # h = win * o, d win / d a_c = -|tau| win
    ddecay = np.sum(dhp * o.reshape(P, N, D) * (-np.abs(tau)[:, None, None] * win[:, None, :]), axis=(0, 1))
    dw3 = a2.T @ do
    db3 = do.sum(0)
    dq2 = (do @ f("w3").T) * np.cos(q2)
    dw2 = a1.T @ dq2
    db2 = dq2.sum(0)
    dq1 = (dq2 @ f("w2").T) * np.cos(q1)
    dw1 = e.T @ dq1
    db1 = dq1.sum(0)
    return dict(w1=dw1, b1=db1, w2=dw2, b2=db2, w3=dw3, b3=db3, decay=ddecay)


def implicit_filter_bwd(params: dict, L: int, N: int, D: int, dh) -> dict:
    """Gradients of sum(dh * h), h = implicit_filter(params, L, N, D), with respect
    to w1, b1, w2, b2, w3, b3 and decay."""
    return _filter_bwd_at(params, np.arange(L, dtype=np.float64) / L, N, D, dh)


def implicit_filter_noncausal_bwd(params: dict, L: int, N: int, D: int, dh2) -> dict:
    """The same for implicit_filter_noncausal (dh2 lag-indexed [N, D, 2L - 1])."""
    return _filter_bwd_at(params, np.arange(-(L - 1), L, dtype=np.float64) / L, N, D, dh2)
