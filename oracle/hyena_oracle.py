"""fp64 oracle for the 1D Hyena operator.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.

What it computes (every step in float64, on the stored input values upcast to
float64, with no intermediate rounding):

  1. p = u W_in, split into column blocks (v, x^1, ..., x^N).
  2. A causal depthwise short convolution of length 3 on every projected channel.
  3. The implicit filters h^n_c(t) = window_c(t) * FFN(PosEnc(t))[(n-1)D + c]
     (an MLP parameterises the long filter: TWIML #690 podcast, 4:29; the filter
     is as long as the input: TWIML #690, 5:48).
  4. The order-N recurrence z^1 = v, z^{n+1} = x^n * (h^n conv z^n) + D^n * z^n,
     i.e. long convolutions interleaved with data-controlled gating (Hyena
     Hierarchy abstract). The convolution is causal (next-token prediction
     "causal style": TWIML #690, 20:00).
  5. y = z^{N+1} W_out.

The long convolution is evaluated either directly (the O(L^2) definition; TWIML
#690, 5:48) or through the convolution theorem with a textbook radix-2 FFT of
size 2L (zero padding to twice the length makes the circular convolution equal
the linear one: HyenaND explainer, Methodology, "Handling Boundaries"; FFT
convolution: TWIML #690, 6:27).

Non-causal (bidirectional) variant: the pages only name causal use and
bidirectional comparators, so its form here is a reading: the same generator
evaluated at signed lags tau in [-(L-1), L-1] (PosEnc at tau / L, window
exp(-a_c |tau| / L)), and c_t = sum_tau h(tau) z_{t - tau} with z zero outside
[0, L); the 2L-point FFT with the filter wrapped (lag tau at tau mod 2L) gives it
exactly. The short convolution keeps its causal taps.

Readings of points the pages leave open (positional-encoding frequencies, FFN
initialisation, window decays, short-conv taps, skip placement, block order) are
conventions of this implementation; the tests pin the code to those
conventions, but no page fixes them: parity unpinned for those conventions.
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------
# Textbook FFT
# ---------------------------------------------------------------------------

def _bit_reverse_indices(n: int) -> np.ndarray:
    bits = n.bit_length() - 1
    idx = np.arange(n, dtype=np.int64)
    rev = np.zeros(n, dtype=np.int64)
    for b in range(bits):
        rev |= ((idx >> b) & 1) << (bits - 1 - b)
    return rev


def fft_radix2(x, inverse: bool = False) -> np.ndarray:
    """Iterative radix-2 Cooley-Tukey DFT along the last axis (power-of-two length).

    Forward: X[k] = sum_n x[n] exp(-2 pi i n k / n_len). Inverse uses exp(+...)
    and divides by n_len. Bit-reversal reordering, then log2(n) stages of
    decimation-in-time butterflies X[k] = E[k] + w^k O[k], X[k+m] = E[k] - w^k O[k].
    """
    a = np.asarray(x, dtype=np.complex128)
    n = a.shape[-1]
    if n < 1 or n & (n - 1):
        raise ValueError("length must be a power of two")
    lead = a.shape[:-1]
    a = np.ascontiguousarray(a[..., _bit_reverse_indices(n)])
    sign = 1.0 if inverse else -1.0
    m = 1
    while m < n:
        w = np.exp(sign * 1j * np.pi * np.arange(m) / m)
        g = a.reshape(lead + (n // (2 * m), 2, m))   # view: [group][even|odd half][k]
        wo = g[..., 1, :] * w
        g[..., 1, :] = g[..., 0, :] - wo
        g[..., 0, :] += wo
        m *= 2
    if inverse:
        a = a / n
    return a


# ---------------------------------------------------------------------------
# Long causal convolution
# ---------------------------------------------------------------------------

def causal_conv_direct(h, z) -> np.ndarray:
    """c[..., t] = sum_{s=0..t} h[..., s] * z[..., t - s]  (definition, O(L^2)).

    h and z are broadcast against each other; the last axis is time.
    """
    h = np.asarray(h, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    L = z.shape[-1]
    out = np.zeros(np.broadcast_shapes(h.shape, z.shape), dtype=np.float64)
    for s in range(L):
        out[..., s:] += h[..., s:s + 1] * z[..., :L - s]
    return out


def causal_conv_fft(h, z) -> np.ndarray:
    """Same result as causal_conv_direct, via the convolution theorem.

    Both operands are zero padded to 2L, transformed with fft_radix2, multiplied
    pointwise, transformed back, and the first L samples are kept.
    """
    h = np.asarray(h, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    L = z.shape[-1]
    hp = np.concatenate([h, np.zeros(h.shape[:-1] + (L,))], axis=-1)
    zp = np.concatenate([z, np.zeros(z.shape[:-1] + (L,))], axis=-1)
    c = fft_radix2(fft_radix2(hp) * fft_radix2(zp), inverse=True)
    return c[..., :L].real


def noncausal_conv_direct(h2, z) -> np.ndarray:
    """c[..., t] = sum_{tau=-(L-1)..L-1} h2[..., tau + L - 1] * z[..., t - tau], z = 0 outside [0, L)
    (definition, O(L^2)).  h2 [..., 2L - 1] is lag-indexed: entry i holds lag i - (L - 1)."""
    h2 = np.asarray(h2, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    L = z.shape[-1]
    out = np.zeros(np.broadcast_shapes(h2.shape[:-1] + (L,), z.shape), dtype=np.float64)
    for tau in range(-(L - 1), L):
        hv = h2[..., tau + L - 1:tau + L]
        if tau >= 0:
            out[..., tau:] += hv * z[..., :L - tau]
        else:
            out[..., :L + tau] += hv * z[..., -tau:]
    return out


def noncausal_conv_fft(h2, z) -> np.ndarray:
    """Same result as noncausal_conv_direct via a 2L-point FFT: the filter wrapped
    (lag tau at index tau mod 2L, index L zero), the input zero padded to 2L, the
    first L samples kept."""
    h2 = np.asarray(h2, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    L = z.shape[-1]
    hw = np.zeros(h2.shape[:-1] + (2 * L,))
    hw[..., :L] = h2[..., L - 1:]                  # lags 0 .. L-1
    hw[..., L + 1:] = h2[..., :L - 1]              # lags -(L-1) .. -1 at 2L + tau
    zp = np.concatenate([z, np.zeros(z.shape[:-1] + (L,))], axis=-1)
    c = fft_radix2(fft_radix2(hw) * fft_radix2(zp), inverse=True)
    return c[..., :L].real


# ---------------------------------------------------------------------------
# Implicit filter
# ---------------------------------------------------------------------------

def posenc_at(tau, K: int) -> np.ndarray:
    """Features [tau, cos(2 pi k tau) for k=1..K, sin(2 pi k tau) for k=1..K] at the
    given normalised positions tau.  Returns [len(tau), 1 + 2K]."""
    tau = np.asarray(tau, dtype=np.float64)
    ang = 2.0 * np.pi * np.outer(tau, np.arange(1, K + 1, dtype=np.float64))
    return np.concatenate([tau[:, None], np.cos(ang), np.sin(ang)], axis=1)


def posenc(L: int, K: int) -> np.ndarray:
    """Features of position t at tau = t / L, t in [0, L).  Returns [L, 1 + 2K]."""
    return posenc_at(np.arange(L, dtype=np.float64) / L, K)


def _filter_at(params: dict, tau, N: int, D: int) -> np.ndarray:
    """exp(-a_c |tau|) * o(tau)[n*D + c] at positions tau (in units of L): [N, D, len(tau)]."""
    f = lambda k: np.asarray(params[k], dtype=np.float64)  # noqa: E731
    tau = np.asarray(tau, dtype=np.float64)
    e = posenc_at(tau, int(params["K"]))
    a1 = np.sin(e @ f("w1") + f("b1"))
    a2 = np.sin(a1 @ f("w2") + f("b2"))
    o = a2 @ f("w3") + f("b3")                               # [P, N*D]
    window = np.exp(-np.outer(np.abs(tau), f("decay")))      # [P, D]
    h = o.reshape(len(tau), N, D) * window[:, None, :]
    return np.ascontiguousarray(h.transpose(1, 2, 0))


def implicit_filter(params: dict, L: int, N: int, D: int) -> np.ndarray:
    """h[n, c, t] = exp(-a_c t / L) * o_t[n*D + c],
    o_t = W3^T sin(W2^T sin(W1^T e_t + b1) + b2) + b3, e_t = posenc(t).

    Returns [N, D, L] float64.
    """
    return _filter_at(params, np.arange(L, dtype=np.float64) / L, N, D)


def implicit_filter_noncausal(params: dict, L: int, N: int, D: int) -> np.ndarray:
    """The same generator at the signed lags tau in [-(L-1), L-1]:
    h[n, c, i] = exp(-a_c |tau| / L) * o(tau / L)[n*D + c] with tau = i - (L - 1).

    Returns [N, D, 2L - 1] float64 (lag-indexed).
    """
    return _filter_at(params, np.arange(-(L - 1), L, dtype=np.float64) / L, N, D)


# ---------------------------------------------------------------------------
# Operator
# ---------------------------------------------------------------------------

def short_conv(p, w) -> np.ndarray:
    """s[b, t, j] = w[j,0] p[b,t,j] + w[j,1] p[b,t-1,j] + w[j,2] p[b,t-2,j], p[t<0] = 0."""
    p = np.asarray(p, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    s = w[:, 0] * p
    s[:, 1:] += w[:, 1] * p[:, :-1]
    s[:, 2:] += w[:, 2] * p[:, :-2]
    return s


def _project_and_gate_inputs(u, w_in, short_w, D, N):
    u = np.asarray(u, dtype=np.float64)
    p = u @ np.asarray(w_in, dtype=np.float64)               # [B, L, (N+1)D]
    s = short_conv(p, short_w)
    v = np.ascontiguousarray(s[..., :D].transpose(0, 2, 1))  # [B, D, L]
    xs = [np.ascontiguousarray(s[..., (n + 1) * D:(n + 2) * D].transpose(0, 2, 1))
          for n in range(N)]
    return v, xs


def _conv_fn(conv: str, causal: bool, L: int):
    if conv == "auto":
        conv = "direct" if L <= 4096 else "fft"
    if causal:
        return causal_conv_direct if conv == "direct" else causal_conv_fft
    return noncausal_conv_direct if conv == "direct" else noncausal_conv_fft


def hyena_recurrence(z, xs, dskip, h, conv: str = "auto", causal: bool = True) -> np.ndarray:
    """z^{N+1} from z^1 = v: z^{n+1} = x^n * (h^n conv z^n) + D^n * z^n, channel-major.

    z [B, D, L]; xs: N arrays [B, D, L]; dskip [N, D]; h [N, D, L] (or
    [N, D, 2L - 1] two-sided).  Every channel is independent of the others (the
    filters and gates act depthwise), so any channel subset can be run alone.
    """
    convf = _conv_fn(conv, causal, np.shape(z)[-1])
    dskip = np.asarray(dskip, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    for n in range(len(xs)):
        c = convf(h[n][None], z)
        z = xs[n] * c + dskip[n][None, :, None] * z
    return z


def hyena_fwd(u, w_in, short_w, dskip, w_out, h, conv: str = "auto", causal: bool = True,
              workers: int = 1) -> np.ndarray:
    """y[B, L, D] of the order-N operator.

    u [B, L, D]; w_in [D, (N+1)D]; short_w [(N+1)D, 3]; dskip [N, D];
    w_out [D, D]; h [N, D, L] (implicit_filter) or, with causal=False,
    [N, D, 2L - 1] (implicit_filter_noncausal).  conv: "direct", "fft" or
    "auto" (direct up to L = 4096, FFT above).  workers > 1 runs the recurrence
    on channel shards in that many processes (same arithmetic per channel).
    """
    B, L, D = np.shape(u)
    N = np.shape(dskip)[0]
    z, xs = _project_and_gate_inputs(u, w_in, short_w, D, N)
    dskip = np.asarray(dskip, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    if workers > 1:
        from ._pool import channel_shards
        z = channel_shards(hyena_recurrence, D, workers,
                           lambda sl: (z[:, sl], [x[:, sl] for x in xs], dskip[:, sl], h[:, sl], conv, causal))
    else:
        z = hyena_recurrence(z, xs, dskip, h, conv, causal)
    return z.transpose(0, 2, 1) @ np.asarray(w_out, dtype=np.float64)


def hyena_fwd_sampled(u, w_in, short_w, dskip, w_out, h, t_samples, chunk: int = 64,
                      causal: bool = True) -> np.ndarray:
    """y[:, t_samples, :] for long sequences.

    Orders 1..N-1 are computed for every t with causal_conv_fft /
    noncausal_conv_fft (channel chunks of `chunk` to bound memory); the last
    order is evaluated only at the sampled times by the direct sum
    c(t) = sum_s h(t - s) z(s).  Returns [B, S, D].
    """
    B, L, D = np.shape(u)
    N = np.shape(dskip)[0]
    dskip = np.asarray(dskip, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    t_samples = np.asarray(t_samples, dtype=np.int64)
    z, xs = _project_and_gate_inputs(u, w_in, short_w, D, N)
    for n in range(N - 1):
        c = np.empty_like(z)
        for c0 in range(0, D, chunk):
            convf = causal_conv_fft if causal else noncausal_conv_fft
            c[:, c0:c0 + chunk] = convf(h[n][None, c0:c0 + chunk], z[:, c0:c0 + chunk])
        z = xs[n] * c + dskip[n][None, :, None] * z
    n = N - 1
    out = np.empty((B, len(t_samples), D))
    for i, t in enumerate(t_samples):
        if causal:
            # c[b, d] = sum_{s=0..t} h[n, d, s] * z[b, d, t - s]
            c = np.einsum("ds,bds->bd", h[n, :, :t + 1], z[:, :, t::-1])
        else:
            # c[b, d] = sum_{s=0..L-1} h(t - s) z[b, d, s], lag t - s at index t - s + L - 1
            c = np.einsum("ds,bds->bd", h[n, :, t:t + L][:, ::-1], z)
        out[:, i, :] = xs[n][:, :, t] * c + dskip[n][None, :] * z[:, :, t]
    return out @ np.asarray(w_out, dtype=np.float64)
