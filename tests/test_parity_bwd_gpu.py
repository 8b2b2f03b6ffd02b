"""Parity of the backward pass (hyena_bwd, hyena_filter_bwd, through the C ABI)
with the fp64 backward oracle (oracle/hyena_bwd_oracle.py, pinned against
finite differences of the forward oracle).

Bar, per gradient: max |g - g_ref| / max |g_ref| <= 1e-4 (fp32 storage) or
<= 2e-2 (bf16 storage, fp32 compute)."""
import numpy as np
import pytest

from synth import bf16_round, make_1d, make_config
from tests.gpu_util import TOL, rel_err, say, to_dev

pytestmark = pytest.mark.gpu

KEYS = ["du", "dw_in", "dshort_w", "ddskip", "dw_out", "dh"]


def _dy(inp, seed):
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal((inp.B, inp.L, inp.D)).astype(np.float32)
    return bf16_round(dy) if inp.dtype == "bf16" else dy


def _gpu_bwd(inp, dy):
    import torch
    import subquadratic_sequence_amd as hs
    dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    layer = hs.HyenaLayer(inp.L, inp.D, inp.N, direction=hs.CAUSAL if inp.causal else hs.NONCAUSAL)
    hs.hyena_filter_gen(layer, to_dev(inp.w1), to_dev(inp.b1), to_dev(inp.w2), to_dev(inp.b2), to_dev(inp.w3),
                        to_dev(inp.b3), to_dev(inp.decay), inp.K)
    g = hs.hyena_bwd(layer, to_dev(inp.u, dt), to_dev(inp.w_in, dt), to_dev(inp.short_w), to_dev(inp.dskip),
                     to_dev(inp.w_out, dt), to_dev(dy, dt))
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy().astype(np.float64) for k, v in g.items()}, layer


def _oracle_bwd(inp, dy):
    import oracle
    from tests.gpu_util import oracle_1d  # noqa: F401  (same filter convention as the forward tests)
    if inp.causal:
        h = oracle.implicit_filter(inp.filter_params, inp.L, inp.N, inp.D)
    else:
        h = oracle.implicit_filter_noncausal(inp.filter_params, inp.L, inp.N, inp.D)
    conv = "direct" if inp.L * inp.B * inp.D <= (1 << 18) else "fft"
    return oracle.hyena_bwd(inp.u, inp.w_in, inp.short_w, inp.dskip, inp.w_out, h, dy, conv=conv,
                            causal=inp.causal), h


def _wrapped(dh2):
    """Lag-indexed [..., 2L-1] -> the wrapped [..., 2L] layout of the library's dh."""
    L = (dh2.shape[-1] + 1) // 2
    out = np.zeros(dh2.shape[:-1] + (2 * L,))
    out[..., :L] = dh2[..., L - 1:]
    out[..., L + 1:] = dh2[..., :L - 1]
    return out


def _check(inp, seed=5, tol=None):
    tol = tol or TOL[inp.dtype]
    say(f"bwd case B={inp.B} L={inp.L} D={inp.D} N={inp.N} {inp.dtype} causal={inp.causal} "
        f"seed={inp.meta['seed']}")
    dy = _dy(inp, seed)
    g, _ = _gpu_bwd(inp, dy)
    ref, _ = _oracle_bwd(inp, dy)
    if not inp.causal:
        ref = dict(ref, dh=_wrapped(ref["dh"]))
    for k in KEYS:
        assert g[k].shape == ref[k].shape, (k, g[k].shape, ref[k].shape)
        assert np.all(np.isfinite(g[k])), k
        err = rel_err(g[k], ref[k])
        say(f"  {k:9s} rel err {err:.3e}")
        assert err <= tol, (k, err)
    return g


def test_bwd_order2_f32_L1k_D64():
    _check(make_config("order2_f32_L1k_D64"))


def test_bwd_order2_bf16_B8_L2k_D768():
    _check(make_config("order2_bf16_B8_L2k_D768"))


@pytest.mark.parametrize("B,L,D,N,dt,causal", [
    (2, 32, 64, 1, "f32", True),        # smallest length, one order
    (1, 64, 128, 3, "f32", True),
    (3, 256, 64, 2, "bf16", True),      # odd batch
    (1, 512, 192, 4, "f32", True),      # four orders, D not a power of two
    (2, 4096, 64, 2, "f32", True),      # 8192-point transforms
    (2, 128, 64, 2, "f32", False),      # two-sided filters
    (1, 1024, 64, 2, "bf16", False),
])
def test_bwd_sweep(B, L, D, N, dt, causal):
    _check(make_1d(700 + B + L + D + N, B, L, D, N=N, K=8, dtype=dt, causal=causal))


# Four-step regime (L > 4096, causal filters): the transposed convolution and the
# filter gradient run on the forward's four-step passes (reversal, one order,
# unit gates) with per-sample spectra of z^n for dh.
@pytest.mark.parametrize("B,L,D,N,dt,causal", [
    (2, 8192, 64, 2, "f32", True),       # 256-point rows, two samples' spectra for dh
    (1, 8192, 64, 3, "f32", True),       # three orders
    (1, 16384, 128, 1, "bf16", True),
    (3, 32768, 64, 2, "bf16", True),     # odd batch, 1024-point rows
    (1, 65536, 64, 2, "bf16", True),     # the 64k length, 2048-point rows
    (2, 8192, 64, 2, "f32", False),      # two-sided filters: negative lags from a second convolution
    (1, 16384, 64, 2, "bf16", False),
])
def test_bwd_four_step(B, L, D, N, dt, causal):
    _check(make_1d(730 + B + L // 1024 + D + N + 5 * causal, B, L, D, N=N, K=8, dtype=dt, causal=causal))


def test_bwd_four_step_is_bit_reproducible():
    import torch
    inp = make_1d(741, 2, 8192, 64, N=2, K=8, dtype="bf16")
    dy = _dy(inp, 11)
    a, _ = _gpu_bwd(inp, dy)
    b, _ = _gpu_bwd(inp, dy)
    torch.cuda.synchronize()
    for k in KEYS:
        assert np.array_equal(a[k], b[k]), k


def test_bwd_is_bit_reproducible():
    import torch
    inp = make_1d(711, 2, 512, 128, N=2, K=8)
    dy = _dy(inp, 9)
    a, _ = _gpu_bwd(inp, dy)
    b, _ = _gpu_bwd(inp, dy)
    torch.cuda.synchronize()
    for k in KEYS:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("L,D,N,K,W,causal", [(1024, 64, 2, 8, 64, True), (2048, 128, 2, 16, 64, True),
                                               (256, 64, 3, 4, 32, False), (64, 64, 1, 32, 128, True),
                                               # long filters: the output-layer pass in position segments,
                                               # banded sums of the weight-gradient splits, segmented bias sums
                                               (16384, 64, 1, 8, 64, True), (8192, 64, 2, 16, 32, False)])
def test_filter_bwd_matches_oracle(L, D, N, K, W, causal):
    import torch
    import oracle
    import subquadratic_sequence_amd as hs
    inp = make_1d(720 + L + K + W, 1, L, D, N=N, K=K, W=W, causal=causal)
    say(f"filter bwd L={L} D={D} N={N} K={K} W={W} causal={causal}")
    rng = np.random.default_rng(3)
    hl = L if causal else 2 * L
    dh = rng.standard_normal((N, D, hl)).astype(np.float32)
    if not causal:
        dh[:, :, L] = 0.0          # wrapped entry L is not a tap
    layer = hs.HyenaLayer(L, D, N, direction=hs.CAUSAL if causal else hs.NONCAUSAL)
    fp = [to_dev(a) for a in (inp.w1, inp.b1, inp.w2, inp.b2, inp.w3, inp.b3, inp.decay)]
    g = hs.hyena_filter_bwd(layer, *fp, K, to_dev(dh))
    torch.cuda.synchronize()
    if causal:
        ref = oracle.implicit_filter_bwd(inp.filter_params, L, N, D, dh.astype(np.float64))
    else:
        lagged = np.concatenate([dh[..., L + 1:], dh[..., :L]], axis=-1)   # lags -(L-1) .. L-1
        ref = oracle.implicit_filter_noncausal_bwd(inp.filter_params, L, N, D, lagged.astype(np.float64))
    for k in ["w1", "b1", "w2", "b2", "w3", "b3", "decay"]:
        got = g[k].cpu().numpy().astype(np.float64)
        err = rel_err(got, ref[k])
        say(f"  d{k:6s} rel err {err:.3e}")
        assert err <= 1e-4, (k, err)


def test_bwd_chain_to_filter_parameters():
    # hyena_bwd's dh fed to hyena_filter_bwd equals the oracle's chain
    import torch
    import oracle
    import subquadratic_sequence_amd as hs
    inp = make_config("order2_f32_L1k_D64")
    dy = _dy(inp, 13)
    g, layer = _gpu_bwd(inp, dy)
    fp = [to_dev(a) for a in (inp.w1, inp.b1, inp.w2, inp.b2, inp.w3, inp.b3, inp.decay)]
    gp = hs.hyena_filter_bwd(layer, *fp, inp.K, to_dev(g["dh"]))
    torch.cuda.synchronize()
    ref, _ = _oracle_bwd(inp, dy)
    refp = oracle.implicit_filter_bwd(inp.filter_params, inp.L, inp.N, inp.D, ref["dh"])
    for k in ["w1", "b1", "w2", "b2", "w3", "b3", "decay"]:
        err = rel_err(gp[k].cpu().numpy().astype(np.float64), refp[k])
        say(f"  chain d{k:6s} rel err {err:.3e}")
        assert err <= 1e-4, (k, err)
