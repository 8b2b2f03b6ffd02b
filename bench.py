#!/usr/bin/env python3
"""Benchmark of the Hyena forward hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

The default workload is the 1D operator at B=1, L=64k, D=768, bf16; the 3D
workload (--workload nd3d_f32_B2_C128_64cube) times hyena_nd_fwd the same way.

One step = one hyena_fwd call (in-projection, short convolutions, all orders of
long FFT convolution with gating and skip, out-projection) over one batch of
synthetic input already resident in HBM. The implicit filters are generated and
their spectra cached once before timing (one cache per layer, reused by every
call). Prints one JSON line on stdout; progress goes to stderr.

Roofline: the FFT long-convolution stage is the dominant kernel sequence. Its
duration comes from HIP events that the library records on the launch stream at
the stage boundaries of every timed step (hyena_fwd_profiled), averaged; the algorithmic bytes per
order are B*L*D*3*s + 8*D*(L+1) (read z^n and x^n, write z^{n+1}, read the
filter spectrum), s the storage size of an activation. Next to it: the
projections' MFMA rate (2*M*N*K over their event time), the conv stage's VALU
instruction and FLOP rates (per-step counts from the rocprofv3 counter summary
under profiles/, over the live stage time), and the bandwidth of a plain device
copy measured in the same run.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "order2_bf16_L64k_D768"
# Kernel sources of the long-convolution stage; a traffic figure measured on other
# sources is stale and is not reported.
CONV_SOURCES = ["fft1d.hip", "common.h", "kernels.h"]
ND_CONV_SOURCES = ["nd.hip", "common.h", "kernels_nd.h"]
METRIC = "Hyena fwd tokens/sec at L=64k,D=768 (1 GPU); FFT-conv HBM GB/s % of peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2516.6  # 256 CUs x 2.4 GHz x 4096 flop/clk (dense)
MFMA_F32_PEAK_TFLOPS = 157.3
# VALU issue: each of the 4 SIMDs of a CU issues one wave64 instruction every 4
# cycles, so 256 CUs x 2.4 GHz wave instructions per second
VALU_PEAK_GINSTR = 256 * 2.4
VALU_F32_PEAK_TFLOPS = 157.3  # packed fp32 FMA; unpacked code tops out at half


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def four_step_spectrum_bytes(s) -> float:
    """Bytes per channel and bin of the filter spectra the four-step row passes
    read as stored: the half spectrum (L + 1 bins) as complex fp32, or as bf16
    pairs for bf16 workloads unless HYENA_SPECTRUM_FP32=1."""
    if s == 2 and os.environ.get("HYENA_SPECTRUM_FP32", "0") in ("", "0"):
        return 4.0
    return 8.0


def conv_alg_bytes(B, L, D, N, s, lds_regime: bool, spectrum_bytes: float = 8.0) -> float:
    """Algorithmic bytes of the long-convolution stage per call.

    Four-step regime, per order: read z^n and x^n, write z^{n+1} (3 B L D s) and
    read the filter's half spectrum, D (L + 1) bins of `spectrum_bytes` each
    (8: complex fp32, the count the roofline is quoted on; 4: the bf16 copy the
    row passes of bf16 workloads actually read). LDS regime (all orders fused
    on chip): read v and x^1..x^N, write z^{N+1}, read N spectra."""
    if lds_regime:
        return (N + 1) * B * L * D * s + B * L * D * s + N * 8.0 * D * (L + 1)
    return N * (3.0 * B * L * D * s + spectrum_bytes * D * (L + 1))


def conv_source_hash(sources=None) -> str:
    import hashlib
    hsh = hashlib.sha256()
    for name in sources or CONV_SOURCES:
        with open(os.path.join(ROOT, "subquadratic_sequence_amd", "csrc", name), "rb") as fh:
            hsh.update(fh.read())
    return hsh.hexdigest()


def _sources_of(workload: str):
    return ND_CONV_SOURCES if workload.startswith("nd") else CONV_SOURCES


def _profile_values(path: str, sources=None):
    """The '@key: value' lines of a profile summary, or None if the file is missing
    or was measured on other kernel sources."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("@") and ":" in line:
                k, v = line[1:].split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("conv_source_sha256") != conv_source_hash(sources):
        return None
    return kv


def measured_traffic(workload: str, path: str | None = None):
    """HBM bytes per step of the long-convolution stage, from the rocprofv3
    FETCH_SIZE / WRITE_SIZE summary under profiles/ (each counter scaled by what it
    reads for a plain copy of known size). None if there is no summary for this
    workload or the kernel sources changed since it was taken."""
    kv = _profile_values(path or os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt"), _sources_of(workload))
    return None if kv is None else float(kv["conv_stage_bytes_per_step"])


def measured_valu(workload: str, path: str | None = None):
    """(VALU wave instructions, fp32 VALU FLOPs) per step of the long-convolution
    stage, from the rocprofv3 SQ counter summary under profiles/; None as for
    measured_traffic."""
    kv = _profile_values(path or os.path.join(ROOT, "profiles", f"valu_mfma_{workload}.txt"), _sources_of(workload))
    if kv is None:
        return None
    return float(kv["conv_valu_instr_per_step"]), float(kv["conv_valu_flops_per_step"])


def copy_probe(torch, mib: int = 1024, reps: int = 5) -> float:
    """GB/s (bytes read + written) of a plain device copy of `mib` MiB."""
    src = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2.0 * src.numel() * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbs


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_workers(requested: int = 0) -> int:
    """Worker processes of the oracle baseline: the cores this process may run
    on (at most 16), or `requested`."""
    from oracle._pool import default_workers
    return requested or default_workers()


def cpu_baseline(inp, budget_tokens: int, workers: int):
    """fp64 oracle on the first `budget_tokens` positions of the same workload,
    channel shards in `workers` processes (one thread each; the parent's
    projections use as many BLAS threads).

    By causality y[:, :T] depends only on u[:, :T] and on the first T filter taps,
    so the oracle runs on that prefix with the filters' first T taps, FFT
    convolution path. A non-causal layer has no such prefix property: the oracle
    then runs the operator on a length-T sequence (the first T inputs, filters
    generated for length T), the same work per token. Filter generation runs
    before the timed region (the GPU step reads cached spectra)."""
    import oracle
    from threadpoolctl import threadpool_limits
    T = min(budget_tokens, inp.L)
    if inp.causal:
        h = oracle.implicit_filter(inp.filter_params, T, inp.N, inp.D) if T == inp.L else \
            oracle.implicit_filter(inp.filter_params, inp.L, inp.N, inp.D)[:, :, :T]
    else:
        h = oracle.implicit_filter_noncausal(inp.filter_params, T, inp.N, inp.D)
    with threadpool_limits(limits=workers):
        t0 = time.perf_counter()
        oracle.hyena_fwd(inp.u[:, :T], inp.w_in, inp.short_w, inp.dskip, inp.w_out, h, conv="fft",
                         causal=inp.causal, workers=workers)
        dt = time.perf_counter() - t0
    what = "first" if inp.causal else "a non-causal operator of length T on the first"
    return {"value": inp.B * T / dt, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{what} {T} of {inp.L} positions x B={inp.B} (all {inp.D} channels), fp64 numpy, "
                      f"FFT path, channel shards in {workers} processes of 1 thread, filters generated "
                      f"beforehand, {dt:.1f} s"}


def nd_conv_alg_bytes(B, X, Y, Z, C, N, circular: bool = False) -> float:
    """Per call: each order reads z^n and x^n and writes z^{n+1} (fp32 [B][C][X][Y][Z])
    and reads the channel's half spectrum (complex fp32, MX MY (MZ/2 + 1) bins with
    (MX, MY, MZ) = (2X, 2Y, 2Z) zero padded, (X, Y, Z) circular).

    2D grids (X = 1, MX = 1) run all orders on chip: v and the N gates x^n are
    read once, z^{N+1} written once, plus the N spectra."""
    V = X * Y * Z
    p = 1 if circular else 2
    spec = 8.0 * C * (1 if X == 1 else p * X) * (p * Y) * (p * Z // 2 + 1)
    if X == 1:
        return (N + 2) * B * C * V * 4.0 + N * spec
    return N * (3.0 * B * C * V * 4 + spec)


def _restrict_channels(inp, params, c, per_channel_keys):
    """Projections and kernel outputs restricted to channels 0..c-1 (indexing only)."""
    N, C = inp.N, inp.C
    w_in = np.concatenate([inp.w_in[:c, j * C:j * C + c] for j in range(N + 1)], axis=1)
    params = dict(params)
    params["w3"] = np.concatenate([params["w3"][:, n * C:n * C + c] for n in range(N)], axis=1)
    params["b3"] = np.concatenate([params["b3"][n * C:n * C + c] for n in range(N)])
    for k in per_channel_keys:
        params[k] = params[k][:c]
    return w_in, params


def cpu_baseline_nd(inp, channels: int, workers: int):
    """fp64 oracle forward on one sample and the first `channels` channels (the
    projections restricted to them), full grid, channel shards in `workers`
    processes, the kernel generated before the timed region (as the GPU step
    uses a cached spectrum); voxel rate scaled by channels / C."""
    import oracle
    from threadpoolctl import threadpool_limits
    c = min(channels, inp.C)
    w_in, params = _restrict_channels(inp, inp.filter_params, c, ["decay"])
    K = oracle.nd_filter(params, inp.X, inp.Y, inp.Z, inp.N, c, circular=inp.circular)
    with threadpool_limits(limits=workers):
        t0 = time.perf_counter()
        oracle.hyena_nd_fwd(inp.u[:1, ..., :c], w_in, inp.dskip[:, :c], inp.gate_a[:, :c], inp.gate_b[:, :c],
                            inp.w_out[:c, :c], K, conv="fft", circular=inp.circular, workers=workers)
        dt = time.perf_counter() - t0
    V = inp.X * inp.Y * inp.Z
    unit = "pixels/s" if inp.X == 1 else "voxels/s"
    return {"value": V / dt * c / inp.C, "unit": unit, "cores": workers, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"sample 0 of {inp.B}, channels 0..{c - 1} of {inp.C} (projections restricted to them), "
                      f"full {inp.X}x{inp.Y}x{inp.Z} grid, fp64 numpy, FFT path (kernel generated beforehand), "
                      f"channel shards in {workers} processes of 1 thread, {dt:.1f} s; rate scaled by {c}/{inp.C}"}


def main_nd(args, torch, hs, make_config):
    log(f"generating inputs for {args.workload}")
    inp = make_config(args.workload)
    B, X, Y, Z, C, N = inp.B, inp.X, inp.Y, inp.Z, inp.C, inp.N
    V = X * Y * Z
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda")  # noqa: E731
    bd = hs.ND_CIRCULAR if inp.circular else hs.ND_ZERO_PAD
    layer = hs.HyenaNDLayer(X, Y, Z, C, N, boundary=bd)
    fargs = [f(a) for a in (inp.w1, inp.b1, inp.w2, inp.b2, inp.w3, inp.b3, inp.decay)]
    hs.hyena_nd_filter_gen(layer, *fargs)
    u, w_in, dskip, ga, gb, w_out = (f(a) for a in (inp.u, inp.w_in, inp.dskip, inp.gate_a, inp.gate_b, inp.w_out))
    y = torch.empty_like(u)
    ws = torch.empty(hs.hyena_nd_workspace_bytes_ex(B, X, Y, Z, C, N, bd), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        hs.hyena_nd_fwd(layer, u, w_in, dskip, ga, gb, w_out, y=y, ws=ws)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for evs in events:
        for ev in evs:
            ev.record()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for k in range(args.steps):
        hs.hyena_nd_fwd_profiled(layer, u, w_in, dskip, ga, gb, w_out, y, ws, events[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stages = np.mean([[evs[i].elapsed_time(evs[i + 1]) for i in range(3)] for evs in events], axis=0)
    step_ms = np.array([evs[0].elapsed_time(evs[3]) for evs in events])
    log(f"stages ms: in-proj {stages[0]:.4f} conv {stages[1]:.4f} out-proj {stages[2]:.4f}")
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record()
    hs.hyena_nd_filter_gen(layer, *fargs)
    f1.record()
    torch.cuda.synchronize()
    alg = nd_conv_alg_bytes(B, X, Y, Z, C, N, inp.circular)
    achieved = alg / (stages[1] * 1e-3) / 1e9
    proj = {}
    for name, n_out, ms in (("in_proj", (N + 1) * C, stages[0]), ("out_proj", C, stages[2])):
        tf = 2.0 * B * V * n_out * C / (ms * 1e-3) / 1e12
        proj[name] = {"tflops": tf, "peak": MFMA_F32_PEAK_TFLOPS, "frac": tf / MFMA_F32_PEAK_TFLOPS}
    valu = measured_valu(args.workload)
    conv_valu = None
    if valu is not None:
        gi = valu[0] / (stages[1] * 1e-3) / 1e9
        tf = valu[1] / (stages[1] * 1e-3) / 1e12
        conv_valu = {"bound": "alu", "achieved": gi, "peak": VALU_PEAK_GINSTR, "unit": "G wave-instr/s",
                     "frac": gi / VALU_PEAK_GINSTR, "fp32_tflops": tf, "fp32_peak_tflops": VALU_F32_PEAK_TFLOPS}
    out = {
        "metric": (f"HyenaND fwd {'pixels' if X == 1 else 'voxels'}/sec ({'2D' if X == 1 else '3D'}, B={B}, C={C}, "
                   f"{f'{Y}x{Z}' if X == 1 else f'{X}x{Y}x{Z}'}{', circular' if inp.circular else ''}, 1 GPU); "
                   f"{'2D' if X == 1 else '3D'} FFT-conv HBM GB/s % of peak"),
        "value": B * V * args.steps / elapsed,
        "unit": "pixels/s" if X == 1 else "voxels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * elapsed / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "X": X, "Y": Y, "Z": Z, "C": C, "N": N,
                   "boundary": "circular" if inp.circular else "zero-padded"},
        "stage_ms": {"in_proj": stages[0], "fft_conv": stages[1], "out_proj": stages[2]},
        "step_ms_events": {"p10": float(np.percentile(step_ms, 10)), "p50": float(np.median(step_ms)),
                           "p90": float(np.percentile(step_ms, 90))},
        "filter_gen_ms": f0.elapsed_time(f1),
        "roofline": {"bound": "hbm", "kernel": f"{'2D' if X == 1 else '3D'} fft_conv stage (all orders)",
                     "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "alg_bytes": alg,
                     "traffic": measured_traffic(args.workload)},
        "conv_valu": conv_valu,
        "projections_mfma": proj,
        "copy_probe_gbs": copy_probe(torch),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        # about 10-20 s of oracle work: all channels of a 2D grid or of a periodic 3D grid's
        # sample, two channels per worker of a zero-padded 3D grid's sample
        P = cpu_workers(args.cpu_workers)
        dflt = inp.C if (X == 1 or inp.circular) else 2 * P
        out["cpu_baseline"] = cpu_baseline_nd(inp, args.cpu_channels or dflt, P)
    print(json.dumps(out), flush=True)


def nd_film_conv_alg_bytes(B, X, Y, Z, C, N, circular: bool = False) -> float:
    """nd_conv_alg_bytes with per-sample kernels: every sample reads its own spectra."""
    V = X * Y * Z
    p = 1 if circular else 2
    spec = 8.0 * C * (1 if X == 1 else p * X) * (p * Y) * (p * Z // 2 + 1)
    if X == 1:
        return (N + 2) * B * C * V * 4.0 + N * B * spec
    return N * (3.0 * B * C * V * 4 + B * spec)


def film_mlp_flops(X, Y, Z, C, N, W, circular: bool = False) -> float:
    """Flops of one sample's coordinate MLP over the offset grid (3 -> W -> W -> N C)."""
    p = 1 if circular else 2
    P = (1 if X == 1 else p * X) * (p * Y) * (p * Z)
    return 2.0 * P * (3 * W + W * W + W * N * C)


def cpu_baseline_nd_film(inp, channels: int, workers: int):
    """fp64 oracle of the register-conditioned layer on one sample and the first
    `channels` channels (kernel outputs and projections restricted to them; the
    control vector and FiLM vectors from all channels), full grid. The kernel
    synthesis is inside the timed region, as on the GPU (its matrix products on
    `workers` BLAS threads); the recurrence runs channel shards in `workers`
    processes. Voxel rate scaled by channels / C."""
    import oracle
    from threadpoolctl import threadpool_limits
    c = min(channels, inp.C)
    w_in, params = _restrict_channels(inp, inp.film_filter_params, c, ["window"])
    with threadpool_limits(limits=workers):
        t0 = time.perf_counter()
        mod = oracle.film_modulation(oracle.film_control(inp.reg[:1], inp.q), inp.film_w, inp.film_b)
        K = oracle.nd_filter_film(params, mod[0], inp.X, inp.Y, inp.Z, inp.N, c, circular=inp.circular)
        oracle.hyena_nd_film_fwd(inp.u[:1, ..., :c], w_in, inp.dskip[:, :c], inp.w_out[:c, :c], K[None],
                                 circular=inp.circular, workers=workers)
        dt = time.perf_counter() - t0
    V = inp.X * inp.Y * inp.Z
    return {"value": V / dt * c / inp.C, "unit": "voxels/s", "cores": workers, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"sample 0 of {inp.B}, channels 0..{c - 1} of {inp.C} (kernel outputs and projections "
                      f"restricted to them), full {inp.X}x{inp.Y}x{inp.Z} grid, fp64 numpy, kernel synthesis "
                      f"and FFT path, channel shards in {workers} processes, {dt:.1f} s; rate scaled by {c}/{inp.C}"}


def main_nd_film(args, torch, hs, make_config):
    log(f"generating inputs for {args.workload}")
    inp = make_config(args.workload)
    B, X, Y, Z, C, N, W = inp.B, inp.X, inp.Y, inp.Z, inp.C, inp.N, inp.W
    V = X * Y * Z
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda")  # noqa: E731
    bd = hs.ND_CIRCULAR if inp.circular else hs.ND_ZERO_PAD
    m = hs.HyenaNDFilm(X, Y, Z, C, N, bd, *(f(a) for a in (inp.w1, inp.b1, inp.w2, inp.b2, inp.w3, inp.b3,
                                                             inp.window, inp.q, inp.film_w, inp.film_b,
                                                             inp.omega0)))
    u, reg, w_in, dskip, w_out = (f(a) for a in (inp.u, inp.reg, inp.w_in, inp.dskip, inp.w_out))
    y = torch.empty_like(u)
    ws = torch.empty(hs.hyena_nd_film_workspace_bytes(B, X, Y, Z, C, N, W, bd), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        hs.hyena_nd_film_fwd(m, u, reg, w_in, dskip, w_out, y=y, ws=ws)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for evs in events:
        for ev in evs:
            ev.record()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for k in range(args.steps):
        hs.hyena_nd_film_fwd_profiled(m, u, reg, w_in, dskip, w_out, y, ws, events[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    st = np.mean([[evs[i].elapsed_time(evs[i + 1]) for i in range(4)] for evs in events], axis=0)
    step_ms = np.array([evs[0].elapsed_time(evs[4]) for evs in events])
    log(f"stages ms: synthesis {st[0]:.4f} in-proj {st[1]:.4f} conv {st[2]:.4f} out-proj {st[3]:.4f}")
    alg = nd_film_conv_alg_bytes(B, X, Y, Z, C, N, inp.circular)
    achieved = alg / (st[2] * 1e-3) / 1e9
    mlp = B * film_mlp_flops(X, Y, Z, C, N, W, inp.circular)
    proj = {}
    for name, n_out, ms in (("in_proj", (N + 1) * C, st[1]), ("out_proj", C, st[3])):
        tf = 2.0 * B * V * n_out * C / (ms * 1e-3) / 1e12
        proj[name] = {"tflops": tf, "peak": MFMA_F32_PEAK_TFLOPS, "frac": tf / MFMA_F32_PEAK_TFLOPS}
    out = {
        "metric": (f"HyenaND fwd voxels/sec (3D, B={B}, C={C}, {X}x{Y}x{Z}"
                   f"{', circular' if inp.circular else ''}, register-conditioned FiLM kernels synthesised "
                   f"per sample in every step, 1 GPU); 3D FFT-conv HBM GB/s % of peak"),
        "value": B * V * args.steps / elapsed,
        "unit": "voxels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * elapsed / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "X": X, "Y": Y, "Z": Z, "C": C, "N": N, "W": W,
                   "registers": int(inp.reg.shape[1]), "boundary": "circular" if inp.circular else "zero-padded"},
        "stage_ms": {"kernel_synthesis": st[0], "in_proj": st[1], "fft_conv": st[2], "out_proj": st[3]},
        "step_ms_events": {"p10": float(np.percentile(step_ms, 10)), "p50": float(np.median(step_ms)),
                           "p90": float(np.percentile(step_ms, 90))},
        "roofline": {"bound": "hbm", "kernel": "3D fft_conv stage (all orders, every sample with its own spectra)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "alg_bytes": alg, "traffic": measured_traffic(args.workload)},
        "kernel_synthesis": {"ms": st[0], "mlp_gflop": mlp / 1e9,
                             "mlp_tflops_if_whole_stage": mlp / (st[0] * 1e-3) / 1e12,
                             "mfma_f32_peak_tflops": MFMA_F32_PEAK_TFLOPS},
        "projections_mfma": proj,
        "copy_probe_gbs": copy_probe(torch),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        P = cpu_workers(args.cpu_workers)
        out["cpu_baseline"] = cpu_baseline_nd_film(inp, args.cpu_channels or 2 * P, P)
    print(json.dumps(out), flush=True)


def main_bwd(args, torch, hs, make_config):
    """Times hyena_bwd (and hyena_filter_bwd) on a 1D workload."""
    log(f"generating inputs for {args.workload} (backward)")
    inp = make_config(args.workload)
    B, L, D, N = inp.B, inp.L, inp.D, inp.N
    tdt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    f = lambda a, d=torch.float32: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda", d)  # noqa: E731
    layer = hs.HyenaLayer(L, D, N, direction=hs.CAUSAL if inp.causal else hs.NONCAUSAL)
    fp = [f(a) for a in (inp.w1, inp.b1, inp.w2, inp.b2, inp.w3, inp.b3, inp.decay)]
    hs.hyena_filter_gen(layer, *fp, inp.K)
    u, w_in, w_out = f(inp.u, tdt), f(inp.w_in, tdt), f(inp.w_out, tdt)
    short_w, dskip = f(inp.short_w), f(inp.dskip)
    dy = torch.randn(B, L, D, device="cuda").to(tdt)
    dt = hs.HYENA_BF16 if inp.dtype == "bf16" else hs.HYENA_F32
    ws = torch.empty(hs.hyena_bwd_workspace_bytes(B, L, D, N, dt, layer.direction), dtype=torch.uint8, device="cuda")
    fws = torch.empty(hs.hyena_filter_bwd_workspace_bytes(L, D, N, inp.K, inp.W, layer.direction),
                      dtype=torch.uint8, device="cuda")
    y = torch.empty_like(u)
    fws_fwd = torch.empty(hs.hyena_workspace_bytes(B, L, D, N, dt), dtype=torch.uint8, device="cuda")
    if args.bwd_only:
        # hyena_bwd alone, back to back (for a kernel trace of its launches)
        for _ in range(args.warmup):
            hs.hyena_bwd(layer, u, w_in, short_w, dskip, w_out, dy, ws=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            hs.hyena_bwd(layer, u, w_in, short_w, dskip, w_out, dy, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        bwd_ms = e0.elapsed_time(e1) / args.steps
        print(json.dumps({"metric": "Hyena bwd tokens/sec (hyena_bwd only)", "value": B * L / (bwd_ms * 1e-3),
                          "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "ms_per_step": bwd_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                          "dtype": inp.dtype, "data": "synthetic",
                          "config": {"workload": args.workload, "B": B, "L": L, "D": D, "N": N}}), flush=True)
        return
    for _ in range(args.warmup):
        g = hs.hyena_bwd(layer, u, w_in, short_w, dskip, w_out, dy, ws=ws)
        hs.hyena_filter_bwd(layer, *fp, inp.K, g["dh"], ws=fws)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record()
    for _ in range(args.steps):
        hs.hyena_fwd(layer, u, w_in, short_w, dskip, w_out, y=y, ws=fws_fwd)
    ev[1].record()
    for _ in range(args.steps):
        g = hs.hyena_bwd(layer, u, w_in, short_w, dskip, w_out, dy, ws=ws)
    ev[2].record()
    for _ in range(args.steps):
        hs.hyena_filter_bwd(layer, *fp, inp.K, g["dh"], ws=fws)
    ev[3].record()
    torch.cuda.synchronize()
    fwd_ms, bwd_ms, fbwd_ms = (ev[i].elapsed_time(ev[i + 1]) / args.steps for i in range(3))
    out = {
        "metric": "Hyena bwd tokens/sec (hyena_bwd: gradients of u, W_in, short conv, skips, W_out and the filters)",
        "value": B * L / (bwd_ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": bwd_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": inp.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "L": L, "D": D, "N": N,
                   "direction": "causal" if inp.causal else "non-causal"},
        "fwd_ms": fwd_ms, "bwd_ms": bwd_ms, "filter_bwd_ms": fbwd_ms, "bwd_over_fwd": bwd_ms / fwd_ms,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time hyena_bwd and hyena_filter_bwd instead (1D workloads)")
    ap.add_argument("--bwd-only", action="store_true",
                    help="with --backward: run and time hyena_bwd alone, back to back")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="positions of the 1D oracle sample (default 0: the whole sequence)")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle worker processes (default: the cores this process may use, at most 16)")
    ap.add_argument("--cpu-channels", type=int, default=0,
                    help="channels of the 3D oracle sample (default: two per worker zero padded, all circular "
                         "and on 2D grids)")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (reads and writes MIB MiB), for calibrating "
                         "the FETCH_SIZE / WRITE_SIZE counters, and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this path is built and "
              f"measured on a single MI355X.", file=sys.stderr)
        sys.exit(2)

    import torch
    import subquadratic_sequence_amd as hs
    from synth import CONFIGS, TEST_SHAPES, make_config

    if args.calib_copy:
        n = args.calib_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)  # one elementwise kernel: reads and writes n * 4 bytes
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n * 4}))
        return

    if args.workload not in CONFIGS and args.workload not in TEST_SHAPES:
        print(f"unknown workload {args.workload}; one of {sorted(CONFIGS) + sorted(TEST_SHAPES)}", file=sys.stderr)
        sys.exit(2)
    cfg = CONFIGS.get(args.workload) or TEST_SHAPES[args.workload]
    if args.backward:
        if cfg["kind"] != "1d":
            print("--backward: the backward pass covers the 1D workloads", file=sys.stderr)
            sys.exit(2)
        return main_bwd(args, torch, hs, make_config)
    if cfg["kind"] == "nd":
        return main_nd(args, torch, hs, make_config)
    if cfg["kind"] == "nd_film":
        return main_nd_film(args, torch, hs, make_config)
    log(f"generating inputs for {args.workload}")
    inp = make_config(args.workload)
    B, L, D, N = inp.B, inp.L, inp.D, inp.N
    tdt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    s = 2 if inp.dtype == "bf16" else 4
    dev = "cuda"
    f = lambda a, d=torch.float32: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev, d)  # noqa: E731

    layer = hs.HyenaLayer(L, D, N, direction=hs.CAUSAL if inp.causal else hs.NONCAUSAL)
    hs.hyena_filter_gen(layer, f(inp.w1), f(inp.b1), f(inp.w2), f(inp.b2), f(inp.w3), f(inp.b3), f(inp.decay),
                        inp.K)
    u, w_in, w_out = f(inp.u, tdt), f(inp.w_in, tdt), f(inp.w_out, tdt)
    short_w, dskip = f(inp.short_w), f(inp.dskip)
    y = torch.empty_like(u)
    ws = torch.empty(hs.hyena_workspace_bytes(B, L, D, N, hs.HYENA_BF16 if s == 2 else hs.HYENA_F32),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        hs.hyena_fwd(layer, u, w_in, short_w, dskip, w_out, y=y, ws=ws)
    torch.cuda.synchronize()
    # Four HIP events per step mark the stage boundaries on the launch stream
    # (recorded by the library between its launches, no synchronisation).
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for evs in events:
        for ev in evs:
            ev.record()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for k in range(args.steps):
        hs.hyena_fwd_profiled(layer, u, w_in, short_w, dskip, w_out, y, ws, events[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    value = B * L * args.steps / elapsed
    stages = np.mean([[evs[i].elapsed_time(evs[i + 1]) for i in range(3)] for evs in events], axis=0)
    step_ms = np.array([evs[0].elapsed_time(evs[3]) for evs in events])
    lds = L <= 4096
    alg = conv_alg_bytes(B, L, D, N, s, lds)
    achieved = alg / (stages[1] * 1e-3) / 1e9
    alg_stored = conv_alg_bytes(B, L, D, N, s, lds, four_step_spectrum_bytes(s))
    achieved_stored = alg_stored / (stages[1] * 1e-3) / 1e9
    log(f"stages ms: in-proj {stages[0]:.4f} conv {stages[1]:.4f} out-proj {stages[2]:.4f}")

    # filter generation (once per layer; outside the step) and a plain copy for scale
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record()
    hs.hyena_filter_gen(layer, f(inp.w1), f(inp.b1), f(inp.w2), f(inp.b2), f(inp.w3), f(inp.b3), f(inp.decay),
                        inp.K)
    f1.record()
    torch.cuda.synchronize()
    filter_gen_ms = f0.elapsed_time(f1)
    copy_gbs = copy_probe(torch)

    mfma_peak = MFMA_BF16_PEAK_TFLOPS if s == 2 else MFMA_F32_PEAK_TFLOPS
    proj = {}
    for name, n_out, k_in, ms in (("in_proj", (N + 1) * D, D, stages[0]), ("out_proj", D, D, stages[2])):
        tf = 2.0 * B * L * n_out * k_in / (ms * 1e-3) / 1e12
        proj[name] = {"tflops": tf, "peak": mfma_peak, "frac": tf / mfma_peak}
    valu = measured_valu(args.workload)
    conv_valu = None
    if valu is not None:
        gi = valu[0] / (stages[1] * 1e-3) / 1e9
        tf = valu[1] / (stages[1] * 1e-3) / 1e12
        conv_valu = {"bound": "alu", "achieved": gi, "peak": VALU_PEAK_GINSTR, "unit": "G wave-instr/s",
                     "frac": gi / VALU_PEAK_GINSTR, "fp32_tflops": tf, "fp32_peak_tflops": VALU_F32_PEAK_TFLOPS}

    out = {
        "metric": METRIC if inp.causal else METRIC + " [non-causal filters]",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "L": L, "D": D, "N": N,
                   "direction": "causal" if inp.causal else "non-causal"},
        "stage_ms": {"in_proj": stages[0], "fft_conv": stages[1], "out_proj": stages[2]},
        "step_ms_events": {"p10": float(np.percentile(step_ms, 10)), "p50": float(np.median(step_ms)),
                           "p90": float(np.percentile(step_ms, 90))},
        "filter_gen_ms": filter_gen_ms,
        "roofline": {"bound": "hbm", "kernel": "fft_conv stage (all orders)", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(args.workload),
                     "alg_bytes": alg, "alg_bytes_basis": "per order 3 B L D s + 8 D (L + 1): spectrum as complex fp32",
                     "stored_precision": {"alg_bytes": alg_stored, "achieved": achieved_stored,
                                          "frac": achieved_stored / HBM_PEAK_GBS,
                                          "basis": "spectrum counted at the precision the row passes read"}},
        "conv_valu": conv_valu,
        "projections_mfma": proj,
        "copy_probe_gbs": copy_gbs,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_tokens or inp.L, cpu_workers(args.cpu_workers))
        # the same oracle on one thread, on a prefix with about the same work
        one = cpu_baseline(inp, min(inp.L, 4096), 1)
        out["cpu_baseline"]["one_thread"] = {"value": one["value"], "unit": one["unit"], "cores": 1,
                                             "sample": one["sample"]}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
