"""Input recipes for the Hyena operator workloads.

Every array is drawn from ``numpy.random.default_rng(seed)`` in a fixed order, in
float64, then stored as float32. For bf16 workloads the activations and the
projection weights are rounded to bfloat16 (round to nearest even) and kept as
float32 arrays whose values are exactly representable in bfloat16, so that the
oracle (which upcasts the stored values to float64) and the GPU path (which
consumes the bfloat16 bits) see identical numbers.

Draw order (1D): u, w_in, short_w, dskip, w_out, w1, b1, w2, b2, w3, b3.
Draw order (ND): u, w_in, dskip, gate_a, gate_b, w_out, w1, b1, w2, b2, w3, b3.
The window decays are deterministic (no draw).

The workloads stand in for the pages' data: a 2k language-model context
(Hyena Hierarchy abstract), the 64k synthetic recall length (TWIML #690, 8:34),
a 1M single-nucleotide DNA context over a four-letter alphabet (HyenaDNA
abstract; TWIML #690, 19:09) and 3D volumes (HyenaND explainer, Results). No
dataset item is reproduced; only shapes and value distributions are taken.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# |ln 1e-2| / 1.5 and |ln 1e-2| / 0.3: the window reaches 1e-2 at tau = 1.5 ... 0.3.
_DECAY_LO = math.log(100.0) / 1.5
_DECAY_HI = math.log(100.0) / 0.3


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float values to the nearest bfloat16 (ties to even); returns float32."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32).reshape(f.shape)


def decay_rates(n: int) -> np.ndarray:
    """Window decay rates a_c, linearly spaced over the channels (slowest first)."""
    if n == 1:
        return np.array([_DECAY_LO], dtype=np.float32)
    return np.linspace(_DECAY_LO, _DECAY_HI, n).astype(np.float32)


def _uniform(rng, shape, bound):
    return rng.uniform(-bound, bound, size=shape)


@dataclass
class Hyena1DInputs:
    B: int
    L: int
    D: int
    N: int
    K: int          # positional-encoding frequencies (features = 1 + 2K)
    W: int          # filter FFN width
    dtype: str      # "f32" or "bf16": storage type of u, w_in, w_out, y
    u: np.ndarray        # [B, L, D]
    w_in: np.ndarray     # [D, (N+1)D]  column blocks (v, x^1..x^N)
    short_w: np.ndarray  # [(N+1)D, 3]  taps for p_t, p_{t-1}, p_{t-2}
    dskip: np.ndarray    # [N, D]
    w_out: np.ndarray    # [D, D]
    w1: np.ndarray       # [1+2K, W]
    b1: np.ndarray       # [W]
    w2: np.ndarray       # [W, W]
    b2: np.ndarray       # [W]
    w3: np.ndarray       # [W, N*D]
    b3: np.ndarray       # [N*D]
    decay: np.ndarray    # [D]
    causal: bool = True  # False: two-sided (non-causal) long filters
    meta: dict = field(default_factory=dict)

    @property
    def filter_params(self):
        return dict(K=self.K, w1=self.w1, b1=self.b1, w2=self.w2, b2=self.b2,
                    w3=self.w3, b3=self.b3, decay=self.decay)


@dataclass
class HyenaNDInputs:
    B: int
    X: int
    Y: int
    Z: int
    C: int
    N: int
    W: int
    u: np.ndarray        # [B, X, Y, Z, C]
    w_in: np.ndarray     # [C, (N+1)C]
    dskip: np.ndarray    # [N, C]
    gate_a: np.ndarray   # [N, C]
    gate_b: np.ndarray   # [N, C]
    w_out: np.ndarray    # [C, C]
    w1: np.ndarray       # [3, W]
    b1: np.ndarray       # [W]
    w2: np.ndarray       # [W, W]
    b2: np.ndarray       # [W]
    w3: np.ndarray       # [W, N*C]
    b3: np.ndarray       # [N*C]
    decay: np.ndarray    # [C]
    circular: bool = False  # periodic grid (circular convolution) instead of zero padding
    meta: dict = field(default_factory=dict)

    @property
    def filter_params(self):
        return dict(w1=self.w1, b1=self.b1, w2=self.w2, b2=self.b2,
                    w3=self.w3, b3=self.b3, decay=self.decay)


def make_1d(seed: int, B: int, L: int, D: int, N: int = 2, K: int = 16, W: int = 64,
            dtype: str = "f32", u_scale: float = 1.0, tokens: int = 0, causal: bool = True) -> Hyena1DInputs:
    """Draw one 1D workload.

    u ~ N(0, 1) * u_scale, or (tokens > 0) u = E[tok] with tok uniform over
    `tokens` symbols and E ~ N(0, 1) of shape [tokens, D].
    w_in, w_out ~ N(0, 1/D); short_w ~ U(-0.5, 0.5); dskip ~ N(0, 1);
    FFN weights and biases ~ U(-1/sqrt(fan_in), 1/sqrt(fan_in)).
    `causal` = False selects two-sided filters; it changes no draw.
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(dtype)
    rng = np.random.default_rng(seed)
    store = bf16_round if dtype == "bf16" else (lambda a: np.asarray(a, dtype=np.float32))
    if tokens > 0:
        tok = rng.integers(0, tokens, size=(B, L))
        table = store(rng.standard_normal((tokens, D)))
        u = table[tok]
    else:
        u = store(rng.standard_normal((B, L, D)) * u_scale)
    sd = 1.0 / math.sqrt(D)
    w_in = store(rng.standard_normal((D, (N + 1) * D)) * sd)
    short_w = rng.uniform(-0.5, 0.5, size=((N + 1) * D, 3)).astype(np.float32)
    dskip = rng.standard_normal((N, D)).astype(np.float32)
    w_out = store(rng.standard_normal((D, D)) * sd)
    F = 1 + 2 * K
    w1 = _uniform(rng, (F, W), 1 / math.sqrt(F)).astype(np.float32)
    b1 = _uniform(rng, (W,), 1 / math.sqrt(F)).astype(np.float32)
    w2 = _uniform(rng, (W, W), 1 / math.sqrt(W)).astype(np.float32)
    b2 = _uniform(rng, (W,), 1 / math.sqrt(W)).astype(np.float32)
    w3 = _uniform(rng, (W, N * D), 1 / math.sqrt(W)).astype(np.float32)
    b3 = _uniform(rng, (N * D,), 1 / math.sqrt(W)).astype(np.float32)
    return Hyena1DInputs(B=B, L=L, D=D, N=N, K=K, W=W, dtype=dtype, u=u, w_in=w_in,
                         short_w=short_w, dskip=dskip, w_out=w_out, w1=w1, b1=b1,
                         w2=w2, b2=b2, w3=w3, b3=b3, decay=decay_rates(D), causal=causal,
                         meta=dict(seed=seed, u_scale=u_scale, tokens=tokens))


def make_nd(seed: int, B: int, X: int, Y: int, Z: int, C: int, N: int = 2, W: int = 64,
            u_mean_spread: float = 0.0, circular: bool = False) -> HyenaNDInputs:
    """Draw one 3D workload (fp32).

    u ~ N(0, 1), plus an optional per-(sample, channel) offset ~ N(0, u_mean_spread^2)
    so that the channel-mean gate sees means away from zero.
    w_in, w_out ~ N(0, 1/C); dskip, gate_a, gate_b ~ N(0, 1);
    MLP weights and biases ~ U(-1/sqrt(fan_in), 1/sqrt(fan_in)).
    `circular` selects the periodic boundary; it changes no draw.
    """
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((B, X, Y, Z, C))
    if u_mean_spread:
        u = u + rng.standard_normal((B, 1, 1, 1, C)) * u_mean_spread
    u = u.astype(np.float32)
    sd = 1.0 / math.sqrt(C)
    w_in = (rng.standard_normal((C, (N + 1) * C)) * sd).astype(np.float32)
    dskip = rng.standard_normal((N, C)).astype(np.float32)
    gate_a = rng.standard_normal((N, C)).astype(np.float32)
    gate_b = rng.standard_normal((N, C)).astype(np.float32)
    w_out = (rng.standard_normal((C, C)) * sd).astype(np.float32)
    w1 = _uniform(rng, (3, W), 1 / math.sqrt(3)).astype(np.float32)
    b1 = _uniform(rng, (W,), 1 / math.sqrt(3)).astype(np.float32)
    w2 = _uniform(rng, (W, W), 1 / math.sqrt(W)).astype(np.float32)
    b2 = _uniform(rng, (W,), 1 / math.sqrt(W)).astype(np.float32)
    w3 = _uniform(rng, (W, N * C), 1 / math.sqrt(W)).astype(np.float32)
    b3 = _uniform(rng, (N * C,), 1 / math.sqrt(W)).astype(np.float32)
    return HyenaNDInputs(B=B, X=X, Y=Y, Z=Z, C=C, N=N, W=W, u=u, w_in=w_in, dskip=dskip,
                         gate_a=gate_a, gate_b=gate_b, w_out=w_out, w1=w1, b1=b1, w2=w2,
                         b2=b2, w3=w3, b3=b3, decay=decay_rates(C), circular=circular,
                         meta=dict(seed=seed, u_mean_spread=u_mean_spread))


@dataclass
class HyenaNDFilmInputs:
    """A 3D workload with register-token conditioning (per-sample FiLM kernels)."""
    base: HyenaNDInputs   # grid input, projections, skips, SIREN weights (decay and gates unused)
    reg: np.ndarray       # [B, R, C] register activations
    q: np.ndarray         # [C] register score vector
    film_w: np.ndarray    # [4, C, W] gamma_1, beta_1, gamma_2, beta_2 projections of z
    film_b: np.ndarray    # [4, W]
    omega0: np.ndarray    # [W] first-layer frequency factors
    window: np.ndarray    # [C] Gaussian window rates

    def __getattr__(self, name):
        if name == "base":
            raise AttributeError(name)
        return getattr(self.base, name)

    @property
    def film_filter_params(self):
        b = self.base
        return dict(w1=b.w1, b1=b.b1, w2=b.w2, b2=b.b2, w3=b.w3, b3=b.b3, omega0=self.omega0,
                    window=self.window)


def make_nd_film(seed: int, B: int, X: int, Y: int, Z: int, C: int, N: int = 2, W: int = 64, R: int = 4,
                 circular: bool = False) -> HyenaNDFilmInputs:
    """Draw one register-conditioned 3D workload (fp32).

    The grid part is make_nd's (same seed). Then: reg ~ N(0, 1) [B, R, C];
    q ~ N(0, 1/C); film_w ~ N(0, 0.25/C); film_b = (1, 0, 1, 0) per row plus
    U(-0.1, 0.1), so that gamma stays near 1 and beta near 0; omega0 in four
    blocks of W/4 units at 1, 3, 10 and 30 (frequency blocks across the hidden
    units); window rates log-spaced over [0.5, 20] across the channels.
    """
    base = make_nd(seed, B, X, Y, Z, C, N=N, W=W, circular=circular)
    rng = np.random.default_rng(seed + 7919)
    reg = rng.standard_normal((B, R, C)).astype(np.float32)
    q = (rng.standard_normal(C) / math.sqrt(C)).astype(np.float32)
    film_w = (rng.standard_normal((4, C, W)) * (0.5 / math.sqrt(C))).astype(np.float32)
    film_b = (np.array([1.0, 0.0, 1.0, 0.0])[:, None] + _uniform(rng, (4, W), 0.1)).astype(np.float32)
    omega0 = np.repeat(np.array([1.0, 3.0, 10.0, 30.0]), -(-W // 4))[:W].astype(np.float32)
    window = np.geomspace(0.5, 20.0, C).astype(np.float32)
    return HyenaNDFilmInputs(base=base, reg=reg, q=q, film_w=film_w, film_b=film_b, omega0=omega0,
                             window=window)


# The five workloads. Names describe what each is; seeds are 1..5 in this order.
CONFIGS = {
    "order2_f32_L1k_D64": dict(kind="1d", seed=1, B=1, L=1024, D=64, N=2, K=8, dtype="f32"),
    "order2_bf16_B8_L2k_D768": dict(kind="1d", seed=2, B=8, L=2048, D=768, N=2, K=16,
                                    dtype="bf16", u_scale=1 / math.sqrt(768)),
    "order2_bf16_L64k_D768": dict(kind="1d", seed=3, B=1, L=65536, D=768, N=2, K=16,
                                  dtype="bf16", u_scale=1 / math.sqrt(768)),
    "order2_bf16_L1M_D256_dna": dict(kind="1d", seed=4, B=1, L=1 << 20, D=256, N=2, K=16,
                                     dtype="bf16", tokens=4),
    "nd3d_f32_B2_C128_64cube": dict(kind="nd", seed=5, B=2, X=64, Y=64, Z=64, C=128, N=2),
}

# Extra long-sequence test shapes (checked at sampled outputs): 256-point column
# DFTs with 2048- and 4096-point rows, between the 64k and the 1M workloads.
TEST_SHAPES = {
    "order2_bf16_L256k_D64": dict(kind="1d", seed=31, B=1, L=1 << 18, D=64, N=2, K=16, dtype="bf16",
                                  u_scale=1 / 8.0),
    "order2_f32_L512k_D64": dict(kind="1d", seed=32, B=1, L=1 << 19, D=64, N=2, K=16, dtype="f32"),
    # periodic 3D grids (circular boundary): the 3D workload's inputs and shape
    # with an unpadded 64^3 transform, and a 128^3 grid (128-point axes)
    "nd3d_circ_f32_B2_C128_64cube": dict(kind="nd", seed=5, B=2, X=64, Y=64, Z=64, C=128, N=2, circular=True),
    "nd3d_circ_f32_B1_C64_128cube": dict(kind="nd", seed=33, B=1, X=128, Y=128, Z=128, C=64, N=2,
                                         circular=True),
    # non-causal (two-sided filters): the 64k workload's inputs
    "order2_bf16_L64k_D768_noncausal": dict(kind="1d", seed=3, B=1, L=65536, D=768, N=2, K=16, dtype="bf16",
                                            u_scale=1 / math.sqrt(768), causal=False),
    # 2D image grids (X = 1): 64 x 64 patch grids at a ViT-Small width, zero padded
    "nd2d_f32_B8_C384_64sq": dict(kind="nd", seed=34, B=8, X=1, Y=64, Z=64, C=384, N=2),
    # register-conditioned (FiLM) kernels, one per sample, on the 3D workload's grid
    "nd3d_film_f32_B2_C128_64cube": dict(kind="nd_film", seed=35, B=2, X=64, Y=64, Z=64, C=128, N=2, W=64, R=4),
    # Full-length / full-grid shapes at the narrowest width the library takes
    # (64 channels), checked at every output: the transform kernels that only the
    # long and large workloads launch (64k bf16 four-step, 1M with 8192-point
    # rows, zero-padded 64^3 planes and pencils, 128^3 periodic grids) run here
    # with the same lengths, grids and storage types as there.
    "order2_bf16_L64k_D64": dict(kind="1d", seed=36, B=1, L=65536, D=64, N=2, K=16, dtype="bf16", u_scale=1 / 8.0),
    "order2_bf16_L64k_D64_noncausal": dict(kind="1d", seed=37, B=1, L=65536, D=64, N=2, K=16, dtype="bf16",
                                           u_scale=1 / 8.0, causal=False),
    "order2_bf16_L1M_D64_dna": dict(kind="1d", seed=38, B=1, L=1 << 20, D=64, N=2, K=16, dtype="bf16", tokens=4),
    "nd3d_f32_B2_C64_64cube": dict(kind="nd", seed=39, B=2, X=64, Y=64, Z=64, C=64, N=2, u_mean_spread=0.5),
    # a lone sample: the packed field's second half is empty
    "nd3d_f32_B1_C64_64cube": dict(kind="nd", seed=42, B=1, X=64, Y=64, Z=64, C=64, N=2, u_mean_spread=0.5),
    "nd3d_film_f32_B1_C64_64cube": dict(kind="nd_film", seed=40, B=1, X=64, Y=64, Z=64, C=64, N=2, W=64, R=4),
    "nd3d_film_f32_B2_C64_64cube": dict(kind="nd_film", seed=41, B=2, X=64, Y=64, Z=64, C=64, N=2, W=64, R=4),
}


def make_config(name: str):
    cfg = dict(CONFIGS[name] if name in CONFIGS else TEST_SHAPES[name])
    kind = cfg.pop("kind")
    if kind == "1d":
        return make_1d(**cfg)
    if kind == "nd_film":
        return make_nd_film(**cfg)
    return make_nd(**cfg)


def sample_positions(L: int, count: int, seed: int = 0) -> np.ndarray:
    """Sorted sample of time indices: both ends, the first few, and uniform draws."""
    rng = np.random.default_rng(10_000 + seed)
    fixed = [0, 1, 2, L // 2, L - 2, L - 1]
    extra = rng.integers(0, L, size=max(0, count - len(fixed)))
    return np.unique(np.clip(np.concatenate([fixed, extra]), 0, L - 1)).astype(np.int64)
