"""ctypes binding of libhyena.so (argument marshalling only).

Every step of the forward path runs in the library's HIP kernels; PyTorch only
provides device memory and the current stream. If the library is missing this
module raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhyena.so")

HYENA_F32 = 0
HYENA_BF16 = 1
STATUS = {0: "HYENA_OK", 1: "HYENA_ERR_INVALID_ARG", 2: "HYENA_ERR_UNSUPPORTED", 3: "HYENA_ERR_WORKSPACE",
          4: "HYENA_ERR_LAYER_MISMATCH", 5: "HYENA_ERR_HIP"}

_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_i = ctypes.c_int


class FilterParams(ctypes.Structure):
    _fields_ = [("pe_freqs", _i), ("width", _i), ("w1", _vp), ("b1", _vp), ("w2", _vp), ("b2", _vp),
                ("w3", _vp), ("b3", _vp), ("decay", _vp)]


class Layer(ctypes.Structure):
    _fields_ = [("L", _i), ("D", _i), ("N", _i), ("built", _i), ("cache", _vp), ("cache_bytes", _sz),
                ("direction", _i)]


# hyena_direction
CAUSAL = 0
NONCAUSAL = 1


class NDFilterParams(ctypes.Structure):
    _fields_ = [("width", _i), ("w1", _vp), ("b1", _vp), ("w2", _vp), ("b2", _vp), ("w3", _vp), ("b3", _vp),
                ("decay", _vp)]


class NDLayer(ctypes.Structure):
    _fields_ = [("X", _i), ("Y", _i), ("Z", _i), ("C", _i), ("N", _i), ("built", _i), ("cache", _vp),
                ("cache_bytes", _sz), ("boundary", _i)]


# hyena_nd_boundary
ND_ZERO_PAD = 0
ND_CIRCULAR = 1


class NDFilmParams(ctypes.Structure):
    _fields_ = [("registers", _i), ("q", _vp), ("film_w", _vp), ("film_b", _vp), ("omega0", _vp)]


# name -> (restype, argtypes)
SIGNATURES = {
    "hyena_status_str": (ctypes.c_char_p, [_i]),
    "hyena_cache_bytes": (_sz, [_i, _i, _i]),
    "hyena_filter_workspace_bytes": (_sz, [_i, _i, _i]),
    "hyena_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "hyena_layer_init": (_i, [ctypes.POINTER(Layer), _i, _i, _i, _vp, _sz]),
    "hyena_layer_init_ex": (_i, [ctypes.POINTER(Layer), _i, _i, _i, _i, _vp, _sz]),
    "hyena_filter_workspace_bytes_ex": (_sz, [_i, _i, _i, _i]),
    "hyena_filter_gen": (_i, [ctypes.POINTER(Layer), ctypes.POINTER(FilterParams), _vp, _vp, _sz, _vp]),
    "hyena_fwd": (_i, [ctypes.POINTER(Layer), _vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _sz, _vp]),
    "hyena_fwd_profiled": (_i, [ctypes.POINTER(Layer), _vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _sz, _vp,
                                ctypes.POINTER(_vp)]),
    "hyena_fwd_noalloc": (_i, [ctypes.POINTER(Layer), _vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _vp]),
    "hyena_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "hyena_bwd": (_i, [ctypes.POINTER(Layer), _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                       _sz, _vp]),
    "hyena_filter_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "hyena_filter_bwd": (_i, [ctypes.POINTER(Layer), ctypes.POINTER(FilterParams), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                              _vp, _vp, _sz, _vp]),
    "hyena_nd_cache_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "hyena_nd_filter_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "hyena_nd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "hyena_nd_layer_init": (_i, [ctypes.POINTER(NDLayer), _i, _i, _i, _i, _i, _vp, _sz]),
    "hyena_nd_cache_bytes_ex": (_sz, [_i, _i, _i, _i, _i, _i]),
    "hyena_nd_filter_workspace_bytes_ex": (_sz, [_i, _i, _i, _i, _i, _i]),
    "hyena_nd_workspace_bytes_ex": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "hyena_nd_layer_init_ex": (_i, [ctypes.POINTER(NDLayer), _i, _i, _i, _i, _i, _i, _vp, _sz]),
    "hyena_nd_filter_gen": (_i, [ctypes.POINTER(NDLayer), ctypes.POINTER(NDFilterParams), _vp, _vp, _sz, _vp]),
    "hyena_nd_fwd": (_i, [ctypes.POINTER(NDLayer), _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _sz, _vp]),
    "hyena_nd_fwd_profiled": (_i, [ctypes.POINTER(NDLayer), _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _sz, _vp,
                                   ctypes.POINTER(_vp)]),
    "hyena_nd_film_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "hyena_nd_film_fwd": (_i, [_i, _i, _i, _i, _i, _i, ctypes.POINTER(NDFilterParams), ctypes.POINTER(NDFilmParams),
                               _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp, _sz, _vp]),
    "hyena_nd_film_fwd_profiled": (_i, [_i, _i, _i, _i, _i, _i, ctypes.POINTER(NDFilterParams),
                                        ctypes.POINTER(NDFilmParams), _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp,
                                        _sz, _vp, ctypes.POINTER(_vp)]),
}

_lib = None


class HyenaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


def lib() -> ctypes.CDLL:
    """Loads libhyena.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m subquadratic_sequence_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def _check(status: int, where: str):
    if status != 0:
        raise HyenaError(status, where)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return HYENA_F32
    if t.dtype == torch.bfloat16:
        return HYENA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


# ------------------------------------------------------------------ 1D


def hyena_cache_bytes(L: int, D: int, N: int) -> int:
    return lib().hyena_cache_bytes(L, D, N)


def hyena_filter_workspace_bytes(L: int, D: int, N: int) -> int:
    return lib().hyena_filter_workspace_bytes(L, D, N)


def hyena_filter_workspace_bytes_ex(L: int, D: int, N: int, direction: int) -> int:
    return lib().hyena_filter_workspace_bytes_ex(L, D, N, direction)


def hyena_workspace_bytes(B: int, L: int, D: int, N: int, dtype: int) -> int:
    return lib().hyena_workspace_bytes(B, L, D, N, dtype)


class HyenaLayer:
    """One layer's filter cache (device memory owned by this object); direction
    CAUSAL (default) or NONCAUSAL (two-sided filters)."""

    def __init__(self, L: int, D: int, N: int, device="cuda", direction: int = CAUSAL):
        nbytes = hyena_cache_bytes(L, D, N)
        if nbytes == 0:
            raise HyenaError(2, "hyena_cache_bytes")
        self.cache = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.c = Layer()
        _check(lib().hyena_layer_init_ex(ctypes.byref(self.c), L, D, N, direction, _ptr(self.cache), nbytes),
               "hyena_layer_init_ex")
        self.L, self.D, self.N = L, D, N
        self.direction = direction


def hyena_filter_gen(layer: HyenaLayer, w1, b1, w2, b2, w3, b3, decay, pe_freqs: int, h_out=None, ws=None):
    """Generates the implicit filters and caches their spectra in layer.cache."""
    width = w1.shape[1]
    p = FilterParams(pe_freqs, width, _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(w3), _ptr(b3), _ptr(decay))
    need = hyena_filter_workspace_bytes_ex(layer.L, layer.D, layer.N, layer.direction)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=layer.cache.device)
    st = lib().hyena_filter_gen(ctypes.byref(layer.c), ctypes.byref(p), _ptr(h_out), _ptr(ws), ws.numel(),
                                _stream())
    _check(st, "hyena_filter_gen")
    return h_out


def hyena_fwd(layer: HyenaLayer, u, w_in, short_w, dskip, w_out, y=None, ws=None):
    """y = Hyena(u) for u [B, L, D] (float32 or bfloat16)."""
    B = u.shape[0]
    dt = _dtype_code(u)
    if y is None:
        y = torch.empty_like(u)
    if ws is None:
        need = hyena_workspace_bytes(B, layer.L, layer.D, layer.N, dt)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=u.device)
    st = lib().hyena_fwd(ctypes.byref(layer.c), _ptr(u), _ptr(w_in), _ptr(short_w), _ptr(dskip), _ptr(w_out),
                         B, dt, _ptr(y), _ptr(ws), ws.numel(), _stream())
    _check(st, "hyena_fwd")
    return y


def hyena_fwd_noalloc(layer: HyenaLayer, u, w_in, short_w, dskip, w_out, y=None):
    """hyena_fwd with the workspace inside the library (no workspace argument)."""
    B = u.shape[0]
    if y is None:
        y = torch.empty_like(u)
    st = lib().hyena_fwd_noalloc(ctypes.byref(layer.c), _ptr(u), _ptr(w_in), _ptr(short_w), _ptr(dskip),
                                 _ptr(w_out), B, _dtype_code(u), _ptr(y), _stream())
    _check(st, "hyena_fwd_noalloc")
    return y


def hyena_fwd_profiled(layer: HyenaLayer, u, w_in, short_w, dskip, w_out, y, ws, events):
    """hyena_fwd that also records four torch.cuda.Event (enable_timing=True) at the
    stage boundaries on the current stream: before the in-projection, after it,
    after the long convolutions, after the out-projection. Does not synchronise."""
    B = u.shape[0]
    if len(events) != 4:
        raise ValueError("hyena_fwd_profiled takes 4 events")
    for ev in events:
        if not ev.cuda_event:  # torch creates the HIP event on its first record
            ev.record()
    handles = (_vp * 4)(*[ev.cuda_event for ev in events])
    st = lib().hyena_fwd_profiled(ctypes.byref(layer.c), _ptr(u), _ptr(w_in), _ptr(short_w), _ptr(dskip),
                                  _ptr(w_out), B, _dtype_code(u), _ptr(y), _ptr(ws), ws.numel(), _stream(), handles)
    _check(st, "hyena_fwd_profiled")


# ------------------------------------------------------------------ 1D backward


def hyena_bwd_workspace_bytes(B, L, D, N, dtype, direction=CAUSAL) -> int:
    return lib().hyena_bwd_workspace_bytes(B, L, D, N, dtype, direction)


def hyena_bwd(layer: HyenaLayer, u, w_in, short_w, dskip, w_out, dy, ws=None):
    """Gradients of sum(dy * y), y = hyena_fwd(layer, u, ...): a dict with du
    (dtype of u) and fp32 dw_in, dshort_w, ddskip, dw_out, dh."""
    B = u.shape[0]
    dt = _dtype_code(u)
    L, D, N = layer.L, layer.D, layer.N
    dev = u.device
    f32 = dict(dtype=torch.float32, device=dev)
    hl = L if layer.direction == CAUSAL else 2 * L
    g = dict(du=torch.empty_like(u), dw_in=torch.empty(D, (N + 1) * D, **f32),
             dshort_w=torch.empty((N + 1) * D, 3, **f32), ddskip=torch.empty(N, D, **f32),
             dw_out=torch.empty(D, D, **f32), dh=torch.empty(N, D, hl, **f32))
    if ws is None:
        need = hyena_bwd_workspace_bytes(B, L, D, N, dt, layer.direction)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib().hyena_bwd(ctypes.byref(layer.c), _ptr(u), _ptr(w_in), _ptr(short_w), _ptr(dskip), _ptr(w_out),
                         _ptr(dy), B, dt, _ptr(g["du"]), _ptr(g["dw_in"]), _ptr(g["dshort_w"]), _ptr(g["ddskip"]),
                         _ptr(g["dw_out"]), _ptr(g["dh"]), _ptr(ws), ws.numel(), _stream())
    _check(st, "hyena_bwd")
    return g


def hyena_filter_bwd_workspace_bytes(L, D, N, pe_freqs, width, direction=CAUSAL) -> int:
    return lib().hyena_filter_bwd_workspace_bytes(L, D, N, pe_freqs, width, direction)


def hyena_filter_bwd(layer: HyenaLayer, w1, b1, w2, b2, w3, b3, decay, pe_freqs: int, dh, ws=None):
    """Gradients of sum(dh * h) with respect to the filter generator's parameters:
    a dict with w1, b1, w2, b2, w3, b3, decay (fp32, shapes of the parameters)."""
    width = w1.shape[1]
    p = FilterParams(pe_freqs, width, _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(w3), _ptr(b3), _ptr(decay))
    g = {k: torch.empty_like(v) for k, v in (("w1", w1), ("b1", b1), ("w2", w2), ("b2", b2), ("w3", w3), ("b3", b3),
                                              ("decay", decay))}
    if ws is None:
        need = hyena_filter_bwd_workspace_bytes(layer.L, layer.D, layer.N, pe_freqs, width, layer.direction)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dh.device)
    st = lib().hyena_filter_bwd(ctypes.byref(layer.c), ctypes.byref(p), _ptr(dh), _ptr(g["w1"]), _ptr(g["b1"]),
                                _ptr(g["w2"]), _ptr(g["b2"]), _ptr(g["w3"]), _ptr(g["b3"]), _ptr(g["decay"]),
                                _ptr(ws), ws.numel(), _stream())
    _check(st, "hyena_filter_bwd")
    return g


# ------------------------------------------------------------------ 3D


def hyena_nd_cache_bytes(X, Y, Z, C, N) -> int:
    return lib().hyena_nd_cache_bytes(X, Y, Z, C, N)


def hyena_nd_filter_workspace_bytes(X, Y, Z, C, N) -> int:
    return lib().hyena_nd_filter_workspace_bytes(X, Y, Z, C, N)


def hyena_nd_workspace_bytes(B, X, Y, Z, C, N) -> int:
    return lib().hyena_nd_workspace_bytes(B, X, Y, Z, C, N)


def hyena_nd_cache_bytes_ex(X, Y, Z, C, N, boundary) -> int:
    return lib().hyena_nd_cache_bytes_ex(X, Y, Z, C, N, boundary)


def hyena_nd_filter_workspace_bytes_ex(X, Y, Z, C, N, boundary) -> int:
    return lib().hyena_nd_filter_workspace_bytes_ex(X, Y, Z, C, N, boundary)


def hyena_nd_workspace_bytes_ex(B, X, Y, Z, C, N, boundary) -> int:
    return lib().hyena_nd_workspace_bytes_ex(B, X, Y, Z, C, N, boundary)


class HyenaNDLayer:
    """3D layer; boundary ND_ZERO_PAD (non-circular, default) or ND_CIRCULAR."""

    def __init__(self, X: int, Y: int, Z: int, C: int, N: int, device="cuda", boundary: int = ND_ZERO_PAD):
        nbytes = hyena_nd_cache_bytes_ex(X, Y, Z, C, N, boundary)
        if nbytes == 0:
            raise HyenaError(2, "hyena_nd_cache_bytes_ex")
        self.cache = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.c = NDLayer()
        _check(lib().hyena_nd_layer_init_ex(ctypes.byref(self.c), X, Y, Z, C, N, boundary, _ptr(self.cache),
                                            nbytes), "hyena_nd_layer_init_ex")
        self.X, self.Y, self.Z, self.C, self.N = X, Y, Z, C, N
        self.boundary = boundary


def hyena_nd_filter_gen(layer: HyenaNDLayer, w1, b1, w2, b2, w3, b3, decay, k_out=None, ws=None):
    width = w1.shape[1]
    p = NDFilterParams(width, _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(w3), _ptr(b3), _ptr(decay))
    need = hyena_nd_filter_workspace_bytes_ex(layer.X, layer.Y, layer.Z, layer.C, layer.N, layer.boundary)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=layer.cache.device)
    st = lib().hyena_nd_filter_gen(ctypes.byref(layer.c), ctypes.byref(p), _ptr(k_out), _ptr(ws), ws.numel(),
                                   _stream())
    _check(st, "hyena_nd_filter_gen")
    return k_out


def hyena_nd_fwd(layer: HyenaNDLayer, u, w_in, dskip, gate_a, gate_b, w_out, y=None, ws=None):
    B = u.shape[0]
    if y is None:
        y = torch.empty_like(u)
    if ws is None:
        need = hyena_nd_workspace_bytes_ex(B, layer.X, layer.Y, layer.Z, layer.C, layer.N, layer.boundary)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=u.device)
    st = lib().hyena_nd_fwd(ctypes.byref(layer.c), _ptr(u), _ptr(w_in), _ptr(dskip), _ptr(gate_a), _ptr(gate_b),
                            _ptr(w_out), B, _ptr(y), _ptr(ws), ws.numel(), _stream())
    _check(st, "hyena_nd_fwd")
    return y


def hyena_nd_fwd_profiled(layer: HyenaNDLayer, u, w_in, dskip, gate_a, gate_b, w_out, y, ws, events):
    """hyena_nd_fwd that also records four torch.cuda.Event (enable_timing=True) at the
    stage boundaries on the current stream: before the gates, after the
    in-projection, after the 3D convolutions, after the out-projection. Does not
    synchronise."""
    B = u.shape[0]
    if len(events) != 4:
        raise ValueError("hyena_nd_fwd_profiled takes 4 events")
    for ev in events:
        if not ev.cuda_event:  # torch creates the HIP event on its first record
            ev.record()
    handles = (_vp * 4)(*[ev.cuda_event for ev in events])
    st = lib().hyena_nd_fwd_profiled(ctypes.byref(layer.c), _ptr(u), _ptr(w_in), _ptr(dskip), _ptr(gate_a),
                                     _ptr(gate_b), _ptr(w_out), B, _ptr(y), _ptr(ws), ws.numel(), _stream(), handles)
    _check(st, "hyena_nd_fwd_profiled")


def hyena_nd_film_workspace_bytes(B, X, Y, Z, C, N, width, boundary=ND_ZERO_PAD) -> int:
    return lib().hyena_nd_film_workspace_bytes(B, X, Y, Z, C, N, width, boundary)


class HyenaNDFilm:
    """Weights of a register-conditioned 3D layer (device tensors, fp32): the SIREN
    (w1 [3, W], b1, w2 [W, W], b2, w3 [W, N C], b3), the Gaussian window rates
    [C], the register score vector q [C], the FiLM maps film_w [4, C, W] and
    film_b [4, W], and omega0 [W]."""

    def __init__(self, X, Y, Z, C, N, boundary, w1, b1, w2, b2, w3, b3, window, q, film_w, film_b, omega0):
        self.X, self.Y, self.Z, self.C, self.N, self.boundary = X, Y, Z, C, N, boundary
        self.t = (w1, b1, w2, b2, w3, b3, window, q, film_w, film_b, omega0)  # keeps the tensors alive
        self.width = w1.shape[1]
        self.p = NDFilterParams(self.width, _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(w3), _ptr(b3),
                                _ptr(window))
        self.registers = 0
        self.fp = NDFilmParams(0, _ptr(q), _ptr(film_w), _ptr(film_b), _ptr(omega0))


def _film_args(m: HyenaNDFilm, u, reg, w_in, dskip, w_out, y, k_out, ws):
    B = u.shape[0]
    m.fp.registers = reg.shape[1]
    if y is None:
        y = torch.empty_like(u)
    if ws is None:
        need = hyena_nd_film_workspace_bytes(B, m.X, m.Y, m.Z, m.C, m.N, m.width, m.boundary)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=u.device)
    args = [m.X, m.Y, m.Z, m.C, m.N, m.boundary, ctypes.byref(m.p), ctypes.byref(m.fp), _ptr(u), _ptr(reg),
            _ptr(w_in), _ptr(dskip), _ptr(w_out), B, _ptr(y), _ptr(k_out), _ptr(ws), ws.numel(), _stream()]
    return y, args


def hyena_nd_film_fwd(m: HyenaNDFilm, u, reg, w_in, dskip, w_out, y=None, k_out=None, ws=None):
    """Register-conditioned forward; reg [B, R, C]. k_out, if given, receives every
    sample's kernel [B, N, C, MX, MY, MZ]."""
    y, args = _film_args(m, u, reg, w_in, dskip, w_out, y, k_out, ws)
    _check(lib().hyena_nd_film_fwd(*args), "hyena_nd_film_fwd")
    return y


def hyena_nd_film_fwd_profiled(m: HyenaNDFilm, u, reg, w_in, dskip, w_out, y, ws, events):
    """hyena_nd_film_fwd recording five torch.cuda.Event (enable_timing=True) on the
    current stream: before the kernel synthesis, after it, after the in-projection,
    after the convolutions, after the out-projection. Does not synchronise."""
    if len(events) != 5:
        raise ValueError("hyena_nd_film_fwd_profiled takes 5 events")
    for ev in events:
        if not ev.cuda_event:
            ev.record()
    handles = (_vp * 5)(*[ev.cuda_event for ev in events])
    y, args = _film_args(m, u, reg, w_in, dskip, w_out, y, None, ws)
    _check(lib().hyena_nd_film_fwd_profiled(*args, handles), "hyena_nd_film_fwd_profiled")
    return y
