"""Python binding of the MI355X sparse-MoE layer library (``libmoe.so``).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  The
functions carry the C-ABI names (``moe_route``, ``moe_dispatch``,
``moe_expert_ffn``, ``moe_combine``, ``moe_forward``); see ``include/moe.h``
for argument meaning, layouts and error behaviour.

There is no fallback: if ``libmoe.so`` is missing, importing the library
raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_GATE_SOFTMAX, MOE_GATE_SIGMOID = 0, 1
MOE_F_RENORM, MOE_F_RESIDUAL, MOE_F_LOGITS_IN, MOE_F_TOPK_IN, MOE_F_STATS = 1, 2, 4, 8, 16
MOE_F_EXPERT_CHOICE = 32
MOE_F_PACKED_UP, MOE_F_PACKED_DOWN = 64, 128
# expert-weight layouts: which GEMMs' weights are packed by moe_pack_weights
PACKINGS = {"none": 0, "up": MOE_F_PACKED_UP, "down": MOE_F_PACKED_DOWN, "both": MOE_F_PACKED_UP | MOE_F_PACKED_DOWN}
# moe_drop_policy: which assignments an expert over capacity drops
DROP_POLICIES = {"first_come": 0, "affinity": 1, "reroute": 2}
# router statistics after the E per-expert mean probabilities (moe.h, MOE_STAT_*)
STAT_NAMES = ("balance", "z_loss", "lif", "cv", "entropy_p", "entropy_f")

KERNEL_NAMES = ["router_logits", "router_topk", "route_scan", "route_scatter", "dispatch", "ffn_tiles",
                "gemm_gate_up", "gemm_down", "combine", "shared_gate_up", "shared_down"]


class MoeError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        super().__init__(f"{fn}: {_status_name(status)}: {detail}")
        self.status = status


class MoeConfig(ctypes.Structure):
    _fields_ = [
        ("tokens", ctypes.c_int64), ("d_model", ctypes.c_int64), ("d_ff", ctypes.c_int64),
        ("n_experts", ctypes.c_int64), ("top_k", ctypes.c_int64), ("gate", ctypes.c_int32),
        ("flags", ctypes.c_uint32), ("capacity_factor", ctypes.c_double), ("n_shared", ctypes.c_int64),
        ("d_ff_shared", ctypes.c_int64), ("act_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32), ("drop_policy", ctypes.c_int32),
    ]


class MoeScales(ctypes.Structure):
    """Per-row fp32 scales of FP8 E4M3 expert weights (device pointers)."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("w1", "w3", "w2", "ws1", "ws3", "ws2")]


class MoeRouting(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("logits", "topk_idx", "topk_w", "counts", "offsets", "dest", "row_src", "dropped", "stats")]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load ``libmoe.so`` (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with mixture_experts_sparse_route_amd/build.py")
    lib = ctypes.CDLL(path)
    vp, sz, i64, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64, ctypes.c_int
    C, R = ctypes.POINTER(MoeConfig), ctypes.POINTER(MoeRouting)
    sigs = {
        "moe_workspace_size": [C, ctypes.POINTER(sz)],
        "moe_max_rows": [C, ctypes.POINTER(i64)],
        "moe_route": [C, vp, vp, vp, vp, R, vp, sz, vp],
        "moe_dispatch": [C, vp, R, vp, vp],
        "moe_expert_ffn": [C, vp, vp, i64, i64, vp, vp, vp, ctypes.POINTER(MoeScales), vp, vp, sz, vp],
        "moe_combine": [C, vp, R, vp, vp, vp, vp],
        "moe_forward": [C, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(MoeScales), vp, R, vp, sz, vp],
        "moe_forward_noalloc": [C, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(MoeScales), vp, R, vp],
        "moe_pack_weights": [vp, vp, i64, i64, i64, i32, vp],
        "moe_profile_enable": [ctypes.c_uint32],
        "moe_profile_reset": [],
        "moe_profile_read": [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_kernel_name.argtypes = [ctypes.c_int]
    lib.moe_kernel_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _status_name(s: int) -> str:
    try:
        return load_library().moe_status_string(s).decode()
    except Exception:  # pragma: no cover - only when the library is absent
        return str(s)


def _check(status: int, fn: str):
    if status != MOE_OK:
        raise MoeError(status, fn, load_library().moe_last_error().decode())


# ------------------------------------------------------------------ config --

@dataclass
class LayerSpec:
    """Layer description, mirrors ``moe_config``."""
    tokens: int
    d_model: int
    d_ff: int
    n_experts: int
    top_k: int
    gate: int = MOE_GATE_SOFTMAX
    renorm: bool = True
    residual: bool = False
    capacity_factor: float = 0.0
    n_shared: int = 0
    d_ff_shared: int = 0
    dtype: str = "bf16"            # "bf16" or "f32" (activations and expert weights)
    wdtype: str = ""               # "fp8": expert weights are E4M3 codes with per-row scales (bf16 layer)
    out_dtype: Optional[str] = None  # dtype of y; None = dtype ("f32" allowed for a bf16 layer)
    logits_in: bool = False
    topk_in: bool = False
    stats: bool = False
    drop_policy: str = "first_come"   # a key of DROP_POLICIES
    expert_choice: bool = False       # expert-choice routing (routing arrays in the K = E form)
    packed: str = "none"              # a key of PACKINGS: weights in moe_pack_weights' layout (bf16)

    def config(self) -> MoeConfig:
        flags = ((MOE_F_RENORM if self.renorm else 0) | (MOE_F_RESIDUAL if self.residual else 0)
                 | (MOE_F_LOGITS_IN if self.logits_in else 0) | (MOE_F_TOPK_IN if self.topk_in else 0)
                 | (MOE_F_STATS if self.stats else 0) | (MOE_F_EXPERT_CHOICE if self.expert_choice else 0)
                 | PACKINGS[self.packed])
        dt = MOE_BF16 if self.dtype == "bf16" else MOE_F32
        ot = dt if self.out_dtype is None else (MOE_BF16 if self.out_dtype == "bf16" else MOE_F32)
        return MoeConfig(self.tokens, self.d_model, self.d_ff, self.n_experts, self.top_k, self.gate, flags,
                         float(self.capacity_factor), self.n_shared, self.d_ff_shared, dt,
                         MOE_FP8_E4M3 if self.wdtype == "fp8" else dt, ot,
                         DROP_POLICIES[self.drop_policy])


def _cfg(spec_or_cfg) -> MoeConfig:
    return spec_or_cfg.config() if isinstance(spec_or_cfg, LayerSpec) else spec_or_cfg


def workspace_size(spec) -> int:
    n = ctypes.c_size_t()
    _check(load_library().moe_workspace_size(ctypes.byref(_cfg(spec)), ctypes.byref(n)), "moe_workspace_size")
    return n.value


def max_rows(spec) -> int:
    n = ctypes.c_int64()
    _check(load_library().moe_max_rows(ctypes.byref(_cfg(spec)), ctypes.byref(n)), "moe_max_rows")
    return n.value


# ----------------------------------------------------------- torch plumbing --

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


class Routing:
    """Device routing arrays (``moe_routing``) for one config."""

    def __init__(self, spec, device="cuda"):
        torch = _torch()
        c = _cfg(spec)
        T, E = c.tokens, c.n_experts
        K = E if c.flags & MOE_F_EXPERT_CHOICE else c.top_k   # expert choice: the K = E form
        self.logits = torch.empty((T, E), dtype=torch.float32, device=device)
        self.topk_idx = torch.empty((T, K), dtype=torch.int32, device=device)
        self.topk_w = torch.empty((T, K), dtype=torch.float32, device=device)
        self.counts = torch.empty((E,), dtype=torch.int32, device=device)
        self.offsets = torch.empty((E + 1,), dtype=torch.int32, device=device)
        self.dest = torch.empty((T * K,), dtype=torch.int32, device=device)
        self.row_src = torch.empty((max(T * K, 1),), dtype=torch.int32, device=device)
        self.dropped = torch.empty((T * K,), dtype=torch.uint8, device=device)
        self.stats = torch.empty((E + len(STAT_NAMES),), dtype=torch.float64, device=device)

    def struct(self) -> MoeRouting:
        return MoeRouting(*(_ptr(getattr(self, n)) for n in
                            ("logits", "topk_idx", "topk_w", "counts", "offsets", "dest", "row_src", "dropped",
                             "stats")))

    def statistics(self) -> dict:
        """The router statistics written with MOE_F_STATS, as host floats:
        {'P': per-expert mean probability [E], 'balance', 'z_loss', 'lif',
        'cv', 'entropy_p', 'entropy_f'}."""
        v = self.stats.cpu().numpy()
        E = v.shape[0] - len(STAT_NAMES)
        d = {"P": v[:E].copy()}
        for i, n in enumerate(STAT_NAMES):
            d[n] = float(v[E + i])
        return d


def alloc_workspace(spec, device="cuda"):
    """A 256-byte aligned device workspace of ``moe_workspace_size`` bytes."""
    torch = _torch()
    n = workspace_size(spec)
    return torch.empty((max(n, 1) + 256,), dtype=torch.uint8, device=device), n


def _ws_ptr(ws) -> int:
    p = ws.data_ptr()
    return (p + 255) // 256 * 256


def _ws_bytes(ws) -> int:
    return ws.numel() - (_ws_ptr(ws) - ws.data_ptr())


# -------------------------------------------------------------- entry points --

def moe_route(spec, x, Wg, logit_bias, sel_bias, routing: Routing, ws, stream=None):
    r = routing.struct()
    _check(load_library().moe_route(ctypes.byref(_cfg(spec)), _ptr(x), _ptr(Wg), _ptr(logit_bias), _ptr(sel_bias),
                                    ctypes.byref(r), _ws_ptr(ws), _ws_bytes(ws), _stream(stream)), "moe_route")


def moe_dispatch(spec, x, routing: Routing, xp, stream=None):
    r = routing.struct()
    _check(load_library().moe_dispatch(ctypes.byref(_cfg(spec)), _ptr(x), ctypes.byref(r), _ptr(xp),
                                       _stream(stream)), "moe_dispatch")


def _scales(scales):
    """MoeScales from a dict of device tensors (keys w1, w3, w2, ws1, ws3, ws2)."""
    if scales is None:
        return None
    return ctypes.byref(MoeScales(*(_ptr(scales.get(k)) for k in ("w1", "w3", "w2", "ws1", "ws3", "ws2"))))


def moe_expert_ffn(spec, xp, offsets, n_groups, max_rows_, W1, W3, W2, yp, ws, stream=None, scales=None):
    """scales: dict of device fp32 row-scale tensors for FP8 E4M3 weights."""
    _check(load_library().moe_expert_ffn(ctypes.byref(_cfg(spec)), _ptr(xp), _ptr(offsets), n_groups, max_rows_,
                                         _ptr(W1), _ptr(W3), _ptr(W2), _scales(scales), _ptr(yp), _ws_ptr(ws),
                                         _ws_bytes(ws), _stream(stream)), "moe_expert_ffn")


def moe_pack_weights(src, dst, stream=None):
    """dst <- src [groups, N, K] (bf16, or uint8 E4M3 codes) in the packed
    layout [groups, N/64, K/64, 64, 64] (moe.h); src is 3-D, dst any device
    tensor of the same size."""
    G, N, K = src.shape
    wd = MOE_FP8_E4M3 if src.element_size() == 1 else MOE_BF16
    _check(load_library().moe_pack_weights(_ptr(src), _ptr(dst), G, N, K, wd, _stream(stream)), "moe_pack_weights")


def moe_combine(spec, yp, routing: Routing, shared_out, x_residual, y, stream=None):
    r = routing.struct()
    _check(load_library().moe_combine(ctypes.byref(_cfg(spec)), _ptr(yp), ctypes.byref(r), _ptr(shared_out),
                                      _ptr(x_residual), _ptr(y), _stream(stream)), "moe_combine")


def moe_forward(spec, x, Wg, logit_bias, sel_bias, W1, W3, W2, Ws1, Ws3, Ws2, y, routing: Optional[Routing], ws,
                stream=None, scales=None):
    """scales: dict of device fp32 row-scale tensors for FP8 E4M3 weights."""
    r = routing.struct() if routing is not None else None
    _check(load_library().moe_forward(ctypes.byref(_cfg(spec)), _ptr(x), _ptr(Wg), _ptr(logit_bias), _ptr(sel_bias),
                                      _ptr(W1), _ptr(W3), _ptr(W2), _ptr(Ws1), _ptr(Ws3), _ptr(Ws2),
                                      _scales(scales), _ptr(y),
                                      ctypes.byref(r) if r is not None else None, _ws_ptr(ws), _ws_bytes(ws),
                                      _stream(stream)), "moe_forward")


# Bytes of the built-in scratch array of moe_forward_noalloc (per GPU).
NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_forward_noalloc(spec, x, Wg, logit_bias, sel_bias, W1, W3, W2, Ws1, Ws3, Ws2, y,
                        routing: Optional[Routing], stream=None, scales=None):
    """moe_forward without a workspace: the library's built-in scratch array
    of NOALLOC_SCRATCH_BYTES per GPU (see moe.h); allocates nothing."""
    r = routing.struct() if routing is not None else None
    _check(load_library().moe_forward_noalloc(ctypes.byref(_cfg(spec)), _ptr(x), _ptr(Wg), _ptr(logit_bias),
                                              _ptr(sel_bias), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(Ws1), _ptr(Ws3),
                                              _ptr(Ws2), _scales(scales), _ptr(y),
                                              ctypes.byref(r) if r is not None else None, _stream(stream)),
           "moe_forward_noalloc")


# ---------------------------------------------------------------- profiling --

def profile_enable(kernels=None):
    """Time the named kernels (all if None; [] turns timing off)."""
    if kernels is None:
        mask = (1 << len(KERNEL_NAMES)) - 1
    else:
        mask = 0
        for k in kernels:
            mask |= 1 << KERNEL_NAMES.index(k)
    _check(load_library().moe_profile_enable(mask), "moe_profile_enable")


def profile_reset():
    _check(load_library().moe_profile_reset(), "moe_profile_reset")


def profile_read() -> dict:
    """{kernel name: (total ms, launches)} since the last reset."""
    lib = load_library()
    out = {}
    for i, name in enumerate(KERNEL_NAMES):
        ms, n = ctypes.c_double(), ctypes.c_int64()
        _check(lib.moe_profile_read(i, ctypes.byref(ms), ctypes.byref(n)), "moe_profile_read")
        out[name] = (ms.value, n.value)
    return out
