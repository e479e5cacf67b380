"""ctypes wrapper of the CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE: imported only by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``.  The HIP library never imports,
links or calls anything here.

All arrays are numpy, host memory.  bf16 tensors are ``uint16`` bit arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None

GATE_SOFTMAX = 0
GATE_SIGMOID = 1


class OrcLayer(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64), ("d", ctypes.c_int64), ("F", ctypes.c_int64), ("E", ctypes.c_int64),
        ("K", ctypes.c_int64), ("gate", ctypes.c_int32), ("renorm", ctypes.c_int32),
        ("residual", ctypes.c_int32), ("bf16", ctypes.c_int32), ("capacity_factor", ctypes.c_double),
        ("n_shared", ctypes.c_int64), ("Fs", ctypes.c_int64), ("round_h", ctypes.c_int32),
        ("w_fp8", ctypes.c_int32),
    ]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: -O2, OpenMP, no fast-math, no FMA contraction."""
    src = os.path.join(_HERE, "moe_oracle.c")
    stale = not os.path.exists(_LIB_PATH) or os.path.getmtime(src) > os.path.getmtime(_LIB_PATH)
    if force or stale:
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
                               src, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        P = ctypes.POINTER(OrcLayer)
        lib.orc_logits.argtypes = [P, vp, vp, vp, vp]
        lib.orc_select.argtypes = [P, vp, vp, vp, vp, vp]
        lib.orc_capacity.argtypes = [P]
        lib.orc_capacity.restype = i64
        lib.orc_permute.argtypes = [P, vp, vp, vp, vp, vp, vp]
        lib.orc_swiglu.argtypes = [i64, i64, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32]
        lib.orc_fp8_e4m3.argtypes = [ctypes.c_uint8]
        lib.orc_fp8_e4m3.restype = ctypes.c_double
        lib.orc_bf16_round.argtypes = [ctypes.c_double]
        lib.orc_bf16_round.restype = ctypes.c_double
        lib.orc_forward_rows.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         i64, vp]
        lib.orc_expert_choice.argtypes = [P, vp, i64, vp, vp]
        lib.orc_select_ranked.argtypes = [P, vp, vp, i64, vp, vp]
        lib.orc_select_ranked.restype = None
        lib.orc_permute_affinity.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
        lib.orc_permute_affinity.restype = None
        lib.orc_permute_reroute.argtypes = [P, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp]
        lib.orc_permute_reroute.restype = None
        lib.orc_router_stats.argtypes = [P, vp, vp, vp]
        lib.orc_router_stats.restype = None
        lib.orc_threads.argtypes = []
        lib.orc_threads.restype = i32
        lib.orc_combine.argtypes = [P, vp, vp, vp, vp, vp, vp]
        lib.orc_combine.restype = None
        for fn in (lib.orc_logits, lib.orc_select, lib.orc_permute, lib.orc_swiglu, lib.orc_forward_rows,
                   lib.orc_expert_choice):
            fn.restype = None
        _lib = lib
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous numpy"
    return a.ctypes.data


def layer(T, d, F, E, K, gate=GATE_SOFTMAX, renorm=True, residual=False, bf16=False, capacity_factor=0.0,
          n_shared=0, Fs=0, round_h=False, w_fp8=False) -> OrcLayer:
    """round_h: False (the definition) keeps the SwiGLU output h in double;
    True stores it in bf16 (ties to even) before the down projection, as a
    bf16 kernel does -- a tighter second reference, never the definition.
    w_fp8: expert weights are FP8 E4M3 codes with per-row scales."""
    return OrcLayer(T, d, F, E, K, gate, int(renorm), int(residual), int(bf16), float(capacity_factor),
                    n_shared, Fs, int(bool(round_h)), int(w_fp8))


def layer_of(wl, residual=False, round_h=False) -> OrcLayer:
    """OrcLayer for a ``moe_synth`` workload."""
    return layer(wl.T, wl.d, wl.F, wl.E, wl.K, gate=wl.gate, renorm=wl.renorm, residual=residual,
                 bf16=(wl.dtype == "bf16"), capacity_factor=wl.capacity_factor, n_shared=wl.n_shared, Fs=wl.Fs,
                 round_h=round_h, w_fp8=(getattr(wl, "wdtype", "") == "fp8"))


def fp8_e4m3(code: int) -> float:
    """The value of an OCP FP8 E4M3 code."""
    return float(_load().orc_fp8_e4m3(int(code)))


def bf16_round(v: float) -> float:
    """v rounded to the nearest bf16 value, ties to even."""
    return float(_load().orc_bf16_round(float(v)))


def threads() -> int:
    """OpenMP threads the oracle uses."""
    return int(_load().orc_threads())


def logits(L: OrcLayer, x, Wg, logit_bias=None) -> np.ndarray:
    out = np.empty((L.T, L.E), dtype=np.float32)
    _load().orc_logits(ctypes.byref(L), _p(x), _p(Wg), _p(logit_bias), _p(out))
    return out


def select(L: OrcLayer, lg, sel_bias=None):
    """-> (idx int32 [T,K], w float64 [T,K], gap float64 [T])"""
    idx = np.empty((L.T, L.K), dtype=np.int32)
    w = np.empty((L.T, L.K), dtype=np.float64)
    gap = np.empty((L.T,), dtype=np.float64)
    _load().orc_select(ctypes.byref(L), _p(np.ascontiguousarray(lg, dtype=np.float32)), _p(sel_bias), _p(idx),
                       _p(w), _p(gap))
    return idx, w, gap


def capacity(L: OrcLayer) -> int:
    return int(_load().orc_capacity(ctypes.byref(L)))


def permute(L: OrcLayer, idx):
    """-> dict(counts [E], offsets [E+1], dest [T*K], row_src [T*K], dropped [T*K])"""
    N = L.T * L.K
    out = dict(counts=np.empty(L.E, np.int32), offsets=np.empty(L.E + 1, np.int32), dest=np.empty(N, np.int32),
               row_src=np.empty(N, np.int32), dropped=np.empty(N, np.uint8))
    _load().orc_permute(ctypes.byref(L), _p(np.ascontiguousarray(idx, dtype=np.int32)), _p(out["counts"]),
                        _p(out["offsets"]), _p(out["dest"]), _p(out["row_src"]), _p(out["dropped"]))
    return out


def select_ranked(L: OrcLayer, lg, n: int, sel_bias=None):
    """The n best experts per token -> (idx int32 [T, n], w float64 [T, n])."""
    idx = np.empty((L.T, n), dtype=np.int32)
    w = np.empty((L.T, n), dtype=np.float64)
    _load().orc_select_ranked(ctypes.byref(L), _p(np.ascontiguousarray(lg, dtype=np.float32)), _p(sel_bias), n,
                              _p(idx), _p(w))
    return idx, w


def _perm_out(L: OrcLayer):
    N = L.T * L.K
    return dict(counts=np.empty(L.E, np.int32), offsets=np.empty(L.E + 1, np.int32), dest=np.empty(N, np.int32),
                row_src=np.empty(N, np.int32), dropped=np.empty(N, np.uint8))


def permute_affinity(L: OrcLayer, idx, aff):
    """a4, affinity-descending drop; aff: fp32 [T, K] affinities."""
    out = _perm_out(L)
    _load().orc_permute_affinity(ctypes.byref(L), _p(np.ascontiguousarray(idx, dtype=np.int32)),
                                 _p(np.ascontiguousarray(aff, dtype=np.float32)), _p(out["counts"]),
                                 _p(out["offsets"]), _p(out["dest"]), _p(out["row_src"]), _p(out["dropped"]))
    return out


def permute_reroute(L: OrcLayer, idx, w, alt_idx, alt_w):
    """a4, overflow re-routing.  alt_idx int32 [T, n_alt], alt_w float64 [T, n_alt].
    Adds 'idx' and 'w' (final expert and weight per assignment) to the result."""
    out = _perm_out(L)
    n_alt = alt_idx.shape[1] if alt_idx.ndim == 2 else 0
    out["idx"] = np.empty((L.T, L.K), np.int32)
    out["w"] = np.empty((L.T, L.K), np.float64)
    _load().orc_permute_reroute(ctypes.byref(L), _p(np.ascontiguousarray(idx, dtype=np.int32)),
                                _p(np.ascontiguousarray(w, dtype=np.float64)),
                                _p(np.ascontiguousarray(alt_idx, dtype=np.int32)),
                                _p(np.ascontiguousarray(alt_w, dtype=np.float64)), n_alt, _p(out["counts"]),
                                _p(out["offsets"]), _p(out["dest"]), _p(out["row_src"]), _p(out["dropped"]),
                                _p(out["idx"]), _p(out["w"]))
    return out


def alternates(L: OrcLayer, lg, sel_bias=None):
    """Re-routing candidates: ranks K .. min(2K, E)-1 of every token."""
    n = min(2 * L.K, L.E)
    ridx, rw = select_ranked(L, lg, n, sel_bias)
    return np.ascontiguousarray(ridx[:, L.K:]), np.ascontiguousarray(rw[:, L.K:])


def swiglu(W1, W3, W2, x, bf16: bool, threads: int = 1, round_h: bool = False, scales=None) -> np.ndarray:
    """One expert on one row: W1, W3 [F, d], W2 [d, F]; x float64 [d].
    uint8 weights are FP8 E4M3 codes; scales = (s1 [F], s3 [F], s2 [d])."""
    F, d = W1.shape
    out = np.empty(d, dtype=np.float64)
    wdt = 2 if W1.dtype == np.uint8 else int(bf16)
    s1, s3, s2 = (None, None, None) if scales is None else (np.ascontiguousarray(a, dtype=np.float32)
                                                             for a in scales)
    _load().orc_swiglu(d, F, wdt, int(round_h), _p(np.ascontiguousarray(W1)), _p(np.ascontiguousarray(W3)),
                       _p(np.ascontiguousarray(W2)), _p(s1), _p(s3), _p(s2),
                       _p(np.ascontiguousarray(x, dtype=np.float64)), _p(out), threads)
    return out


def forward_rows(L: OrcLayer, x, idx, w, dest, W1e, W3e, W2e, Ws1=None, Ws3=None, Ws2=None, tokens=None,
                 S1=None, S3=None, S2=None, Ss1=None, Ss3=None, Ss2=None):
    """y (float64 [n, d]) for the listed tokens (all tokens if None).

    W1e/W3e/W2e: either stacked arrays [E, ...] or lists of per-expert arrays
    (None for experts no listed token uses).  FP8 layers (L.w_fp8): S1/S3
    [E, F] and S2 [E, d] row scales (stacked or per-expert lists), Ss1/Ss3
    [S, Fs] and Ss2 [S, d]."""
    if tokens is None:
        tokens = np.arange(L.T, dtype=np.int64)
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)

    def ptrs(W):
        arr = (ctypes.c_void_p * L.E)()
        keep = []
        for e in range(L.E):
            a = W[e] if W is not None else None
            if a is not None:
                a = np.ascontiguousarray(a)
                keep.append(a)
                arr[e] = a.ctypes.data
        return arr, keep

    p1, k1 = ptrs(W1e)
    p3, k3 = ptrs(W3e)
    p2, k2 = ptrs(W2e)
    q1, kq1 = ptrs(S1)
    q3, kq3 = ptrs(S3)
    q2, kq2 = ptrs(S2)
    sh = [None if a is None else np.ascontiguousarray(a, dtype=np.float32) for a in (Ss1, Ss3, Ss2)]
    y = np.empty((len(tokens), L.d), dtype=np.float64)
    _load().orc_forward_rows(ctypes.byref(L), _p(x), _p(np.ascontiguousarray(idx, dtype=np.int32)),
                             _p(np.ascontiguousarray(w, dtype=np.float64)),
                             _p(None if dest is None else np.ascontiguousarray(dest, dtype=np.int32)),
                             ctypes.cast(p1, ctypes.c_void_p), ctypes.cast(p3, ctypes.c_void_p),
                             ctypes.cast(p2, ctypes.c_void_p), _p(Ws1), _p(Ws3), _p(Ws2),
                             None if S1 is None else ctypes.cast(q1, ctypes.c_void_p),
                             None if S3 is None else ctypes.cast(q3, ctypes.c_void_p),
                             None if S2 is None else ctypes.cast(q2, ctypes.c_void_p),
                             _p(sh[0]), _p(sh[1]), _p(sh[2]), _p(tokens), len(tokens), _p(y))
    del k1, k3, k2, kq1, kq3, kq2
    return y


STAT_NAMES = ["balance", "z_loss", "lif", "cv", "entropy_p", "entropy_f"]


def router_stats(L: OrcLayer, lg, idx) -> dict:
    """{'P': [E], 'balance', 'z_loss', 'lif', 'cv', 'entropy_p', 'entropy_f'} (float64)."""
    out = np.empty(L.E + len(STAT_NAMES), dtype=np.float64)
    _load().orc_router_stats(ctypes.byref(L), _p(np.ascontiguousarray(lg, dtype=np.float32)),
                             _p(np.ascontiguousarray(idx, dtype=np.int32)), _p(out))
    d = {"P": out[:L.E].copy()}
    for i, n in enumerate(STAT_NAMES):
        d[n] = float(out[L.E + i])
    return d


def combine(L: OrcLayer, yp, w, dest, shared=None, x=None) -> np.ndarray:
    """a9 alone: y float64 [T, d] from fp32 expert rows yp [R, d]."""
    y = np.empty((L.T, L.d), dtype=np.float64)
    _load().orc_combine(ctypes.byref(L), _p(np.ascontiguousarray(yp, dtype=np.float32)),
                        _p(np.ascontiguousarray(w, dtype=np.float64)), _p(np.ascontiguousarray(dest, dtype=np.int32)),
                        _p(None if shared is None else np.ascontiguousarray(shared, dtype=np.float32)),
                        _p(x), _p(y))
    return y


def expert_choice(L: OrcLayer, lg, cap: int):
    """-> (tok int32 [E, cap], g float64 [E, cap])"""
    tok = np.empty((L.E, cap), dtype=np.int32)
    g = np.empty((L.E, cap), dtype=np.float64)
    _load().orc_expert_choice(ctypes.byref(L), _p(np.ascontiguousarray(lg, dtype=np.float32)), cap, _p(tok), _p(g))
    return tok, g


def ec_capacity(L: OrcLayer) -> int:
    """Tokens each expert takes under expert choice: floor(C * T * K / E) with
    C = capacity_factor (1 when C <= 0), at most T -- the token-choice
    capacity formula [TD §3.2], so both routings process about C*T*K
    (token, expert) pairs."""
    c = L.capacity_factor if L.capacity_factor > 0 else 1.0
    return min(int(np.floor(c * L.T * L.K / L.E)), L.T)


def ec_layer(L: OrcLayer) -> OrcLayer:
    """The layer seen as K = E token choice with a drop mask: assignment
    (t, e) is expert e, kept iff expert e chose token t."""
    return OrcLayer(L.T, L.d, L.F, L.E, L.E, L.gate, 0, L.residual, L.bf16, 0.0, L.n_shared, L.Fs, L.round_h,
                    L.w_fp8)


def route_expert_choice(L: OrcLayer, x=None, Wg=None, logit_bias=None, lg=None):
    """Expert-choice routing [TD §3.3]: S = the logits [T, E]; expert e takes
    the ec_capacity(L) tokens with the largest S[:, e] (ties to the lower
    token).  Returned in the K = E form of ec_layer(L): idx[t][e] = e,
    w[t][e] = g (the token's softmax-over-experts probability of e) where e
    chose t (NaN elsewhere), dest[t*E + e] = e * cap + (rank of t among the
    tokens e chose, ascending t), or -1.  counts[e] = cap; offsets = e * cap."""
    if lg is None:
        lg = logits(L, x, Wg, logit_bias)
    T, E = L.T, L.E
    cap = ec_capacity(L)
    tok, g = expert_choice(L, lg, cap)
    idx = np.tile(np.arange(E, dtype=np.int32), (T, 1))
    w = np.full((T, E), np.nan)
    dest = np.full(T * E, -1, np.int32)
    row_src = np.full(T * E, -1, np.int32)
    for e in range(E):
        order = np.argsort(tok[e], kind="stable")
        for rank, c in enumerate(order):
            t = int(tok[e, c])
            w[t, e] = g[e, c]
            dest[t * E + e] = e * cap + rank
            row_src[e * cap + rank] = t * E + e
    return dict(logits=lg, idx=idx, w=w, dest=dest, row_src=row_src, dropped=(dest < 0).astype(np.uint8),
                counts=np.full(E, cap, np.int32), offsets=(np.arange(E + 1) * cap).astype(np.int32), cap=cap,
                tok=tok, g=g)


POLICIES = ("first_come", "affinity", "reroute")


def route(L: OrcLayer, x, Wg, logit_bias=None, sel_bias=None, policy: str = "first_come", lg=None):
    """a1-a4 in order: logits, selection, permutation under a drop policy.

    first_come: the first K_max arrivals in flat order are kept [TD §3.2];
    affinity:   the K_max highest-affinity assignments are kept, the
                affinity being the fp32 gate weight [TD §5.2];
    reroute:    overflow goes to the next-best expert [LN §3.2]; 'idx' and 'w'
                are then the final assignment, 'idx_first' / 'w_first' the
                Top-K choice.
    lg: fp32 logits to route instead of computing them."""
    if lg is None:
        lg = logits(L, x, Wg, logit_bias)
    idx, w, gap = select(L, lg, sel_bias)
    if policy == "first_come":
        perm = permute(L, idx)
    elif policy == "affinity":
        perm = permute_affinity(L, idx, w.astype(np.float32))
    elif policy == "reroute":
        ai, aw = alternates(L, lg, sel_bias)
        perm = permute_reroute(L, idx, w, ai, aw)
        perm["idx_first"], perm["w_first"] = idx, w
        idx, w = perm.pop("idx"), perm.pop("w")
    else:
        raise ValueError(policy)
    return dict(logits=lg, idx=idx, w=w, gap=gap, **perm)
