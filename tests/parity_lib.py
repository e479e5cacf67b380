"""Helpers for the GPU parity tests: build a workload's inputs once, run the
HIP library on them through the C-ABI binding, run the CPU oracle on the same
inputs, and compare.

Tolerances (one place, used by every parity test):
  fp32 layer:  max_i |y_i - r_i| / max(|r_i|, RMS(r)) <= 1e-4
  bf16 layer:  max_i |y_i - r_i| <= 2e-2 * RMS(r), RMS over the rows of tokens
               that are neither dropped nor excluded as near-ties, measured on
               the layer's fp32 result before its final rounding; the bf16
               output must then equal the round-to-nearest-even image of that
               result bit for bit.  (Rounding the exact result to bf16 alone
               can already cost 2e-2 x RMS when max|y| / RMS exceeds about 5.)
  router logits: |l_gpu - l_ref| <= (3d + 2) * 2^-24 * sum_i |x_i w_i| + 2^-24 |l_ref|
               (the forward-error bound of an fp32 sum of 3d exact products:
               the bf16 path splits each fp32 router weight into three bf16
               parts), and the RMS of (l_gpu - l_ref) / sum_i |x_i w_i| below
               4 * sqrt(3d) * 2^-24, which a dropped or misplaced term breaks
  Top-K weights: |w_gpu - w_ref| <= 1e-5 * |w_ref| + 1e-6
  Integer routing (indices, counts, offsets, dest, row_src, drop mask): exact.
A token whose K-th / (K+1)-th key gap is below 1e-4 is a near-tie: its choice
may legitimately differ between two correct fp32 routers; it is excluded from
the index comparison of the free-running path and counted.
"""
from __future__ import annotations

import numpy as np
import torch

import moe_synth
import oracle
import mixture_experts_sparse_route_amd as moe

NEAR_TIE = 1e-4
F32_TOL = 1e-4
# bf16 layers: max |y - r| <= 2e-2 * RMS(r) is the stated bound; against the
# oracle that stores h in bf16 as the layer does, the remaining differences
# are fp32 accumulation and rare one-ulp differences in h's rounding, so the
# tests hold the tighter 5e-3.
BF16_TOL = 2e-2
BF16_H_TOL = 5e-3


def scales_of(h: dict) -> dict:
    """The FP8 row scales of a generated input set (all None for bf16 / fp32)."""
    return {k: h.get(k) for k in ("S1", "S3", "S2", "Ss1", "Ss3", "Ss2")}


def dev(a: np.ndarray | None):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a bf16 device tensor as uint16."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def spec_of(wl, **kw) -> moe.LayerSpec:
    return moe.LayerSpec(tokens=wl.T, d_model=wl.d, d_ff=wl.F, n_experts=wl.E, top_k=wl.K, gate=wl.gate,
                         renorm=wl.renorm, capacity_factor=wl.capacity_factor, n_shared=wl.n_shared,
                         d_ff_shared=wl.Fs, dtype=wl.dtype, wdtype=wl.wdtype, **kw)


def device_scales(d: dict):
    """The library's scales dict from device input tensors (None without FP8 weights)."""
    if d.get("S1") is None:
        return None
    return dict(w1=d["S1"], w3=d["S3"], w2=d["S2"], ws1=d.get("Ss1"), ws3=d.get("Ss3"), ws2=d.get("Ss2"))


class Case:
    """Inputs of one workload on the host (for the oracle) and the device."""

    def __init__(self, wl):
        self.wl = wl
        self.h = wl.gen_all()
        self.d = {k: dev(v) for k, v in self.h.items()}
        self.L = oracle.layer_of(wl)
        self._route = None

    # ---------------------------------------------------------- GPU side --
    def gpu_forward(self, residual=False, logits_in=None, topk_in=None, out_dtype=None, stats=False,
                    drop_policy="first_come", expert_choice=False):
        """moe_forward through the C-ABI.  logits_in: fp32 [T, E] host array;
        topk_in: (idx int32 [T, K], w fp32 [T, K]) host arrays; out_dtype:
        "f32" or "bf16" (default: the layer's dtype); stats: also write the
        router statistics (Routing.statistics()); drop_policy: a key of
        moe.DROP_POLICIES."""
        wl = self.wl
        spec = spec_of(wl, residual=residual, logits_in=logits_in is not None, topk_in=topk_in is not None,
                       out_dtype=out_dtype, stats=stats, drop_policy=drop_policy, expert_choice=expert_choice)
        r = moe.Routing(spec)
        if logits_in is not None:
            r.logits.copy_(torch.from_numpy(np.ascontiguousarray(logits_in, dtype=np.float32)))
        if topk_in is not None:
            r.topk_idx.copy_(torch.from_numpy(np.ascontiguousarray(topk_in[0], dtype=np.int32)))
            r.topk_w.copy_(torch.from_numpy(np.ascontiguousarray(topk_in[1], dtype=np.float32)))
        ws, _ = moe.alloc_workspace(spec)
        ydt = torch.bfloat16 if (out_dtype or wl.dtype) == "bf16" else torch.float32
        y = torch.empty((wl.T, wl.d), dtype=ydt, device="cuda")
        d = self.d
        moe.moe_forward(spec, d["x"], d["Wg"], d["logit_bias"], d["sel_bias"], d["W1"], d["W3"], d["W2"],
                        d["Ws1"], d["Ws3"], d["Ws2"], y, r, ws, scales=device_scales(d))
        torch.cuda.synchronize()
        return y, r

    # ------------------------------------------------------- oracle side --
    def oracle_route(self):
        if self._route is None:
            h = self.h
            self._route = oracle.route(self.L, h["x"], h["Wg"], h["logit_bias"], h["sel_bias"])
        return self._route

    def oracle_y(self, idx, w, dest, tokens=None, residual=False, round_h=None):
        """round_h=False: h kept in double (no bf16 storage of the SwiGLU output)."""
        h = self.h
        L = oracle.layer_of(self.wl, residual=residual, round_h=round_h)
        return oracle.forward_rows(L, h["x"], idx, w, dest, h["W1"], h["W3"], h["W2"], h["Ws1"], h["Ws3"], h["Ws2"],
                                   tokens=tokens, **scales_of(h))

    def logit_bound(self):
        x = self.h["x"]
        xf = moe_synth.bf16_to_f32(x) if x.dtype == np.uint16 else x
        s = np.abs(xf.astype(np.float64)) @ np.abs(self.h["Wg"].astype(np.float64)).T
        return s


# ------------------------------------------------------------ comparisons --

def routing_host(r: moe.Routing) -> dict:
    return dict(logits=r.logits.cpu().numpy(), idx=r.topk_idx.cpu().numpy(), w=r.topk_w.cpu().numpy(),
                counts=r.counts.cpu().numpy(), offsets=r.offsets.cpu().numpy(), dest=r.dest.cpu().numpy(),
                row_src=r.row_src.cpu().numpy(), dropped=r.dropped.cpu().numpy())


def assert_permutation_equal(g: dict, o: dict, label=""):
    assert np.array_equal(g["counts"], o["counts"]), f"{label}: counts differ"
    assert np.array_equal(g["offsets"], o["offsets"]), f"{label}: offsets differ"
    assert np.array_equal(g["dest"], o["dest"]), f"{label}: dest differs"
    assert np.array_equal(g["dropped"], o["dropped"]), f"{label}: drop mask differs"
    R = int(o["offsets"][-1])
    assert np.array_equal(g["row_src"][:R], o["row_src"][:R]), f"{label}: row_src differs"


def assert_weights_close(wg: np.ndarray, wo: np.ndarray, label=""):
    err = np.abs(wg.astype(np.float64) - wo)
    bound = 1e-5 * np.abs(wo) + 1e-6
    assert np.all(err <= bound), f"{label}: top-k weight error {err.max():.3g}"


def y_error(y_gpu: np.ndarray, y_ref: np.ndarray, dtype: str, rows=None):
    """-> (error measure, limit) on the given rows."""
    if rows is not None:
        y_gpu, y_ref = y_gpu[rows], y_ref[rows]
    if y_ref.size == 0:
        return 0.0, 1.0
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    if dtype == "f32":
        den = np.maximum(np.abs(y_ref), rms)
        return float(np.max(np.abs(y_gpu - y_ref) / den)), F32_TOL
    return float(np.max(np.abs(y_gpu - y_ref))) / rms, min(BF16_TOL, BF16_H_TOL)


def assert_y_close(y_gpu: np.ndarray, y_ref: np.ndarray, dtype: str, rows=None, label=""):
    err, lim = y_error(y_gpu, y_ref, dtype, rows)
    assert err <= lim, f"{label}: output error {err:.4g} > {lim}"
    return err


def kept_tokens(dest: np.ndarray, K: int, n_shared: int) -> np.ndarray:
    """Tokens with at least one kept assignment (or a shared expert)."""
    T = dest.size // K
    if n_shared:
        return np.ones(T, bool)
    return (dest.reshape(T, K) >= 0).any(1)
