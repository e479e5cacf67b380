"""The five synthetic MoE-layer workloads and how their inputs are drawn.

Each workload is named for what it is.  Shapes, gate type, Top-K, capacity
factor and the input distributions are the workload's definition; none of the
layer's arithmetic lives here (the capacity *factor* is stored, never the
per-expert capacity derived from it).

Input recipe (every workload, seed 0 unless a caller says otherwise):
  x            ~ N(0, 1)                       tensor id 0
  W_g [E, d]   ~ N(0, 1/d), fp32               tensor id 1
  W1, W3 [E, F, d] ~ N(0, 1/d)                 tensor ids 2, 3
  W2 [E, d, F] ~ N(0, 1/F)                     tensor id 4
  shared Ws1, Ws3 [S, Fs, d] ~ N(0, 1/d); Ws2 [S, d, Fs] ~ N(0, 1/Fs)   ids 5, 6, 7
  selection bias [E] ~ U(-0.1, 0.1), fp32      tensor id 8
  logit bias [E] (Switch workload only): 2.0 * (e + 1)^-1.1, a Zipf(s = 1.1)
      profile over expert rank scaled so the first expert gets 2.0.
FP8 expert weights (wdtype "fp8"; activations stay bf16): E4M3 codes from
  random bits (moe_synth.fp8_codes, same tensor ids as the bf16 weights; the
  decoded codes have standard deviation about 3.6) and per-row fp32 scales
  ~ U(0.5, 1.5) / (4 sqrt(fan-in)) (W1, W3 rows: d; W2 rows: F), tensor ids
  9 .. 14.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

GATE_SOFTMAX = 0
GATE_SIGMOID = 1


@dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens
    d: int            # d_model
    F: int            # expert d_ff
    E: int            # routed experts
    K: int            # top-k
    gate: int         # GATE_SOFTMAX / GATE_SIGMOID
    renorm: bool      # renormalise the K selected weights to sum to 1
    capacity_factor: float = 0.0   # <= 0: no capacity limit
    n_shared: int = 0
    Fs: int = 0       # shared-expert d_ff
    dtype: str = "bf16"            # activations and expert weights: "f32" or "bf16"
    wdtype: str = ""               # "fp8": expert weights are E4M3 codes with per-row scales
    logit_bias: Optional[str] = None   # None or "zipf1.1x2"
    sel_bias: Optional[str] = None     # None or "u0.1"
    seed: int = 0
    note: str = ""

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    # ---- input generation -------------------------------------------------
    def gen_x(self, t0: int = 0, nt: Optional[int] = None) -> np.ndarray:
        from . import TID_X, normal
        nt = self.T - t0 if nt is None else nt
        return normal(self.seed, TID_X, (nt, self.d), 1.0, self.dtype, offset=t0 * self.d)

    def gen_wg(self) -> np.ndarray:
        from . import TID_WG, normal
        return normal(self.seed, TID_WG, (self.E, self.d), 1.0 / np.sqrt(self.d), "f32")

    def gen_logit_bias(self) -> Optional[np.ndarray]:
        if self.logit_bias is None:
            return None
        if self.logit_bias == "zipf1.1x2":
            e = np.arange(self.E, dtype=np.float64)
            return (2.0 * (e + 1.0) ** -1.1).astype(np.float32)
        raise ValueError(self.logit_bias)

    def gen_sel_bias(self) -> Optional[np.ndarray]:
        from . import TID_SEL_BIAS, uniform
        if self.sel_bias is None:
            return None
        if self.sel_bias == "u0.1":
            return uniform(self.seed, TID_SEL_BIAS, (self.E,), -0.1, 0.1)
        raise ValueError(self.sel_bias)

    def gen_expert(self, e0: int = 0, ne: Optional[int] = None):
        """W1, W3 [ne, F, d] and W2 [ne, d, F] for experts e0 .. e0+ne-1."""
        from . import TID_W1, TID_W2, TID_W3, fp8_codes, normal
        ne = self.E - e0 if ne is None else ne
        fd = self.F * self.d
        if self.wdtype == "fp8":
            return (fp8_codes(self.seed, TID_W1, (ne, self.F, self.d), offset=e0 * fd),
                    fp8_codes(self.seed, TID_W3, (ne, self.F, self.d), offset=e0 * fd),
                    fp8_codes(self.seed, TID_W2, (ne, self.d, self.F), offset=e0 * fd))
        w1 = normal(self.seed, TID_W1, (ne, self.F, self.d), 1.0 / np.sqrt(self.d), self.dtype, offset=e0 * fd)
        w3 = normal(self.seed, TID_W3, (ne, self.F, self.d), 1.0 / np.sqrt(self.d), self.dtype, offset=e0 * fd)
        w2 = normal(self.seed, TID_W2, (ne, self.d, self.F), 1.0 / np.sqrt(self.F), self.dtype, offset=e0 * fd)
        return w1, w3, w2

    def gen_scales(self):
        """Per-row scales of FP8 weights: S1, S3 [E, F], S2 [E, d], Ss1, Ss3
        [S, Fs], Ss2 [S, d] (None when the weights are not FP8)."""
        from . import TID_S1, TID_S2, TID_S3, TID_SS1, TID_SS2, TID_SS3, uniform
        if self.wdtype != "fp8":
            return dict(S1=None, S3=None, S2=None, Ss1=None, Ss3=None, Ss2=None)
        E, F, d, S, Fs = self.E, self.F, self.d, self.n_shared, self.Fs
        rd, rf = 0.25 / np.sqrt(d), 0.25 / np.sqrt(F)   # codes have std about 3.6
        out = dict(S1=uniform(self.seed, TID_S1, (E, F), 0.5 * rd, 1.5 * rd),
                   S3=uniform(self.seed, TID_S3, (E, F), 0.5 * rd, 1.5 * rd),
                   S2=uniform(self.seed, TID_S2, (E, d), 0.5 * rf, 1.5 * rf),
                   Ss1=None, Ss3=None, Ss2=None)
        if S:
            rs = 0.25 / np.sqrt(Fs)
            out.update(Ss1=uniform(self.seed, TID_SS1, (S, Fs), 0.5 * rd, 1.5 * rd),
                       Ss3=uniform(self.seed, TID_SS3, (S, Fs), 0.5 * rd, 1.5 * rd),
                       Ss2=uniform(self.seed, TID_SS2, (S, d), 0.5 * rs, 1.5 * rs))
        return out

    def gen_shared(self):
        from . import TID_WS1, TID_WS2, TID_WS3, fp8_codes, normal
        if self.n_shared == 0:
            return None, None, None
        s, fs, d = self.n_shared, self.Fs, self.d
        if self.wdtype == "fp8":
            return (fp8_codes(self.seed, TID_WS1, (s, fs, d)), fp8_codes(self.seed, TID_WS3, (s, fs, d)),
                    fp8_codes(self.seed, TID_WS2, (s, d, fs)))
        ws1 = normal(self.seed, TID_WS1, (s, fs, d), 1.0 / np.sqrt(d), self.dtype)
        ws3 = normal(self.seed, TID_WS3, (s, fs, d), 1.0 / np.sqrt(d), self.dtype)
        ws2 = normal(self.seed, TID_WS2, (s, d, fs), 1.0 / np.sqrt(fs), self.dtype)
        return ws1, ws3, ws2

    def gen_all(self) -> dict:
        w1, w3, w2 = self.gen_expert()
        ws1, ws3, ws2 = self.gen_shared()
        return dict(x=self.gen_x(), Wg=self.gen_wg(), logit_bias=self.gen_logit_bias(),
                    sel_bias=self.gen_sel_bias(), W1=w1, W3=w3, W2=w2, Ws1=ws1, Ws3=ws3, Ws2=ws2,
                    **self.gen_scales())


WORKLOADS = {
    "tiny_top2_fp32": Workload(
        name="tiny_top2_fp32", T=64, d=128, F=256, E=8, K=2, gate=GATE_SOFTMAX, renorm=True,
        dtype="f32", note="tiny top-2 softmax MoE, fp32 throughout"),
    "switch_top1_capacity": Workload(
        name="switch_top1_capacity", T=8192, d=1024, F=4096, E=64, K=1, gate=GATE_SOFTMAX,
        renorm=False, capacity_factor=1.25, dtype="bf16", logit_bias="zipf1.1x2",
        note="Switch-style top-1, capacity factor 1.25, Zipf-skewed logit bias, bf16"),
    "mixtral_prefill": Workload(
        name="mixtral_prefill", T=4096, d=4096, F=14336, E=8, K=2, gate=GATE_SOFTMAX, renorm=True,
        dtype="bf16", note="Mixtral-shaped prefill, top-2 of 8, bf16"),
    "mixtral_decode": Workload(
        name="mixtral_decode", T=32, d=4096, F=14336, E=8, K=2, gate=GATE_SOFTMAX, renorm=True,
        dtype="bf16", note="Mixtral-shaped decode step, 32 tokens, bf16"),
    "deepseek_v3_fine": Workload(
        name="deepseek_v3_fine", T=4096, d=7168, F=2048, E=256, K=8, gate=GATE_SIGMOID, renorm=True,
        n_shared=1, Fs=2048, dtype="bf16", sel_bias="u0.1",
        note="fine-grained 256 experts, sigmoid top-8 with selection bias, 1 shared expert, bf16"),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.with_(**overrides) if overrides else w
