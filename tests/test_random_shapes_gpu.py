"""GPU parity over seeded random layer shapes: token counts, widths, expert
counts, K, gate, renormalisation, capacity, shared expert and residual drawn
from a fixed generator, each case checked against the oracle by the checker
of its path (every output compared):
  token choice   the free, logits_in and topk_in paths;
  E4M3 weights   logits_in, fp32 and bf16 outputs;
  drop policies  affinity-ordered drops and re-routing under capacity;
  expert choice  logits_in and free-running.
The shapes are small enough for the oracle to finish in seconds and cover
ragged tails of every tiling (tokens per router chunk, m-tiles, weight tiles).
"""
import numpy as np
import pytest

from moe_synth import workload
from moe_synth.configs import GATE_SIGMOID, GATE_SOFTMAX
from test_parity_gpu import _gpu, check_case  # noqa: F401  (module fixture)
from test_drop_policy_gpu import check_policy
from test_expert_choice_gpu import check_ec
from test_fp8_gpu import check_fp8
from parity_lib import Case

pytestmark = pytest.mark.gpu


def _dims(r, f32):
    E = int(r.integers(1, 81))
    K = int(r.integers(1, min(E, 8) + 1))
    T = int(r.integers(1, 700))
    if f32:
        d, F = int(r.integers(16, 200)), int(r.integers(16, 200))
    else:  # bf16 layers take widths in multiples of 64
        d, F = 64 * int(r.integers(1, 6)), 64 * int(r.integers(1, 7))
    return T, d, F, E, K


def _layer(r, i, f32, seed0, **fixed):
    T, d, F, E, K = _dims(r, f32)
    gate = GATE_SIGMOID if r.random() < 0.4 else GATE_SOFTMAX
    shared = int(r.random() < 0.3)
    Fs = (64 * int(r.integers(1, 4)) if not f32 else int(r.integers(16, 130))) if shared else 0
    kw = dict(T=T, d=d, F=F, E=E, K=K, gate=gate, renorm=bool(r.random() < 0.6),
              capacity_factor=float(r.choice([0.0, 0.0, 0.6, 1.0, 1.25, 2.0])), n_shared=shared, Fs=Fs,
              sel_bias="u0.1" if gate == GATE_SIGMOID and r.random() < 0.5 else None,
              logit_bias="zipf1.1x2" if r.random() < 0.3 else None, seed=seed0 + i)
    kw.update(fixed)
    return workload("tiny_top2_fp32" if f32 else "mixtral_prefill", **kw)


def _id(i, wl, extra=""):
    return (f"{i}-{wl.dtype}{'-fp8' if wl.wdtype else ''}-T{wl.T}-d{wl.d}-F{wl.F}-E{wl.E}-K{wl.K}"
            f"-{'sig' if wl.gate == GATE_SIGMOID else 'soft'}-c{wl.capacity_factor}-s{wl.n_shared}{extra}")


def _token_choice(n, seed=2024):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        wl = _layer(r, i, i % 5 == 4, 100)
        residual = bool(r.random() < 0.3)
        out.append(pytest.param(wl, residual, id=_id(i, wl, "-res" if residual else "")))
    return out


def _fp8(n, seed=2025):
    r = np.random.default_rng(seed)
    return [pytest.param(wl, id=_id(i, wl)) for i, wl in
            ((i, _layer(r, i, False, 200, wdtype="fp8")) for i in range(n))]


def _policies(n, seed=2026):
    # capacity below one slot per assignment, so that drops happen
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        wl = _layer(r, i, i % 4 == 3, 300, capacity_factor=float(r.choice([0.5, 0.7, 0.9])))
        wl = wl.with_(T=max(wl.T, 64))
        out.append(pytest.param(wl, "affinity" if i % 2 == 0 else "reroute", id=_id(i, wl)))
    return out


def _expert_choice(n, seed=2027):
    # expert choice: softmax gate, raw weights, capacity factor > 0
    r = np.random.default_rng(seed)
    return [pytest.param(wl, id=_id(i, wl)) for i, wl in
            ((i, _layer(r, i, i % 4 == 3, 400, gate=GATE_SOFTMAX, renorm=False, sel_bias=None,
                        capacity_factor=float(r.choice([0.5, 1.0, 1.5, 3.0])))) for i in range(n))]


@pytest.mark.parametrize("wl,residual", _token_choice(24))
def test_random_shape(wl, residual):
    print(wl, check_case(Case(wl), residual=residual))


@pytest.mark.parametrize("wl", _fp8(8))
def test_random_shape_fp8(wl):
    print(wl, check_fp8(Case(wl)))


@pytest.mark.parametrize("wl,policy", _policies(8))
def test_random_shape_drop_policy(wl, policy):
    print(wl, policy, check_policy(Case(wl), policy))


@pytest.mark.parametrize("wl", _expert_choice(8))
def test_random_shape_expert_choice(wl):
    print(wl, check_ec(Case(wl)))
