"""GPU parity of expert-choice routing (Tech Daily 2026-04-14, §3.3) against
the oracle.

Each expert takes the cap = floor(C*T*K/E) tokens with the largest logit in
its column; the library writes the routing in the K = E form (entry (t, e)
kept iff e took t).  With identical fp32 logits (logits_in) the choice is
made on identical values, so dest / row_src / drop mask / counts / offsets
must be bit-exact.  Free-running, an expert whose cap-th and next logits lie
within 1e-4 may legitimately take a different token; its column is excluded
and counted.  Outputs are held to the layer's tolerance.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
import mixture_experts_sparse_route_amd as moe
from moe_synth import workload
from parity_lib import (NEAR_TIE, Case, assert_permutation_equal, assert_y_close, host_f64, oracle_refs,
                        routing_host, tile_sample_tokens)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    moe.load_library()
    moe_synth.build(force=False)
    oracle.build(force=False)


CASES = {
    "switch_small": workload("switch_top1_capacity", T=1000, d=256, F=128, E=16),
    "mixtral_small": workload("mixtral_prefill", T=300, d=256, F=128, renorm=False, capacity_factor=1.0),
    "mixtral_shared_residual": workload("mixtral_prefill", T=200, d=128, F=64, renorm=False, n_shared=1, Fs=64),
    "fp32_tiny": workload("tiny_top2_fp32", T=64, d=40, F=24, E=6, renorm=False, capacity_factor=1.5),
    "capacity_all_tokens": workload("tiny_top2_fp32", T=20, d=16, F=8, E=4, K=2, renorm=False, capacity_factor=4.0),
}


def ec_oracle(case: Case, lg):
    L = case.L
    return oracle.route_expert_choice(L, lg=lg), oracle.ec_layer(L)


def near_tie_experts(lg, cap):
    amb = []
    for e in range(lg.shape[1]):
        v = np.sort(lg[:, e].astype(np.float64))[::-1]
        if 0 < cap < len(v) and v[cap - 1] - v[cap] < NEAR_TIE:
            amb.append(e)
    return amb


def check_ec(case: Case, residual=False, tokens=None, strict=False):
    wl = case.wl
    T, E = wl.T, wl.E
    lg = case.oracle_route()["logits"]
    orc, Lec = ec_oracle(case, lg)
    chosen = orc["dest"] >= 0
    rows = np.arange(T) if tokens is None else tokens
    h = case.h
    L_res = oracle.ec_layer(oracle.layer_of(wl, residual=residual))
    y_ref = oracle_refs(L_res, h, orc["idx"], np.nan_to_num(orc["w"]), orc["dest"], tokens=rows)
    live = np.ones(len(rows), bool) if (wl.n_shared or residual) else chosen.reshape(T, E)[rows].any(1)
    report = {"cap": orc["cap"], "unchosen_tokens": int((~chosen.reshape(T, E).any(1)).sum())}
    # identical logits
    y, r = case.gpu_forward(residual=residual, logits_in=lg, out_dtype="f32", expert_choice=True)
    g = routing_host(r)
    assert_permutation_equal(g, orc, "ec logits_in")
    assert np.array_equal(g["idx"], orc["idx"])
    wo = orc["w"].reshape(-1)[chosen]
    assert np.all(np.abs(g["w"].reshape(-1)[chosen] - wo) <= 1e-5 * wo + 1e-7), "gate weights"
    report["err_logits_in"] = assert_y_close(host_f64(y)[rows], y_ref, rows=live, label="ec", strict=strict)
    # free-running
    y2, r2 = case.gpu_forward(residual=residual, out_dtype="f32", expert_choice=True)
    g2 = routing_host(r2)
    amb = near_tie_experts(lg, orc["cap"])
    ok = ~np.isin(np.tile(np.arange(E), T), amb)
    assert np.array_equal(g2["dest"][ok], orc["dest"][ok]), "free-running expert choice differs"
    report["near_tie_experts"] = len(amb)
    if not amb:
        report["err_free"] = assert_y_close(host_f64(y2)[rows], y_ref, rows=live, label="ec free", strict=strict)
    return report


@pytest.mark.parametrize("name", list(CASES))
def test_ec_small(name):
    print(name, check_ec(Case(CASES[name])))


def test_ec_residual():
    print(check_ec(Case(CASES["switch_small"]), residual=True))


def test_ec_entry_points_and_max_rows():
    """moe_max_rows is E * cap, and each expert holds exactly cap rows."""
    wl = CASES["mixtral_small"]
    spec = moe.LayerSpec(tokens=wl.T, d_model=wl.d, d_ff=wl.F, n_experts=wl.E, top_k=wl.K, renorm=False,
                         capacity_factor=wl.capacity_factor, dtype=wl.dtype, expert_choice=True)
    cap = int(np.floor(wl.capacity_factor * wl.T * wl.K / wl.E))
    assert moe.max_rows(spec) == wl.E * cap
    case = Case(wl)
    _, r = case.gpu_forward(out_dtype="f32", expert_choice=True)
    g = routing_host(r)
    assert np.array_equal(np.bincount(g["idx"].reshape(-1)[g["dest"] >= 0], minlength=wl.E), np.full(wl.E, cap))


@pytest.mark.timeout(900)
def test_ec_full_size_switch():
    """The Switch workload (T=8192, d=1024, F=4096, E=64, C=1.25): routing of
    all tokens, outputs on a sample of tokens."""
    case = Case(workload("switch_top1_capacity"))
    # tokens covering every (expert, m-tile) of both GEMMs: the chosen tokens
    # of each expert at multiples of 32 within its group, and its last one
    orc, _ = ec_oracle(case, case.oracle_route()["logits"])
    toks = tile_sample_tokens(orc, case.wl.E, case.wl.T)
    print(check_ec(case, tokens=toks))
