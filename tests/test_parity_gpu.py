"""GPU parity: the HIP library (through the C-ABI) against the CPU oracle on
the same seeded inputs.

Three paths per case, each checked end to end:
  free      the library computes its own logits; logits within the fp32
            forward-error bound, indices equal except near-ties (counted),
            weights, permutation and outputs checked when no choice flipped;
  logits_in both sides route the oracle's fp32 logits: indices, counts,
            offsets, dest, row_src and drop mask bit-exact, outputs within
            tolerance;
  topk_in   both sides use the oracle's Top-K choice: permutation bit-exact,
            outputs within tolerance.
Small cases (several tiles and a ragged tail) compare every output; the five
full-size workloads compare routing over all tokens and outputs on a sample of
tokens the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
import mixture_experts_sparse_route_amd as moe
from moe_synth import workload
from parity_lib import (NEAR_TIE, Case, assert_permutation_equal, assert_weights_close, assert_y_close, dev,
                        device_scales, host_f64, kept_tokens, routing_host, spec_of, tile_sample_tokens)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    moe.load_library()
    moe_synth.build(force=False)
    oracle.build(force=False)


def sample_tokens(case: Case):
    """Tokens covering every (expert, m-tile) of both GEMMs, plus the first
    and last few dropped tokens of a capacity layer."""
    T = case.wl.T
    orc = case.oracle_route()
    extra = []
    if case.wl.capacity_factor > 0:
        dropped = np.nonzero(orc["dropped"].reshape(T, -1).all(1))[0]
        extra = list(dropped[:4]) + list(dropped[-4:])
    return tile_sample_tokens(orc, case.wl.K, T, extra)


def check_case(case: Case, tokens=None, residual=False, strict=False):
    """strict: the stated bound against the definition with no h-storage
    allowance (the full-size workloads)."""
    wl = case.wl
    T, K = wl.T, wl.K
    orc = case.oracle_route()
    rows = np.arange(T) if tokens is None else tokens
    y_ref = case.oracle_y(orc["idx"], orc["w"], orc["dest"], tokens=rows, residual=residual)
    live = kept_tokens(orc["dest"], K, wl.n_shared)[rows]
    dead = ~live
    report = {"tokens_checked": int(len(rows))}

    # ---- free-running path (fp32 output; for a bf16 layer the bf16 output is
    # checked to be exactly its round-to-nearest-even image)
    y, r = case.gpu_forward(residual=residual, out_dtype="f32")
    g = routing_host(r)
    if wl.dtype == "bf16":
        yb, _ = case.gpu_forward(residual=residual, out_dtype="bf16")
        assert torch.equal(yb.view(torch.int16), y.to(torch.bfloat16).view(torch.int16)), \
            "bf16 output is not the rounded fp32 output"
    sxw = case.logit_bound()
    bound = (3 * wl.d + 2) * 2.0 ** -24 * sxw + 2.0 ** -24 * np.abs(orc["logits"])
    if case.h["logit_bias"] is not None:
        bound += 2.0 ** -24 * np.abs(case.h["logit_bias"])[None, :]
    lerr = np.abs(g["logits"].astype(np.float64) - orc["logits"])
    assert np.all(lerr <= bound), f"logits outside the forward-error bound: {np.max(lerr / bound):.3g}x"
    rel_rms = float(np.sqrt(np.mean((lerr / sxw) ** 2)))
    assert rel_rms <= 4 * np.sqrt(3 * wl.d) * 2.0 ** -24, f"logit error RMS {rel_rms:.3g} is not rounding noise"
    report["logit_rel_rms"] = rel_rms
    near = orc["gap"] < NEAR_TIE
    flip = (g["idx"] != orc["idx"]).any(1)
    assert not np.any(flip & ~near), f"{int(np.sum(flip & ~near))} tokens changed experts without a near-tie"
    report["near_ties"] = int(near.sum())
    report["flips"] = int(flip.sum())
    if not flip.any():
        assert_weights_close(g["w"], orc["w"], "free")
        assert_permutation_equal(g, orc, "free")
        yg = host_f64(y)[rows]
        report["err_free"] = assert_y_close(yg, y_ref, rows=live, label="free", strict=strict)
        if dead.any():
            xf = case.h["x"] if wl.dtype == "f32" else moe_synth.bf16_to_f32(case.h["x"])
            want = xf.astype(np.float64)[rows][dead] if residual else 0.0
            assert np.array_equal(yg[dead], np.broadcast_to(want, yg[dead].shape)), "dropped rows are not pass-through"

    # ---- logits_in: identical fp32 logits on both sides
    y2, r2 = case.gpu_forward(residual=residual, logits_in=orc["logits"], out_dtype="f32")
    g2 = routing_host(r2)
    assert np.array_equal(g2["idx"], orc["idx"]), \
        f"indices differ given identical logits on {int((g2['idx'] != orc['idx']).any(1).sum())} tokens"
    assert_weights_close(g2["w"], orc["w"], "logits_in")
    assert_permutation_equal(g2, orc, "logits_in")
    yg2 = host_f64(y2)[rows]
    report["err_logits_in"] = assert_y_close(yg2, y_ref, rows=live, label="logits_in", strict=strict)

    # ---- topk_in: identical Top-K choice on both sides
    y3, r3 = case.gpu_forward(residual=residual, topk_in=(orc["idx"], orc["w"].astype(np.float32)),
                              out_dtype="f32")
    g3 = routing_host(r3)
    assert_permutation_equal(g3, orc, "topk_in")
    report["err_topk_in"] = assert_y_close(host_f64(y3)[rows], y_ref, rows=live, label="topk_in", strict=strict)
    return report


# ------------------------------------------------------------ small cases --

SMALL = {
    "tiny_top2_fp32": workload("tiny_top2_fp32"),
    "switch_capacity_small": workload("switch_top1_capacity", T=1000, d=256, F=512, E=16),
    "mixtral_small": workload("mixtral_prefill", T=300, d=512, F=1024),
    "mixtral_two_mtiles": workload("mixtral_prefill", T=1100, d=256, F=384),
    "deepseek_small": workload("deepseek_v3_fine", T=200, d=512, F=256, E=64, Fs=256),
    "decode_small": workload("mixtral_decode", T=5, d=512, F=1024),
    "dense_k_equals_e": workload("mixtral_prefill", T=100, d=128, F=128, E=4, K=4, renorm=False),
    "fp32_ragged": workload("tiny_top2_fp32", T=50, d=100, F=37, E=5),
    "single_expert": workload("mixtral_prefill", T=77, d=128, F=128, E=1, K=1),
    "sigmoid_unnormalised": workload("deepseek_v3_fine", T=64, d=256, F=128, E=32, K=4, renorm=False, n_shared=0,
                                     Fs=0),
    # reductions of 2 k-steps (d = F = 64): the shallowest weight rings
    "short_reduction_decode": workload("mixtral_decode", T=6, d=64, F=64),
    "short_reduction_prefill": workload("mixtral_prefill", T=700, d=64, F=128),
    # expert capacity floor(1.25 * 2048 / 16) = 160: the down GEMM takes
    # 192-row m-tiles, each expert one part-filled tile
    "switch_capacity_160": workload("switch_top1_capacity", T=2048, d=256, F=512, E=16),
    # about 550 rows per expert: 192-row down m-tiles with a ragged last one
    "mixtral_550_rows_per_expert": workload("mixtral_prefill", T=2200, d=256, F=384),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_case(name):
    rep = check_case(Case(SMALL[name]))
    print(name, rep)


# GEMM1's m-tiles split evenly in 32-row units (the plan does so when groups
# average 512 rows or more); forced here on groups that the even split cuts
# differently from full tiles plus a remainder (275 rows: 160 + 115 instead of
# 192 + 83; 160 rows: 96 + 64 instead of 128 + 32)
@pytest.mark.parametrize("name", ["mixtral_two_mtiles", "switch_capacity_160", "deepseek_small"])
def test_even_m_tiles(name, monkeypatch):
    monkeypatch.setenv("MOE_TUNING", "1")
    monkeypatch.setenv("MOE_GEMM_EVEN_UP", "1")
    print(name, check_case(Case(SMALL[name])))


def test_residual_pass_through_with_capacity():
    rep = check_case(Case(SMALL["switch_capacity_small"]), residual=True)
    print(rep)


def test_everything_dropped():
    # floor(1.0 * 10 / 64) = 0: every assignment overflows
    wl = workload("switch_top1_capacity", T=10, d=128, F=128, E=64, capacity_factor=1.0)
    case = Case(wl)
    y, r = case.gpu_forward()
    assert torch.all(y == 0)
    assert int(r.offsets[-1]) == 0 and torch.all(r.dropped == 1) and torch.all(r.dest == -1)
    y2, _ = case.gpu_forward(residual=True)
    assert torch.equal(y2.view(torch.int16), case.d["x"].view(torch.int16))


# Exact ties: logits on a coarse grid (a handful of values, +0.0 and -0.0
# among them) given to both sides; equal keys go to the lower expert and -0.0
# equals +0.0, so indices, weights, counts, offsets, dest and the outputs are
# fixed exactly (no near-tie exclusions).
@pytest.mark.parametrize("name,wl", [
    ("softmax_top2", workload("mixtral_prefill", T=300, d=128, F=64)),
    ("switch_capacity", workload("switch_top1_capacity", T=500, d=128, F=64, E=16, logit_bias=None)),
    ("sigmoid_top8", workload("deepseek_v3_fine", T=200, d=128, F=64, E=64, Fs=64, sel_bias=None)),
])
def test_exact_ties(name, wl):
    case = Case(wl)
    r = np.random.default_rng(7)
    lg = (r.integers(-2, 3, size=(wl.T, wl.E)) * 0.5).astype(np.float32)
    lg[lg == 0] = np.where(r.random(int((lg == 0).sum())) < 0.5, np.float32(-0.0), np.float32(0.0))
    assert np.signbit(lg[lg == 0]).any() and (~np.signbit(lg[lg == 0])).any()
    orc = oracle.route(case.L, None, None, sel_bias=case.h["sel_bias"], lg=lg)
    y, rr = case.gpu_forward(logits_in=lg, out_dtype="f32")
    g = routing_host(rr)
    assert np.array_equal(g["idx"], orc["idx"]), "tied keys resolved differently"
    assert_weights_close(g["w"], orc["w"], name)
    assert_permutation_equal(g, orc, name)
    live = kept_tokens(orc["dest"], wl.K, wl.n_shared)
    y_ref = case.oracle_y(orc["idx"], orc["w"], orc["dest"])
    print(name, assert_y_close(host_f64(y), y_ref, rows=live, label=name))


# Logits far outside exp's fp32 range (|l| up to 3000): the softmax weights
# must come from max-shifted exponentials on both sides (no inf / NaN).
@pytest.mark.parametrize("name,wl", [
    ("softmax_top2_renorm", workload("mixtral_prefill", T=300, d=128, F=64)),
    ("switch_raw", workload("switch_top1_capacity", T=500, d=128, F=64, E=16, logit_bias=None)),
])
def test_extreme_logits(name, wl):
    case = Case(wl)
    r = np.random.default_rng(11)
    lg = r.uniform(-3000.0, 3000.0, size=(wl.T, wl.E)).astype(np.float32)
    lg[::7] *= np.float32(1e-3)  # some tokens with ordinary logits
    orc = oracle.route(case.L, None, None, sel_bias=case.h["sel_bias"], lg=lg)
    y, rr = case.gpu_forward(logits_in=lg, out_dtype="f32")
    g = routing_host(rr)
    assert np.all(np.isfinite(g["w"])) and np.all(np.isfinite(host_f64(y)))
    assert np.array_equal(g["idx"], orc["idx"])
    assert_weights_close(g["w"], orc["w"], name)
    assert_permutation_equal(g, orc, name)
    live = kept_tokens(orc["dest"], wl.K, wl.n_shared)
    y_ref = case.oracle_y(orc["idx"], orc["w"], orc["dest"])
    print(name, assert_y_close(host_f64(y), y_ref, rows=live, label=name))


# Tile plans (shapes, stage widths, persistent grids, even m-tiles) leave
# every output bit unchanged: each output sums its k-steps in k order.
PLAN_OVERRIDES = {
    "even_m_tiles": {"MOE_GEMM_EVEN_UP": "1"},
    "k32_128x256": {"MOE_GEMM_K64": "0", "MOE_GEMM_BM": "128", "MOE_GEMM_BNB_UP": "256", "MOE_GEMM_NS_UP": "3"},
    "persistent": {"MOE_GEMM_WGS": "1"},
    "xcd_ranges": {"MOE_GEMM_XCD_CHUNK": "0"},
    "xcd_chunks_of_1": {"MOE_GEMM_XCD_CHUNK": "1"},
    "xcd_chunks_of_3": {"MOE_GEMM_XCD_CHUNK_UP": "3", "MOE_GEMM_XCD_CHUNK_DOWN": "5"},
    # cache policy only: non-temporal weight loads everywhere, or for whole-group tiles
    "nt_everywhere": {"MOE_GEMM_NT_UP": "1", "MOE_GEMM_NT_DOWN": "1"},
    "nt_whole_groups": {"MOE_GEMM_NT_ROWS_UP": "100000", "MOE_GEMM_NT_ROWS_DOWN": "100000"},
}


@pytest.mark.parametrize("over", list(PLAN_OVERRIDES))
def test_plan_overrides_bitwise_identical(over, monkeypatch):
    case = Case(SMALL["mixtral_two_mtiles"])
    y0, _ = case.gpu_forward(out_dtype="f32")
    for k, v in PLAN_OVERRIDES[over].items():
        monkeypatch.setenv(k, v)
    monkeypatch.setenv("MOE_TUNING", "1")
    y1, _ = case.gpu_forward(out_dtype="f32")
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32)), f"plan override {over} changed the output"


# Decode-sized groups (at most 32 rows per expert) take the weight-streaming
# GEMM2 (and, forced with MOE_GEMM_STREAM=1, GEMM1); they must give the tile
# kernels' outputs (MOE_GEMM_STREAM=0) bit for bit: same MFMAs, fragments
# and k order.
STREAM_CASES = {
    "decode_small": workload("mixtral_decode", T=5, d=512, F=1024),
    "two_row_blocks": workload("mixtral_decode", T=30, d=256, F=384, E=2, K=2),   # groups of 30 rows
    "shared_expert": workload("deepseek_v3_fine", T=24, d=256, F=128, E=16, K=4, Fs=192),
    "short_reduction": workload("mixtral_decode", T=6, d=64, F=64),
}


@pytest.mark.parametrize("name", list(STREAM_CASES))
def test_stream_plan_bitwise_identical(name, monkeypatch):
    case = Case(STREAM_CASES[name])
    y_default, _ = case.gpu_forward(out_dtype="f32")
    monkeypatch.setenv("MOE_TUNING", "1")
    for both in ("1", "0"):
        monkeypatch.setenv("MOE_GEMM_STREAM", both)
        y, _ = case.gpu_forward(out_dtype="f32")
        assert torch.equal(y_default.view(torch.int32), y.view(torch.int32)), f"MOE_GEMM_STREAM={both} differs"
    monkeypatch.delenv("MOE_GEMM_STREAM")
    print(name, check_case(case))


def test_stream_group_over_32_rows(monkeypatch):
    """moe_expert_ffn with a caller's group of 40 rows under a decode-sized
    config (the plan streams): the kernel walks the rows in chunks of 32; the
    output equals the tile kernels' bit for bit."""
    wl = workload("mixtral_decode", T=32, d=256, F=256, E=4, K=2)
    case = Case(wl)
    spec = spec_of(wl)
    mr = moe.max_rows(spec)
    rows = 40
    xp = case.d["x"].repeat(2, 1)[:mr].contiguous()
    offs = torch.tensor([0, rows], dtype=torch.int32, device="cuda")
    out = []
    for stream in ("1", "0"):
        monkeypatch.setenv("MOE_TUNING", "1")
        monkeypatch.setenv("MOE_GEMM_STREAM", stream)
        ws, _ = moe.alloc_workspace(spec)
        yp = torch.full((mr, wl.d), float("nan"), dtype=torch.float32, device="cuda")
        moe.moe_expert_ffn(spec, xp, offs, 1, rows, case.d["W1"], case.d["W3"], case.d["W2"], yp, ws)
        torch.cuda.synchronize()
        out.append(yp[:rows].clone())
    assert torch.equal(out[0].view(torch.int32), out[1].view(torch.int32))
    ref = np.stack([oracle.swiglu(case.h["W1"][0], case.h["W3"][0], case.h["W2"][0],
                                  moe_synth.bf16_to_f32(case.h["x"][i % wl.T]).astype(np.float64), bf16=True)
                    for i in range(rows)])
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(host_f64(out[0]) - ref)) <= 2e-2 * rms


def test_single_token():
    rep = check_case(Case(workload("deepseek_v3_fine", T=1, d=256, F=128, E=16, K=3, Fs=128)))
    print(rep)


def test_run_twice_bitwise_identical():
    case = Case(SMALL["deepseek_small"])
    y1, r1 = case.gpu_forward()
    y2, r2 = case.gpu_forward()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(r1.topk_idx, r2.topk_idx) and torch.equal(r1.topk_w, r2.topk_w)


def test_entry_points_in_isolation():
    """moe_route, moe_dispatch, moe_expert_ffn and moe_combine called one by
    one, each checked against the oracle's version of that step."""
    wl = SMALL["mixtral_two_mtiles"]
    case = Case(wl)
    orc = case.oracle_route()
    spec = spec_of(wl)
    ws, _ = moe.alloc_workspace(spec)
    r = moe.Routing(spec)
    moe.moe_route(spec, case.d["x"], case.d["Wg"], None, None, r, ws)
    torch.cuda.synchronize()
    g = routing_host(r)
    assert np.array_equal(g["idx"], orc["idx"])
    assert_permutation_equal(g, orc, "moe_route")

    R = int(orc["offsets"][-1])
    mr = moe.max_rows(spec)
    xp = torch.empty((mr, wl.d), dtype=torch.bfloat16, device="cuda")
    moe.moe_dispatch(spec, case.d["x"], r, xp)
    torch.cuda.synchronize()
    xp_h = xp[:R].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(xp_h, case.h["x"][orc["row_src"][:R] // wl.K])

    yp = torch.empty((mr, wl.d), dtype=torch.float32, device="cuda")
    moe.moe_expert_ffn(spec, xp, r.offsets, wl.E, mr, case.d["W1"], case.d["W3"], case.d["W2"], yp, ws,
                       scales=device_scales(case.d))
    torch.cuda.synchronize()
    yp_h = yp[:R].cpu().numpy().astype(np.float64)
    xrows = moe_synth.bf16_to_f32(case.h["x"][orc["row_src"][:R] // wl.K]).astype(np.float64)
    grp = np.searchsorted(orc["offsets"], np.arange(R), side="right") - 1
    pick = np.unique(np.concatenate([np.arange(0, R, 37), [R - 1], orc["offsets"][1:-1] - 1]))
    ref = np.stack([oracle.swiglu(case.h["W1"][grp[i]], case.h["W3"][grp[i]], case.h["W2"][grp[i]], xrows[i],
                                  bf16=True, threads=4) for i in pick])
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(yp_h[pick] - ref)) <= 2e-2 * rms

    # combine on the oracle's routing with seeded expert rows (fp32 output)
    ypr = moe_synth.normal(0, 99, (R, wl.d), 1.0, "f32")
    y = torch.empty((wl.T, wl.d), dtype=torch.float32, device="cuda")
    rr = moe.Routing(spec)
    rr.topk_w.copy_(torch.from_numpy(orc["w"].astype(np.float32)))
    rr.dest.copy_(torch.from_numpy(orc["dest"]))
    moe.moe_combine(spec_of(wl, out_dtype="f32"), dev(ypr), rr, None, None, y)
    torch.cuda.synchronize()
    ref_c = oracle.combine(oracle.layer_of(wl), ypr, orc["w"].astype(np.float32).astype(np.float64), orc["dest"])
    # fp32 accumulation of K terms in the same order: a few fp32 ulps
    assert np.max(np.abs(host_f64(y) - ref_c) / np.maximum(np.abs(ref_c), np.sqrt(np.mean(ref_c ** 2)))) <= 1e-5


def test_entry_points_in_isolation_even_m_tiles(monkeypatch):
    """The same, with moe_expert_ffn's GEMM1 m-tiles split evenly."""
    monkeypatch.setenv("MOE_TUNING", "1")
    monkeypatch.setenv("MOE_GEMM_EVEN_UP", "1")
    test_entry_points_in_isolation()


# -------------------------------------------------------- full-size cases --

FULL = ["tiny_top2_fp32", "switch_top1_capacity", "mixtral_prefill", "mixtral_decode", "deepseek_v3_fine"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    """Routing over all tokens; outputs on every token of the small workloads
    and, on the others, on tokens covering every (expert, m-tile) of both
    GEMMs -- held to the stated bound against the definition (h in double)
    with no h-storage allowance."""
    case = Case(workload(name))
    toks = None if case.wl.T <= 64 else sample_tokens(case)
    rep = check_case(case, tokens=toks, strict=True)
    print(name, "sampled" if toks is not None else "all", rep)
