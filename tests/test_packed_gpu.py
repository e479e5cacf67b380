"""Packed expert weights (moe_pack_weights + MOE_F_PACKED_UP / _DOWN).

The packed layout only moves weight values (each 64-element step of a
group's rows stored contiguously), so a layer run on packed weights must
give the row-major layer's results bit for bit, whatever plan its GEMMs
take; the row-major layer is itself held to the oracle by the parity tests,
and one case here is also checked against the oracle directly.  The pack
itself is compared with torch's reshape of the same tensor."""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
import mixture_experts_sparse_route_amd as moe
from moe_synth import workload
from parity_lib import (Case, assert_y_close, device_scales, host_f64, kept_tokens, routing_host, spec_of,
                        tile_sample_tokens)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load_library()
    moe_synth.build(force=False)
    oracle.build(force=False)


def packed_of(w: torch.Tensor) -> torch.Tensor:
    out = torch.empty_like(w)
    moe.moe_pack_weights(w, out)
    return out


@pytest.mark.parametrize("shape", [(1, 64, 64), (3, 128, 192), (2, 320, 4096), (5, 64, 128)])
def test_pack_equals_reshape(shape):
    G, N, K = shape
    print("pack", shape, flush=True)
    g = torch.Generator().manual_seed(G * 1000 + N + K)
    src = torch.randint(-32768, 32767, shape, dtype=torch.int16, generator=g).cuda().view(torch.bfloat16)
    dst = packed_of(src)
    torch.cuda.synchronize()
    ref = src.view(torch.int16).cpu().reshape(G, N // 64, 64, K // 64, 64).permute(0, 1, 3, 2, 4).contiguous()
    assert torch.equal(dst.view(torch.int16).cpu().reshape(G, N // 64, K // 64, 64, 64), ref)


@pytest.mark.parametrize("shape", [(2, 64, 96), (2, 72, 128)])
def test_pack_rejects_bad_sizes(shape):
    src = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.moe_pack_weights(src, torch.empty_like(src))


UP, DOWN = ("W1", "W3", "Ws1", "Ws3"), ("W2", "Ws2")


def forward(case: Case, packed: str):
    wl = case.wl
    spec = spec_of(wl, out_dtype="f32", packed=packed)
    d = dict(case.d)
    names = {"none": (), "up": UP, "down": DOWN, "both": UP + DOWN}[packed]
    for k in names:
        if d.get(k) is not None:
            d[k] = packed_of(d[k])
    r = moe.Routing(spec)
    ws, _ = moe.alloc_workspace(spec)
    y = torch.full((wl.T, wl.d), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_forward(spec, d["x"], d["Wg"], d["logit_bias"], d["sel_bias"], d["W1"], d["W3"], d["W2"], d["Ws1"],
                    d["Ws3"], d["Ws2"], y, r, ws, scales=device_scales(d))
    torch.cuda.synchronize()
    return y, r


CASES = {
    "deepseek_small": workload("deepseek_v3_fine", T=300, d=512, F=256, E=64, Fs=256),
    "mixtral_two_mtiles": workload("mixtral_prefill", T=1100, d=256, F=384),
    "mixtral_550_rows": workload("mixtral_prefill", T=2200, d=256, F=384),
    # uncapped groups averaging 250 rows: GEMM2 on packed W2 takes 192 x 128 tiles of 64 k
    "deepseek_mid": workload("deepseek_v3_fine", T=2000, d=256, F=256, E=64, Fs=256),
    # capacity 160: GEMM1 on packed W1 / W3 takes 192 x 128 tiles of 64 k
    "switch_capacity_160": workload("switch_top1_capacity", T=2048, d=256, F=512, E=16),
    "decode_small": workload("mixtral_decode", T=8, d=256, F=512),
    "short_reduction": workload("mixtral_prefill", T=700, d=64, F=128),
}


@pytest.mark.parametrize("name", list(CASES))
def test_packed_layer_bit_identical(name):
    case = Case(CASES[name])
    print(name, flush=True)
    y0, r0 = forward(case, "none")
    for packed in ("up", "down", "both"):
        y1, r1 = forward(case, packed)
        assert torch.equal(y0.view(torch.int32), y1.view(torch.int32)), f"output with {packed} packed differs"
        a, b = routing_host(r0), routing_host(r1)
        for k in ("idx", "offsets", "dest"):
            assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("name", ["deepseek_v3_fine", "mixtral_decode"])
def test_packed_full_size(name):
    """Full-size layers: bit-identical to row-major weights, and the sampled
    tokens (one in every m-tile of both GEMMs) within the stated bound of the
    oracle's definition."""
    print(name, "full size", flush=True)
    case = Case(workload(name))
    y0, _ = forward(case, "none")
    y1, r1 = forward(case, "both")
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32)), "packed-weight output differs"
    wl = case.wl
    orc = case.oracle_route()
    g = routing_host(r1)
    live = kept_tokens(orc["dest"], wl.K, wl.n_shared)
    same = np.all(g["idx"] == orc["idx"], axis=1)   # near-tie tokens may pick other experts
    toks = np.array([t for t in tile_sample_tokens(orc, wl.K, wl.T) if same[t]], dtype=np.int64)
    assert len(toks) > 0
    ref = case.oracle_y(orc["idx"], orc["w"], orc["dest"], tokens=toks)
    print(assert_y_close(host_f64(y1)[toks], ref, rows=live[toks], label=f"{name} packed", strict=True))


def test_packed_needs_bf16_or_e4m3_weights():
    wl = workload("tiny_top2_fp32")
    spec = spec_of(wl, packed="both")
    with pytest.raises(moe.MoeError):
        moe.workspace_size(spec)


def test_packed_noalloc_matches_forward():
    """moe_forward_noalloc on packed weights gives moe_forward's output on
    the same packed weights bit for bit (same kernels and plans)."""
    case = Case(CASES["deepseek_mid"])
    wl = case.wl
    y0, _ = forward(case, "both")
    spec = spec_of(wl, out_dtype="f32", packed="both")
    d = dict(case.d)
    for k in UP + DOWN:
        d[k] = packed_of(d[k])
    y1 = torch.full((wl.T, wl.d), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_forward_noalloc(spec, d["x"], d["Wg"], d["logit_bias"], d["sel_bias"], d["W1"], d["W3"], d["W2"],
                            d["Ws1"], d["Ws3"], d["Ws2"], y1, None)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32)), "noalloc output on packed weights differs"


def forward_variant(case: Case, packed: str, **spec_kw):
    """moe_forward with the routing variants of spec_kw (expert choice, drop
    policy, statistics, residual) on packed or row-major weights."""
    wl = case.wl
    spec = spec_of(wl, out_dtype="f32", packed=packed, **spec_kw)
    if spec_kw.get("expert_choice"):
        spec.renorm = False
    d = dict(case.d)
    names = {"none": (), "up": UP, "down": DOWN, "both": UP + DOWN}[packed]
    for k in names:
        if d.get(k) is not None:
            d[k] = packed_of(d[k])
    r = moe.Routing(spec)
    ws, _ = moe.alloc_workspace(spec)
    y = torch.full((wl.T, wl.d), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_forward(spec, d["x"], d["Wg"], d["logit_bias"], d["sel_bias"], d["W1"], d["W3"], d["W2"], d["Ws1"],
                    d["Ws3"], d["Ws2"], y, r, ws, scales=device_scales(d))
    torch.cuda.synchronize()
    return y


VARIANTS = {
    "expert_choice": dict(expert_choice=True),
    "drop_affinity": dict(drop_policy="affinity"),
    "drop_reroute": dict(drop_policy="reroute"),
    "stats_residual": dict(stats=True, residual=True),
}


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_packed_routing_variants_bit_identical(variant):
    """The routing variants feed the same grouped GEMMs: packed weights give
    the row-major outputs bit for bit (Switch shape with capacity 160)."""
    case = Case(CASES["switch_capacity_160"])
    print(variant, flush=True)
    y0 = forward_variant(case, "none", **VARIANTS[variant])
    for packed in ("up", "down", "both"):
        y1 = forward_variant(case, packed, **VARIANTS[variant])
        assert torch.equal(y0.view(torch.int32), y1.view(torch.int32)), f"{variant} with {packed} packed differs"


# ---------------------------------------------------------------- E4M3 weights

def test_pack_e4m3_equals_reshape():
    G, N, K = 3, 128, 192
    g = torch.Generator().manual_seed(7)
    src = torch.randint(0, 256, (G, N, K), dtype=torch.uint8, generator=g).cuda()
    dst = packed_of(src)
    torch.cuda.synchronize()
    ref = src.cpu().reshape(G, N // 64, 64, K // 64, 64).permute(0, 1, 3, 2, 4).contiguous()
    assert torch.equal(dst.cpu().reshape(G, N // 64, K // 64, 64, 64), ref)


FP8_CASES = {
    "mixtral_small": workload("mixtral_prefill", T=300, d=512, F=1024, wdtype="fp8"),
    "deepseek_shared": workload("deepseek_v3_fine", T=200, d=512, F=256, E=64, Fs=256, wdtype="fp8"),
    "deepseek_mid": workload("deepseek_v3_fine", T=2000, d=256, F=256, E=64, Fs=256, wdtype="fp8"),
    "decode_small": workload("mixtral_decode", T=8, d=256, F=512, wdtype="fp8"),
    "switch_capacity_160": workload("switch_top1_capacity", T=2048, d=256, F=512, E=16, wdtype="fp8"),
}


@pytest.mark.parametrize("name", list(FP8_CASES))
def test_packed_e4m3_bit_identical(name, monkeypatch):
    """E4M3 weights packed: every GEMM's and both, in the plans' stages of 64 k
    and, forced, in stages of 32 k: the row-major layer's output bit for bit."""
    case = Case(FP8_CASES[name])
    print(name, flush=True)
    y0, _ = forward(case, "none")
    for packed in ("up", "down", "both"):
        y1, _ = forward(case, packed)
        assert torch.equal(y0.view(torch.int32), y1.view(torch.int32)), f"E4M3 with {packed} packed differs"
    monkeypatch.setenv("MOE_TUNING", "1")
    for k, v in {"MOE_GEMM_K64": "0", "MOE_GEMM_BM": "128", "MOE_GEMM_BM_DOWN": "128", "MOE_GEMM_BNB_UP": "128",
                 "MOE_GEMM_NS_UP": "3", "MOE_GEMM_BNB_DOWN": "128", "MOE_GEMM_NS_DOWN": "3"}.items():
        monkeypatch.setenv(k, v)   # E4M3 in stages of 32 k, 128 x 128 tiles
    y2, _ = forward(case, "both")
    assert torch.equal(y0.view(torch.int32), y2.view(torch.int32)), "E4M3 packed in stages of 32 k differs"


def test_packed_e4m3_full_size():
    case = Case(workload("deepseek_v3_fine", wdtype="fp8"))
    print("deepseek_v3_fine fp8 full size", flush=True)
    y0, _ = forward(case, "none")
    y1, _ = forward(case, "both")
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32)), "E4M3 packed output differs"
