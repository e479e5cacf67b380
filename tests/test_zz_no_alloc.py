"""moe_forward_noalloc, the entry point that allocates nothing, against
moe_forward on the same inputs: same kernels, so outputs and routing must be
bit-identical, and both within the layer tolerance of the oracle.  Two calls
in a row share the GPU's one scratch array, the second with fewer tokens, so
what the first leaves behind in the array must not leak into the second."""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
import mixture_experts_sparse_route_amd as moe
from moe_synth import workload
from parity_lib import Case, assert_y_close, device_scales, host_f64, kept_tokens, routing_host, spec_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load_library()
    moe_synth.build(force=False)
    oracle.build(force=False)


def forward_both(case: Case, with_routing=True):
    """(y, routing) of moe_forward and of moe_forward_noalloc, fp32 outputs."""
    wl = case.wl
    spec = spec_of(wl, out_dtype="f32")
    d = case.d
    args = (d["x"], d["Wg"], d["logit_bias"], d["sel_bias"], d["W1"], d["W3"], d["W2"], d["Ws1"], d["Ws3"], d["Ws2"])
    ws, _ = moe.alloc_workspace(spec)
    r0 = moe.Routing(spec)
    y0 = torch.empty((wl.T, wl.d), dtype=torch.float32, device="cuda")
    moe.moe_forward(spec, *args, y0, r0, ws, scales=device_scales(d))
    r1 = moe.Routing(spec) if with_routing else None
    y1 = torch.full((wl.T, wl.d), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_forward_noalloc(spec, *args, y1, r1, scales=device_scales(d))
    torch.cuda.synchronize()
    return (y0, r0), (y1, r1)


def check(case: Case, with_routing=True):
    (y0, r0), (y1, r1) = forward_both(case, with_routing)
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32)), "noalloc output differs from moe_forward"
    if r1 is not None:
        a, b = routing_host(r0), routing_host(r1)
        R = int(a["offsets"][-1])
        for k in ("logits", "idx", "w", "counts", "offsets", "dest", "dropped"):
            assert np.array_equal(a[k], b[k]), k
        assert np.array_equal(a["row_src"][:R], b["row_src"][:R])
    # and the layer tolerance against the oracle
    orc = case.oracle_route()
    g = routing_host(r0)
    if np.array_equal(g["idx"], orc["idx"]):
        live = kept_tokens(orc["dest"], case.wl.K, case.wl.n_shared)
        ref = case.oracle_y(orc["idx"], orc["w"], orc["dest"])
        return assert_y_close(host_f64(y1), ref, rows=live, label="noalloc")
    return None


def test_two_calls_second_smaller():
    big = workload("deepseek_v3_fine", T=300, d=512, F=256, E=64, Fs=256)
    small = big.with_(T=37)
    print("first", check(Case(big)))
    print("second", check(Case(small)))


def test_internal_routing_then_decode_full_size():
    """Routing arrays kept in the scratch array (no caller routing), then the
    full-size Mixtral-shaped decode step (T=32, d=4096, F=14336, E=8, K=2)."""
    print(check(Case(workload("deepseek_v3_fine", T=120, d=256, F=128, E=32, K=4, Fs=128)), with_routing=False))
    print(check(Case(workload("mixtral_decode"))))


def test_oversize_layer_is_rejected():
    spec = spec_of(workload("mixtral_prefill"))
    assert moe.workspace_size(spec) > moe.NOALLOC_SCRATCH_BYTES
    y = torch.empty((1,), device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_noalloc(spec, y, y, None, None, y, y, y, None, None, None, y, None)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE and "built-in" in str(ei.value)
