"""The C-ABI library loads, exports every symbol ``include/moe.h`` declares,
and rejects bad arguments on the host before touching the GPU.  CPU only:
no call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import mixture_experts_sparse_route_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        from mixture_experts_sparse_route_amd import build
        build.build()
    return moe.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_entry_points():
    names = declared_functions()
    for n in ("moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward", "moe_workspace_size"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(3) == b"MOE_ERR_WORKSPACE"
    assert [lib.moe_kernel_name(i).decode() for i in range(len(moe.KERNEL_NAMES))] == moe.KERNEL_NAMES
    assert lib.moe_kernel_name(len(moe.KERNEL_NAMES)) is None


def spec(**kw):
    base = dict(tokens=64, d_model=128, d_ff=256, n_experts=8, top_k=2, dtype="bf16")
    base.update(kw)
    return moe.LayerSpec(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(tokens=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(d_model=0), moe.MOE_ERR_INVALID_ARG),
    (dict(n_experts=0), moe.MOE_ERR_INVALID_ARG),
    (dict(n_experts=2048), moe.MOE_ERR_INVALID_ARG),
    (dict(top_k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(top_k=9), moe.MOE_ERR_INVALID_ARG),
    (dict(n_experts=64, top_k=33), moe.MOE_ERR_INVALID_ARG),
    (dict(gate=7), moe.MOE_ERR_INVALID_ARG),
    (dict(n_shared=2, d_ff_shared=256), moe.MOE_ERR_INVALID_ARG),
    (dict(n_shared=1, d_ff_shared=0), moe.MOE_ERR_INVALID_ARG),
    (dict(d_model=100), moe.MOE_ERR_UNSUPPORTED),          # bf16 needs multiples of 64
    (dict(d_ff=96), moe.MOE_ERR_UNSUPPORTED),
    (dict(capacity_factor=float("nan")), moe.MOE_ERR_INVALID_ARG),
    (dict(capacity_factor=float("inf")), moe.MOE_ERR_INVALID_ARG),
])
def test_invalid_configs_are_rejected_on_the_host(lib, kw, status):
    n = ctypes.c_size_t()
    got = lib.moe_workspace_size(ctypes.byref(spec(**kw).config()), ctypes.byref(n))
    assert got == status, lib.moe_last_error()
    assert lib.moe_last_error()


def test_unknown_flags_and_dtype_mismatch(lib):
    c = spec().config()
    c.flags |= 0x100
    assert lib.moe_workspace_size(ctypes.byref(c), ctypes.byref(ctypes.c_size_t())) == moe.MOE_ERR_INVALID_ARG
    c = spec().config()
    c.w_dtype = moe.MOE_F32
    assert lib.moe_workspace_size(ctypes.byref(c), ctypes.byref(ctypes.c_size_t())) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_workspace_size(None, ctypes.byref(ctypes.c_size_t())) == moe.MOE_ERR_INVALID_ARG


def test_fp32_accepts_any_sizes():
    assert moe.workspace_size(spec(d_model=100, d_ff=37, dtype="f32")) > 0


def test_max_rows_follows_the_capacity_formula():
    # Switch top-1: floor(1.25 * 8192 / 64) = 160 per expert, 64 experts -> 8192 (= T*K) bound
    assert moe.max_rows(spec(tokens=8192, d_model=1024, d_ff=4096, n_experts=64, top_k=1,
                             capacity_factor=1.25)) == 8192
    # capacity binds: floor(0.5 * 1000 / 10) = 50 per expert -> 500 rows at most
    assert moe.max_rows(spec(tokens=1000, n_experts=10, top_k=1, capacity_factor=0.5)) == 500
    # no capacity: every assignment
    assert moe.max_rows(spec(tokens=77, top_k=2)) == 154
    # tiny capacity: zero rows
    assert moe.max_rows(spec(tokens=10, n_experts=64, top_k=1, capacity_factor=1.0)) == 0


def test_workspace_grows_with_tokens():
    a = moe.workspace_size(spec(tokens=64))
    b = moe.workspace_size(spec(tokens=640))
    assert b > a > 0
    assert moe.workspace_size(spec(tokens=0)) > 0


def test_entry_points_reject_null_and_small_workspace_without_launching(lib):
    c = spec().config()
    r = moe.MoeRouting()
    # routing arrays missing
    assert lib.moe_route(ctypes.byref(c), 256, 256, None, None, ctypes.byref(r), 256, 1 << 30, None) \
        == moe.MOE_ERR_INVALID_ARG
    r = moe.MoeRouting(*([256] * 8))
    # workspace NULL, misaligned, too small
    assert lib.moe_route(ctypes.byref(c), 256, 256, None, None, ctypes.byref(r), None, 0, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_route(ctypes.byref(c), 256, 256, None, None, ctypes.byref(r), 257, 1 << 30, None) \
        == moe.MOE_ERR_WORKSPACE
    assert lib.moe_route(ctypes.byref(c), 256, 256, None, None, ctypes.byref(r), 256, 16, None) == moe.MOE_ERR_WORKSPACE
    # x / Wg missing
    assert lib.moe_route(ctypes.byref(c), None, None, None, None, ctypes.byref(r), 256, 1 << 30, None) \
        == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch(ctypes.byref(c), None, ctypes.byref(r), 256, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_ffn(ctypes.byref(c), 256, 256, 0, 16, 256, 256, 256, None, 256, 256, 1 << 30, None) \
        == moe.MOE_ERR_INVALID_ARG  # n_groups = 0
    assert lib.moe_expert_ffn(ctypes.byref(c), 256, 256, 8, 1 << 20, 256, 256, 256, None, 256, 256, 1 << 30, None) \
        == moe.MOE_ERR_INVALID_ARG  # max_rows above the config's bound
    cr = spec(residual=True).config()
    assert lib.moe_combine(ctypes.byref(cr), 256, ctypes.byref(r), None, None, 256, None) == moe.MOE_ERR_INVALID_ARG
    # shared expert weights required
    cs = spec(n_shared=1, d_ff_shared=256).config()
    assert lib.moe_forward(ctypes.byref(cs), 256, 256, None, None, 256, 256, 256, None, None, None, None, 256, None, 256, 1 << 30,
                           None) == moe.MOE_ERR_INVALID_ARG
    # *_IN flags need the routing arrays
    ci = spec(logits_in=True).config()
    assert lib.moe_forward(ctypes.byref(ci), 256, 256, None, None, 256, 256, 256, None, None, None, None, 256, None, 256, 1 << 30,
                           None) == moe.MOE_ERR_INVALID_ARG


def test_zero_tokens_is_a_no_op(lib):
    c = spec(tokens=0).config()
    r = moe.MoeRouting(*([256] * 8))
    n = moe.workspace_size(spec(tokens=0))
    assert lib.moe_route(ctypes.byref(c), 256, 256, None, None, ctypes.byref(r), 256, n, None) == moe.MOE_OK
    assert lib.moe_dispatch(ctypes.byref(c), 256, ctypes.byref(r), 256, None) == moe.MOE_OK
    assert lib.moe_combine(ctypes.byref(c), 256, ctypes.byref(r), None, None, 256, None) == moe.MOE_OK
    assert lib.moe_forward(ctypes.byref(c), 256, 256, None, None, 256, 256, 256, None, None, None, None, 256, None, 256, n,
                           None) == moe.MOE_OK


def test_statistics_flag_validation(lib):
    """MOE_F_STATS: needs logits (rejected with MOE_F_TOPK_IN), needs
    routing->stats, and adds its per-chunk partial sums to the workspace."""
    n = ctypes.c_size_t()
    c = spec(stats=True, topk_in=True).config()
    assert lib.moe_workspace_size(ctypes.byref(c), ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG
    assert b"MOE_F_STATS" in lib.moe_last_error()
    assert moe.workspace_size(spec(stats=True, tokens=4096)) > moe.workspace_size(spec(tokens=4096))
    c = spec(stats=True).config()
    r = moe.MoeRouting(*([256] * 8), None)   # stats pointer missing
    assert lib.moe_route(ctypes.byref(c), 256, 256, None, None, ctypes.byref(r), 256, 1 << 30, None) \
        == moe.MOE_ERR_INVALID_ARG
    assert b"stats" in lib.moe_last_error()
    # moe_forward with statistics needs caller routing arrays
    assert lib.moe_forward(ctypes.byref(c), 256, 256, None, None, 256, 256, 256, None, None, None, None, 256, None, 256, 1 << 30,
                           None) == moe.MOE_ERR_INVALID_ARG


def test_routing_struct_matches_the_header():
    """moe_routing in moe.h: eight array pointers, then the statistics pointer."""
    src = open(HEADER).read()
    body = re.search(r"typedef struct moe_routing \{(.*?)\} moe_routing;", src, re.S).group(1)
    names = re.findall(r"\*\s*(\w+);", body)
    assert names == [f[0] for f in moe.MoeRouting._fields_]
    assert ctypes.sizeof(moe.MoeRouting) == 8 * len(names)


def test_drop_policy_validation(lib):
    """drop_policy: known values only; re-routing needs logits; the policies'
    scratch arrays enlarge the workspace only when capacity is on."""
    n = ctypes.c_size_t()
    c = spec(capacity_factor=1.0).config()
    c.drop_policy = 3
    assert lib.moe_workspace_size(ctypes.byref(c), ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG
    c = spec(capacity_factor=1.0, drop_policy="reroute", topk_in=True).config()
    assert lib.moe_workspace_size(ctypes.byref(c), ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG
    assert b"MOE_DROP_REROUTE" in lib.moe_last_error()
    base = moe.workspace_size(spec(tokens=4096, capacity_factor=1.0))
    for p in ("affinity", "reroute"):
        assert moe.workspace_size(spec(tokens=4096, capacity_factor=1.0, drop_policy=p)) > base
        assert moe.workspace_size(spec(tokens=4096, drop_policy=p)) == moe.workspace_size(spec(tokens=4096))
    assert moe.workspace_size(spec(capacity_factor=1.0, drop_policy="affinity", topk_in=True)) > 0


def test_expert_choice_validation(lib):
    n = ctypes.c_size_t()
    for kw, st in ((dict(gate=moe.MOE_GATE_SIGMOID), moe.MOE_ERR_UNSUPPORTED), (dict(topk_in=True), moe.MOE_ERR_INVALID_ARG),
                   (dict(stats=True), moe.MOE_ERR_INVALID_ARG), (dict(renorm=True), moe.MOE_ERR_INVALID_ARG)):
        base = dict(expert_choice=True, renorm=False)
        base.update(kw)
        c = spec(**base).config()
        assert lib.moe_workspace_size(ctypes.byref(c), ctypes.byref(n)) == st, kw
    # cap = floor(C*T*K/E), at most T; rows = E * cap
    assert moe.max_rows(spec(expert_choice=True, renorm=False, tokens=100, n_experts=8, top_k=2,
                             capacity_factor=1.25)) == 8 * 31
    assert moe.max_rows(spec(expert_choice=True, renorm=False, tokens=100, n_experts=8, top_k=2)) == 8 * 25
    assert moe.max_rows(spec(expert_choice=True, renorm=False, tokens=10, n_experts=2, top_k=2,
                             capacity_factor=3.0)) == 2 * 10


def test_fp8_weight_validation(lib):
    """MOE_FP8_E4M3 expert weights: only with bf16 activations, and the scales
    are required by moe_expert_ffn and moe_forward."""
    n = ctypes.c_size_t()
    c = spec(dtype="f32", wdtype="fp8").config()
    assert lib.moe_workspace_size(ctypes.byref(c), ctypes.byref(n)) == moe.MOE_ERR_UNSUPPORTED
    c = spec(wdtype="fp8").config()
    assert c.w_dtype == moe.MOE_FP8_E4M3 and c.act_dtype == moe.MOE_BF16
    assert lib.moe_workspace_size(ctypes.byref(c), ctypes.byref(n)) == moe.MOE_OK
    assert lib.moe_expert_ffn(ctypes.byref(c), 256, 256, 8, 16, 256, 256, 256, None, 256, 256, 1 << 30, None) \
        == moe.MOE_ERR_INVALID_ARG
    assert b"scales" in lib.moe_last_error()
    half = moe.MoeScales(256, 256, None, None, None, None)
    assert lib.moe_expert_ffn(ctypes.byref(c), 256, 256, 8, 16, 256, 256, 256, ctypes.byref(half), 256, 256, 1 << 30, None) \
        == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_forward(ctypes.byref(c), 256, 256, None, None, 256, 256, 256, None, None, None, None, 256, None, 256, 1 << 30,
                           None) == moe.MOE_ERR_INVALID_ARG
    cs = spec(wdtype="fp8", n_shared=1, d_ff_shared=128).config()
    full = moe.MoeScales(256, 256, 256, None, None, None)      # shared-expert scales missing
    assert lib.moe_forward(ctypes.byref(cs), 256, 256, None, None, 256, 256, 256, 256, 256, 256, ctypes.byref(full), 256, None, 256,
                           1 << 30, None) == moe.MOE_ERR_INVALID_ARG


def test_misaligned_arrays_are_rejected_without_launching(lib):
    """Activation, weight, scale and output arrays are accessed 16 bytes at a
    time: a pointer off a 16-byte boundary is an argument error."""
    c = spec().config()
    r = moe.MoeRouting(*([256] * 8))
    assert lib.moe_route(ctypes.byref(c), 256 + 8, 256, None, None, ctypes.byref(r), 256, 1 << 30, None) \
        == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch(ctypes.byref(c), 256, ctypes.byref(r), 256 + 4, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_ffn(ctypes.byref(c), 256, 256, 8, 16, 256, 256, 256, None, 256 + 8, 256, 1 << 30, None) \
        == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(ctypes.byref(c), 256, ctypes.byref(r), None, None, 256 + 2, None) \
        == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_forward(ctypes.byref(c), 256, 256, None, None, 256, 256 + 8, 256, None, None, None, None, 256, None,
                           256, 1 << 30, None) == moe.MOE_ERR_INVALID_ARG
    assert b"16-byte aligned" in lib.moe_last_error()


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for several it exits with status 2
    and says so, before touching a device."""
    import subprocess
    import sys
    for args, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                           timeout=120, env={**os.environ, **env}, cwd=ROOT)
        assert p.returncode == 2, (args, env, p.returncode, p.stderr[-500:])
        assert "one GPU only" in p.stderr and p.stdout == ""


def test_noalloc_rejects_a_layer_larger_than_its_scratch(lib):
    """moe_forward_noalloc checks the layer's scratch need against its
    built-in array on the host, before any HIP call (this machine has no
    GPU: a call that got further would fail with MOE_ERR_HIP)."""
    sp = spec(tokens=4096, d_model=4096, d_ff=14336, n_experts=8, top_k=2)
    assert moe.workspace_size(sp) > moe.NOALLOC_SCRATCH_BYTES
    st = lib.moe_forward_noalloc(ctypes.byref(moe._cfg(sp)), *([None] * 10), None, None, None, None)
    assert st == moe.MOE_ERR_WORKSPACE and b"built-in" in lib.moe_last_error()


def test_packed_weight_validation(lib):
    """MOE_F_PACKED_UP / _DOWN only with bf16 weights; moe_pack_weights checks
    sizes, alignment and overlap on the host before any launch."""
    n = ctypes.c_size_t()
    assert (moe.MOE_F_PACKED_UP, moe.MOE_F_PACKED_DOWN) == (64, 128)
    for packed, bits in (("up", 64), ("down", 128), ("both", 192)):
        for ok in (spec(packed=packed), spec(packed=packed, wdtype="fp8")):
            c = ok.config()
            assert c.flags & 192 == bits
            assert lib.moe_workspace_size(ctypes.byref(c), ctypes.byref(n)) == moe.MOE_OK
        c = spec(packed=packed, dtype="f32").config()
        assert lib.moe_workspace_size(ctypes.byref(c), ctypes.byref(n)) == moe.MOE_ERR_UNSUPPORTED
    def pack(src, dst, g, n, k, wd=moe.MOE_BF16):
        return lib.moe_pack_weights(src, dst, g, n, k, wd, None)
    big = 1 << 40
    assert pack(None, big, 2, 64, 64) == moe.MOE_ERR_INVALID_ARG
    assert pack(256, big, 2, 64, 96) == moe.MOE_ERR_INVALID_ARG       # K not a multiple of 64
    assert pack(256, big, 2, 72, 64) == moe.MOE_ERR_INVALID_ARG       # N not a multiple of 64
    assert pack(256, big, 0, 64, 64) == moe.MOE_ERR_INVALID_ARG       # no groups
    assert pack(256, big, 2, 0, 64) == moe.MOE_ERR_INVALID_ARG        # no rows
    assert pack(256 + 8, big, 2, 64, 64) == moe.MOE_ERR_INVALID_ARG   # misaligned
    assert pack(256, big, 2, 64, 64, moe.MOE_F32) == moe.MOE_ERR_INVALID_ARG   # fp32 weights are not packed
    assert pack(4096, 4096 + 1024, 2, 64, 64) == moe.MOE_ERR_INVALID_ARG  # overlapping (2 x 64 x 64 x 2 bytes)
    assert pack(4096, 4096 + 4096, 2, 64, 64, moe.MOE_FP8_E4M3) == moe.MOE_ERR_INVALID_ARG  # 8 KB of E4M3: overlapping
    assert b"overlap" in lib.moe_last_error()
