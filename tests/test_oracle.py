"""Pins of the CPU oracle against things other than itself.

Library routines (numpy, scipy, torch in float64), brute force on tiny
inputs, closed forms, invariants, and the worked numbers the pages print
(``tests/golden/``).  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import moe_synth
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _built():
    moe_synth.build(force=False)
    oracle.build(force=False)


def rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- generator --

def test_splitmix64_published_sequence():
    g = json.load(open(os.path.join(GOLDEN, "splitmix64_seed0.json")))
    got = moe_synth.splitmix64(g["state"], len(g["outputs_hex"]))
    assert [f"{int(v):016x}" for v in got] == g["outputs_hex"]


def test_generator_distribution_and_slicing():
    a = moe_synth.normal(0, 7, (1 << 20,), 1.0, "f32")
    assert abs(a.mean()) < 5e-3 and abs(a.std() - 1.0) < 5e-3
    import scipy.stats
    assert scipy.stats.kstest(a[:20000].astype(np.float64), "norm").pvalue > 1e-3
    # any slice is generated on its own
    b = moe_synth.normal(0, 7, (1000,), 1.0, "f32", offset=12345)
    assert np.array_equal(a[12345:13345], b)
    # bf16 = RNE(fp32 draw)
    c = moe_synth.normal(0, 7, (4096,), 1.0, "bf16")
    t = torch.from_numpy(a[:4096].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(c, t)
    u = moe_synth.uniform(0, 8, (100000,), -0.1, 0.1)
    assert u.min() >= -0.1 and u.max() <= 0.1 and abs(u.mean()) < 2e-3


# ------------------------------------------------------------------ a1 logits --

def test_logits_exact_on_small_integers():
    r = rng(1)
    T, d, E = 17, 40, 6
    x = r.integers(-8, 9, size=(T, d)).astype(np.float32)
    Wg = r.integers(-8, 9, size=(E, d)).astype(np.float32)
    b = r.integers(-4, 5, size=E).astype(np.float32)
    L = oracle.layer(T, d, 8, E, 2)
    got = oracle.logits(L, x, Wg, b)
    want = (x.astype(np.int64) @ Wg.astype(np.int64).T + b.astype(np.int64)).astype(np.float32)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("bf16", [False, True])
def test_logits_match_float64_matmul(bf16):
    r = rng(2)
    T, d, E = 33, 96, 10
    xf = r.standard_normal((T, d)).astype(np.float32)
    x = moe_synth.f32_to_bf16(xf) if bf16 else xf
    xw = moe_synth.bf16_to_f32(x) if bf16 else xf
    Wg = (r.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    L = oracle.layer(T, d, 8, E, 2, bf16=bf16)
    got = oracle.logits(L, x, Wg, None)
    want = xw.astype(np.float64) @ Wg.astype(np.float64).T
    # the only difference is the summation order inside a double sum, then one fp32 rounding
    np.testing.assert_allclose(got, want, rtol=2 ** -23, atol=1e-12)


# ------------------------------------------------------------ a2 + a3 select --

def brute_topk(key, K):
    """Brute force: stable sort of (-key, expert)."""
    T, E = key.shape
    out = np.empty((T, K), np.int32)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(key[t, e]), e))
        out[t] = order[:K]
    return out


@pytest.mark.parametrize("K,renorm", [(1, False), (2, True), (3, False), (8, True)])
def test_softmax_select_vs_brute_force(K, renorm):
    r = rng(3)
    T, E = 50, 8
    lg = r.standard_normal((T, E)).astype(np.float32)
    L = oracle.layer(T, 4, 4, E, K, renorm=renorm)
    idx, w, gap = oracle.select(L, lg)
    assert np.array_equal(idx, brute_topk(lg, K))
    p = scipy.special.softmax(lg.astype(np.float64), axis=1)
    pk = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    want = pk / pk.sum(1, keepdims=True) if renorm else pk
    np.testing.assert_allclose(w, want, rtol=1e-14, atol=0)
    if K < E:
        srt = -np.sort(-lg.astype(np.float64), axis=1)
        np.testing.assert_array_equal(gap, srt[:, K - 1] - srt[:, K])
    else:
        assert np.all(np.isinf(gap))


def test_keep_topk_then_softmax_equals_renormalised_topk():
    """G = Softmax(KeepTopK(H, k)) (Tech Daily §3.1) equals the renormalised
    Top-K of the full softmax (Tech Daily §9.1)."""
    r = rng(4)
    T, E, K = 64, 16, 4
    lg = (3 * r.standard_normal((T, E))).astype(np.float32)
    L = oracle.layer(T, 4, 4, E, K, renorm=True)
    idx, w, _ = oracle.select(L, lg)
    for t in range(T):
        masked = np.full(E, -np.inf)
        top = np.argsort(-lg[t].astype(np.float64), kind="stable")[:K]
        masked[top] = lg[t, top]
        G = scipy.special.softmax(masked)
        np.testing.assert_allclose(w[t], G[idx[t]], rtol=1e-14)
        assert abs(G.sum() - 1) < 1e-15 and np.count_nonzero(G) == K


def test_renormalised_weights_sum_to_one_and_k1_is_one():
    r = rng(5)
    lg = (4 * r.standard_normal((200, 64))).astype(np.float32)
    for K in (2, 6):
        _, w, _ = oracle.select(oracle.layer(200, 4, 4, 64, K, renorm=True), lg)
        assert np.max(np.abs(w.sum(1) - 1)) < 4e-16
    _, w1, _ = oracle.select(oracle.layer(200, 4, 4, 64, 1, renorm=True), lg)
    assert np.all(w1 == 1.0)


def test_softmax_gap_ratio_golden():
    g = json.load(open(os.path.join(GOLDEN, "softmax_gap_ratio.json")))
    lg = np.array([[g["gap"], 0.0]], np.float32)
    _, w, _ = oracle.select(oracle.layer(1, 4, 4, 2, 2, renorm=False), lg)
    ratio = w[0, 0] / w[0, 1]
    assert abs(ratio - g["ratio_printed"]) <= g["ratio_tolerance"]
    assert abs(ratio - math.e) < 1e-12


def test_ties_go_to_lower_expert_and_signed_zero_is_a_tie():
    lg = np.array([[0.5, 1.0, 1.0, 0.5], [-0.0, 0.0, -1.0, -0.0]], np.float32)
    L = oracle.layer(2, 4, 4, 4, 3)
    idx, _, gap = oracle.select(L, lg)
    assert idx[0].tolist() == [1, 2, 0]
    assert idx[1].tolist() == [0, 1, 3]
    assert gap[0] == 0.0 and gap[1] == 1.0


def test_shift_invariance_of_softmax_routing():
    r = rng(6)
    # dyadic logits so that adding 0.5 is exact in fp32
    lg = (r.integers(-64, 64, size=(40, 12)) / 8.0).astype(np.float32)
    L = oracle.layer(40, 4, 4, 12, 3, renorm=False)
    i1, w1, _ = oracle.select(L, lg)
    i2, w2, _ = oracle.select(L, lg + np.float32(0.5))
    assert np.array_equal(i1, i2)
    np.testing.assert_allclose(w1, w2, rtol=1e-14)


def test_sigmoid_gate_bias_selects_but_does_not_weight():
    """Tech Daily §4.3 / §9.2: the bias enters only the selection."""
    r = rng(7)
    T, E, K = 30, 16, 4
    lg = r.standard_normal((T, E)).astype(np.float32)
    sb = (0.1 * r.uniform(-1, 1, E)).astype(np.float32)
    L = oracle.layer(T, 4, 4, E, K, gate=oracle.GATE_SIGMOID, renorm=False)
    idx, w, _ = oracle.select(L, lg, sb)
    s = scipy.special.expit(lg.astype(np.float64))
    key = s.astype(np.float32) + sb
    assert np.array_equal(idx, brute_topk(key, K))
    np.testing.assert_allclose(w, np.take_along_axis(s, idx.astype(np.int64), 1), rtol=1e-15)
    # a huge bias on expert j puts j first in every set; its weight stays s_j
    j = 5
    sb2 = sb.copy()
    sb2[j] = 1e4
    idx2, w2, _ = oracle.select(L, lg, sb2)
    assert np.all(idx2[:, 0] == j)
    np.testing.assert_allclose(w2[:, 0], s[:, j], rtol=1e-15)
    # renormalised: the K weights sum to 1
    Lr = oracle.layer(T, 4, 4, E, K, gate=oracle.GATE_SIGMOID, renorm=True)
    _, w3, _ = oracle.select(Lr, lg, sb)
    assert np.max(np.abs(w3.sum(1) - 1)) < 4e-16


# ---------------------------------------------------------------- a4 permute --

def test_capacity_golden():
    g = json.load(open(os.path.join(GOLDEN, "capacity_examples.json")))
    for c in g["cases"]:
        L = oracle.layer(c["tokens"], 4, 4, c["experts"], c["top_k"], capacity_factor=c["C"])
        assert oracle.capacity(L) == c["K_max"], c["cite"]
    assert oracle.capacity(oracle.layer(100, 4, 4, 8, 2, capacity_factor=0.0)) == -1


def brute_permute(idx_flat, E, cap):
    """Stable sort of the assignments by expert (numpy), then capacity."""
    N = idx_flat.size
    order = np.argsort(idx_flat, kind="stable")
    counts = np.bincount(idx_flat, minlength=E).astype(np.int32)
    kept = np.minimum(counts, cap) if cap >= 0 else counts
    offsets = np.concatenate([[0], np.cumsum(kept)]).astype(np.int32)
    start = np.concatenate([[0], np.cumsum(counts)])
    dest = np.full(N, -1, np.int32)
    row_src = np.full(N, -1, np.int32)
    for e in range(E):
        members = order[start[e]:start[e + 1]]
        for p, f in enumerate(members):
            if cap < 0 or p < cap:
                dest[f] = offsets[e] + p
                row_src[dest[f]] = f
    return counts, offsets, dest, row_src


@pytest.mark.parametrize("T,K,E,cf", [(300, 1, 16, 1.25), (257, 2, 8, 1.0), (128, 4, 32, 0.0),
                                      (64, 1, 8, 0.05), (0, 2, 8, 1.0), (90, 3, 5, 2.0)])
def test_permute_vs_stable_sort(T, K, E, cf):
    r = rng(8)
    # skewed demand so that capacity bites
    p = np.arange(E, 0, -1, dtype=np.float64) ** 2
    idx = r.choice(E, size=(T, K), p=p / p.sum()).astype(np.int32)
    L = oracle.layer(T, 4, 4, E, K, capacity_factor=cf)
    cap = oracle.capacity(L)
    got = oracle.permute(L, idx)
    counts, offsets, dest, row_src = brute_permute(idx.reshape(-1), E, cap)
    assert np.array_equal(got["counts"], counts)
    assert np.array_equal(got["offsets"], offsets)
    assert np.array_equal(got["dest"], dest)
    assert np.array_equal(got["row_src"], row_src)
    assert np.array_equal(got["dropped"], (dest < 0).astype(np.uint8))
    assert counts.sum() == T * K
    if cap >= 0:
        assert np.all(np.diff(offsets) == np.minimum(counts, cap))
    R = offsets[-1]
    assert sorted(row_src[:R].tolist()) == sorted(np.nonzero(dest >= 0)[0].tolist())


def test_capacity_zero_drops_everything():
    idx = np.zeros((10, 1), np.int32)
    L = oracle.layer(10, 4, 4, 64, 1, capacity_factor=1.0)  # floor(10/64) = 0
    assert oracle.capacity(L) == 0
    got = oracle.permute(L, idx)
    assert got["offsets"][-1] == 0 and np.all(got["dest"] == -1) and np.all(got["dropped"] == 1)


# -------------------------------------------------------------- a6-a7 expert --

def torch_swiglu(W1, W3, W2, x):
    W1, W3, W2, x = (torch.from_numpy(np.asarray(a, dtype=np.float64)) for a in (W1, W3, W2, x))
    return (W2 @ (torch.nn.functional.silu(W1 @ x) * (W3 @ x))).numpy()


@pytest.mark.parametrize("bf16", [False, True])
def test_swiglu_vs_torch(bf16):
    r = rng(9)
    d, F = 48, 80
    W = [r.standard_normal(s).astype(np.float32) / 5 for s in ((F, d), (F, d), (d, F))]
    if bf16:
        W = [moe_synth.f32_to_bf16(a) for a in W]
        Wf = [moe_synth.bf16_to_f32(a) for a in W]
    else:
        Wf = W
    x = r.standard_normal(d)
    for threads in (1, 4):
        got = oracle.swiglu(*W, x, bf16=bf16, threads=threads)
        np.testing.assert_allclose(got, torch_swiglu(*Wf, x), rtol=1e-12, atol=1e-14)


def test_bf16_round():
    """Against the integer round-to-nearest-even of fp32 bit patterns (values
    that are exact in fp32, normal and subnormal) and at exact ties."""
    r = rng(31)
    f = np.concatenate([r.standard_normal(20000) * 10.0 ** r.integers(-30, 30, 20000),
                        r.standard_normal(2000) * 1e-39]).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    want = (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32)
    got = np.array([oracle.bf16_round(float(v)) for v in f])
    assert np.array_equal(got, want.astype(np.float64))
    one_ulp = 2.0 ** -7
    assert oracle.bf16_round(1 + one_ulp / 2) == 1.0                   # tie to the even 1.0
    assert oracle.bf16_round(1 + 3 * one_ulp / 2) == 1 + 2 * one_ulp    # tie to the even mantissa
    assert oracle.bf16_round(-(1 + one_ulp / 2)) == -1.0
    assert oracle.bf16_round(1 + one_ulp / 2 + 2.0 ** -40) == 1 + one_ulp  # above the tie (not fp32-exact)
    assert oracle.bf16_round(0.0) == 0.0


def test_swiglu_round_h_vs_torch():
    """round_h: h stored as bf16 before W2 (torch's bf16 cast of the fp32 h;
    the fp32 step rounds twice only inside a 2^-29-wide window that random
    data does not hit)."""
    r = rng(32)
    d, F = 48, 80
    W = [moe_synth.f32_to_bf16(r.standard_normal(s).astype(np.float32) / 5) for s in ((F, d), (F, d), (d, F))]
    Wf = [torch.from_numpy(moe_synth.bf16_to_f32(a).astype(np.float64)) for a in W]
    x = r.standard_normal(d)
    xt = torch.from_numpy(x)
    hh = torch.nn.functional.silu(Wf[0] @ xt) * (Wf[1] @ xt)
    want = (Wf[2] @ hh.float().bfloat16().double()).numpy()
    got = oracle.swiglu(*W, x, bf16=True, round_h=True)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)
    assert not np.allclose(got, oracle.swiglu(*W, x, bf16=True), rtol=1e-6, atol=0)


def test_swiglu_closed_forms():
    r = rng(10)
    d, F = 16, 24
    W1, W3, W2 = (r.standard_normal(s).astype(np.float32) for s in ((F, d), (F, d), (d, F)))
    x = r.standard_normal(d)
    # SiLU(0) = 0: a zero gate projection gives exactly zero
    assert np.all(oracle.swiglu(np.zeros_like(W1), W3, W2, x, bf16=False) == 0)
    # doubling W2 doubles the output exactly
    y1 = oracle.swiglu(W1, W3, W2, x, bf16=False)
    y2 = oracle.swiglu(W1, W3, (2 * W2).astype(np.float32), x, bf16=False)
    assert np.array_equal(2 * y1, y2)
    # d = F = 1: SiLU(a) * b * w2 with SiLU(a) = a * sigmoid(a)
    a, b, c = 1.5, -0.75, 2.0
    got = oracle.swiglu(np.array([[1.0]], np.float32), np.array([[b / a]], np.float32) * 0 + np.float32(b),
                        np.array([[c]], np.float32), np.array([a]), bf16=False)
    assert abs(got[0] - a * scipy.special.expit(a) * (b * a) * c) < 1e-14


# ---------------------------------------------------------- a9 end to end ----

def small_layer(T=12, d=16, F=24, E=6, K=2, renorm=True, shared=0, seed=11):
    r = rng(seed)
    x = r.standard_normal((T, d)).astype(np.float32)
    Wg = (r.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    W1 = (r.standard_normal((E, F, d)) / np.sqrt(d)).astype(np.float32)
    W3 = (r.standard_normal((E, F, d)) / np.sqrt(d)).astype(np.float32)
    W2 = (r.standard_normal((E, d, F)) / np.sqrt(F)).astype(np.float32)
    Ws = None
    if shared:
        Ws = ((r.standard_normal((shared, F, d)) / np.sqrt(d)).astype(np.float32),
              (r.standard_normal((shared, F, d)) / np.sqrt(d)).astype(np.float32),
              (r.standard_normal((shared, d, F)) / np.sqrt(F)).astype(np.float32))
    L = oracle.layer(T, d, F, E, K, renorm=renorm, n_shared=shared, Fs=F if shared else 0)
    return L, x, Wg, W1, W3, W2, Ws


def oracle_forward(L, x, Wg, W1, W3, W2, Ws=None, sel_bias=None):
    rt = oracle.route(L, x, Wg, None, sel_bias)
    Ws = Ws or (None, None, None)
    return oracle.forward_rows(L, x, rt["idx"], rt["w"], rt["dest"], W1, W3, W2, *Ws), rt


def test_sparse_equals_run_all_experts_then_mask():
    """Brute force: every expert on every token, then the KeepTopK softmax
    gate of Tech Daily §3.1 (zero outside the Top-K) weights the sum."""
    L, x, Wg, W1, W3, W2, _ = small_layer()
    y, rt = oracle_forward(L, x, Wg, W1, W3, W2)
    # the router's logits are fp32 (pinned on their own above)
    lg = rt["logits"].astype(np.float64)
    for t in range(L.T):
        masked = np.full(L.E, -np.inf)
        top = np.argsort(-lg[t], kind="stable")[:L.K]
        masked[top] = lg[t, top]
        G = scipy.special.softmax(masked)
        want = sum(G[e] * torch_swiglu(W1[e], W3[e], W2[e], x[t].astype(np.float64)) for e in range(L.E))
        np.testing.assert_allclose(y[t], want, rtol=1e-10, atol=1e-13)


def test_k_equals_e_is_the_dense_softmax_mixture():
    L, x, Wg, W1, W3, W2, _ = small_layer(E=5, K=5, renorm=False)
    y, rt = oracle_forward(L, x, Wg, W1, W3, W2)
    lg = rt["logits"].astype(np.float64)
    p = scipy.special.softmax(lg, axis=1)
    for t in range(L.T):
        want = sum(p[t, e] * torch_swiglu(W1[e], W3[e], W2[e], x[t].astype(np.float64)) for e in range(L.E))
        np.testing.assert_allclose(y[t], want, rtol=1e-10, atol=1e-13)


def test_identical_experts_reproduce_single_expert():
    L, x, Wg, W1, W3, W2, _ = small_layer(K=3)
    W1[:] = W1[0]
    W3[:] = W3[0]
    W2[:] = W2[0]
    y, _ = oracle_forward(L, x, Wg, W1, W3, W2)
    for t in range(L.T):
        np.testing.assert_allclose(y[t], torch_swiglu(W1[0], W3[0], W2[0], x[t].astype(np.float64)), rtol=1e-12,
                                   atol=1e-14)


def test_shared_expert_and_residual_add():
    L, x, Wg, W1, W3, W2, Ws = small_layer(shared=1)
    y, rt = oracle_forward(L, x, Wg, W1, W3, W2, Ws)
    L0 = oracle.layer(L.T, L.d, L.F, L.E, L.K, renorm=True)
    y0 = oracle.forward_rows(L0, x, rt["idx"], rt["w"], rt["dest"], W1, W3, W2)
    for t in range(L.T):
        sh = torch_swiglu(Ws[0][0], Ws[1][0], Ws[2][0], x[t].astype(np.float64))
        np.testing.assert_allclose(y[t], y0[t] + sh, rtol=1e-12, atol=1e-14)
    Lr = oracle.layer(L.T, L.d, L.F, L.E, L.K, renorm=True, residual=True)
    yr = oracle.forward_rows(Lr, x, rt["idx"], rt["w"], rt["dest"], W1, W3, W2)
    np.testing.assert_allclose(yr, y0 + x.astype(np.float64), rtol=1e-14, atol=1e-15)


def test_dropped_tokens_pass_through():
    """Tech Daily §3.2: overflow tokens are dropped and their representation
    passes through on the residual."""
    L, x, Wg, W1, W3, W2, _ = small_layer(T=40, E=4, K=1, renorm=False)
    Lc = oracle.layer(L.T, L.d, L.F, L.E, 1, renorm=False, residual=True, capacity_factor=0.5)
    cap = oracle.capacity(Lc)
    assert cap == 5
    rt = oracle.route(Lc, x, Wg)
    y = oracle.forward_rows(Lc, x, rt["idx"], rt["w"], rt["dest"], W1, W3, W2)
    dropped = rt["dropped"].astype(bool)
    assert dropped.sum() == L.T - rt["offsets"][-1] > 0
    assert np.array_equal(y[dropped], x[dropped].astype(np.float64))
    Lz = oracle.layer(L.T, L.d, L.F, L.E, 1, renorm=False, capacity_factor=1e-9)
    rz = oracle.route(Lz, x, Wg)
    yz = oracle.forward_rows(Lz, x, rz["idx"], rz["w"], rz["dest"], W1, W3, W2)
    assert np.all(yz == 0)


def test_token_permutation_equivariance():
    L, x, Wg, W1, W3, W2, _ = small_layer(T=20)
    y, _ = oracle_forward(L, x, Wg, W1, W3, W2)
    perm = rng(12).permutation(L.T)
    yp, _ = oracle_forward(L, np.ascontiguousarray(x[perm]), Wg, W1, W3, W2)
    np.testing.assert_array_equal(yp, y[perm])


def test_forward_rows_subset_and_per_expert_pointers():
    L, x, Wg, W1, W3, W2, _ = small_layer(T=16)
    y, rt = oracle_forward(L, x, Wg, W1, W3, W2)
    toks = np.array([3, 0, 11], np.int64)
    used = set(rt["idx"][toks].reshape(-1).tolist())
    W1l = [W1[e] if e in used else None for e in range(L.E)]
    W3l = [W3[e] if e in used else None for e in range(L.E)]
    W2l = [W2[e] if e in used else None for e in range(L.E)]
    ys = oracle.forward_rows(L, x, rt["idx"], rt["w"], rt["dest"], W1l, W3l, W2l, tokens=toks)
    np.testing.assert_array_equal(ys, y[toks])


# ------------------------------------------------------------- expert choice --

def test_expert_choice_vs_brute_force():
    r = rng(13)
    T, E, cap = 40, 6, 9
    lg = r.standard_normal((T, E)).astype(np.float32)
    lg[5, 2] = lg[7, 2]  # an exact tie: the lower token wins
    L = oracle.layer(T, 4, 4, E, 1)
    tok, g = oracle.expert_choice(L, lg, cap)
    p = scipy.special.softmax(lg.astype(np.float64), axis=1)
    for e in range(E):
        order = sorted(range(T), key=lambda t: (-float(lg[t, e]), t))[:cap]
        assert tok[e].tolist() == order
        np.testing.assert_allclose(g[e], p[order, e], rtol=1e-14)


def test_combine_vs_direct_sum():
    r = rng(14)
    T, d, K, R = 30, 12, 3, 70
    yp = r.standard_normal((R, d)).astype(np.float32)
    w = r.uniform(0, 1, (T, K))
    dest = r.integers(-1, R, size=(T * K,)).astype(np.int32)
    sh = r.standard_normal((T, d)).astype(np.float32)
    x = r.standard_normal((T, d)).astype(np.float32)
    L = oracle.layer(T, d, 4, 8, K, residual=True)
    got = oracle.combine(L, yp, w, dest, sh, x)
    want = sh.astype(np.float64) + x
    for t in range(T):
        for k in range(K):
            if dest[t * K + k] >= 0:
                want[t] += w[t, k] * yp[dest[t * K + k]].astype(np.float64)
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-14)
    L0 = oracle.layer(T, d, 4, 8, K)
    assert np.all(oracle.combine(L0, yp, w, np.full(T * K, -1, np.int32)) == 0)


# ---------------------------------------------------------- router statistics --

def test_router_stats_vs_numpy():
    """[TD §4.2, §4.4, §9.1] definitions recomputed with numpy / scipy."""
    import scipy.stats
    r = rng(15)
    for gate, K in ((oracle.GATE_SOFTMAX, 2), (oracle.GATE_SIGMOID, 3)):
        T, E = 200, 12
        lg = (2 * r.standard_normal((T, E))).astype(np.float32)
        L = oracle.layer(T, 4, 4, E, K, gate=gate)
        idx, _, _ = oracle.select(L, lg)
        st = oracle.router_stats(L, lg, idx)
        l64 = lg.astype(np.float64)
        if gate == oracle.GATE_SOFTMAX:
            p = scipy.special.softmax(l64, axis=1)
        else:
            s = scipy.special.expit(l64)
            p = s / s.sum(1, keepdims=True)
        P = p.mean(0)
        f = np.bincount(idx.reshape(-1), minlength=E) / (T * K)
        np.testing.assert_allclose(st["P"], P, rtol=1e-12)
        assert abs(st["balance"] - E * np.sum(f * P)) < 1e-12
        assert abs(st["z_loss"] - np.mean(scipy.special.logsumexp(l64, axis=1) ** 2)) < 1e-10
        assert abs(st["lif"] - E * f.max()) < 1e-12
        assert abs(st["cv"] - f.std() / f.mean()) < 1e-12
        assert abs(st["entropy_p"] - scipy.stats.entropy(P)) < 1e-12
        assert abs(st["entropy_f"] - scipy.stats.entropy(f)) < 1e-12


def test_router_stats_balanced_optimum():
    """Equal logits: P_i = f_i = 1/N is the balanced optimum of the Switch
    loss ([TD §4.2]); the balance term is then exactly 1, LIF = 1, CV = 0 and
    both entropies are ln N."""
    T, E, K = 64, 8, 1
    lg = np.zeros((T, E), np.float32)
    L = oracle.layer(T, 4, 4, E, K)
    idx = (np.arange(T) % E).astype(np.int32).reshape(T, 1)  # a balanced assignment
    st = oracle.router_stats(L, lg, idx)
    np.testing.assert_allclose(st["P"], 1 / E, rtol=1e-15)
    assert abs(st["balance"] - 1) < 1e-14 and abs(st["lif"] - 1) < 1e-14 and abs(st["cv"]) < 1e-14
    assert abs(st["entropy_p"] - math.log(E)) < 1e-14 and abs(st["entropy_f"] - math.log(E)) < 1e-14
    assert abs(st["z_loss"] - math.log(E) ** 2) < 1e-12


# ------------------------------------------------------------ drop policies --

def _perm_consistent(L, idx_final, p):
    """dest / row_src / dropped / offsets agree with each other and rows of an
    expert lie in its offsets range."""
    N = L.T * L.K
    dest, rs, dr, off = p["dest"], p["row_src"], p["dropped"], p["offsets"]
    R = off[-1]
    assert np.array_equal(dr, (dest < 0).astype(np.uint8))
    kept = np.nonzero(dest >= 0)[0]
    assert len(kept) == R and np.array_equal(np.sort(dest[kept]), np.arange(R))
    assert np.array_equal(rs[dest[kept]], kept) and np.all(rs[R:N] == -1)
    e = idx_final.reshape(-1)[kept]
    assert np.all(dest[kept] >= off[e]) and np.all(dest[kept] < off[e + 1])


def test_select_ranked_brute_force():
    """Ranks = a stable sort of the keys (descending, ties to the lower
    expert); weights use the first K's normaliser."""
    r = rng(21)
    T, E, K = 40, 9, 2
    lg = np.round(r.standard_normal((T, E)), 1).astype(np.float32)  # many exact ties
    L = oracle.layer(T, 4, 4, E, K, renorm=True)
    idx, w = oracle.select_ranked(L, lg, E)
    p = scipy.special.softmax(lg.astype(np.float64), axis=1)
    for t in range(T):
        order = np.lexsort((np.arange(E), -lg[t].astype(np.float64)))
        assert np.array_equal(idx[t], order)
        np.testing.assert_allclose(w[t], p[t, order] / p[t, order[:K]].sum(), rtol=1e-13)
    i2, w2, _ = oracle.select(L, lg)
    assert np.array_equal(i2, idx[:, :K]) and np.allclose(w2, w[:, :K], rtol=0, atol=0)


def test_affinity_drop_golden():
    g = json.load(open(os.path.join(GOLDEN, "affinity_drop_small.json")))
    L = oracle.layer(g["T"], 4, 4, g["E"], g["K"], capacity_factor=g["capacity_factor"])
    assert oracle.capacity(L) == g["capacity"]
    p = oracle.permute_affinity(L, np.array(g["idx"], np.int32).reshape(-1, 1),
                                np.array(g["aff"], np.float32).reshape(-1, 1))
    for k, v in g["expect"].items():
        assert p[k].tolist() == v, k


def test_affinity_drop_invariants_and_special_cases():
    r = rng(22)
    T, E, K = 500, 8, 2
    lg = (r.standard_normal((T, E)) + np.linspace(0, 2, E)).astype(np.float32)
    L = oracle.layer(T, 4, 4, E, K, capacity_factor=0.9)
    cap = oracle.capacity(L)
    idx, w, _ = oracle.select(L, lg)
    aff = w.astype(np.float32)
    p = oracle.permute_affinity(L, idx, aff)
    _perm_consistent(L, idx, p)
    fi, a, dest = idx.reshape(-1), aff.reshape(-1), p["dest"]
    assert np.array_equal(p["counts"], np.bincount(fi, minlength=E))
    for e in range(E):
        fs = np.nonzero(fi == e)[0]
        kept, drop = fs[dest[fs] >= 0], fs[dest[fs] < 0]
        assert len(kept) == min(len(fs), cap)
        assert np.all(np.diff(dest[kept]) == 1)          # kept rows in flat order
        if len(drop):
            lo = a[kept].min()
            assert lo >= a[drop].max()
            tie = kept[a[kept] == lo]
            assert np.all(a[drop] < lo) or tie.max() < drop[a[drop] == lo].min()
    assert p["dropped"].sum() > 0
    # equal affinities: the first-come rule
    same = oracle.permute_affinity(L, idx, np.full_like(aff, 0.5))
    fc = oracle.permute(L, idx)
    for k in fc:
        assert np.array_equal(same[k], fc[k]), k
    # no capacity pressure: nothing dropped, the first-come permutation
    L2 = oracle.layer(T, 4, 4, E, K, capacity_factor=8.0)
    a2, f2 = oracle.permute_affinity(L2, idx, aff), oracle.permute(L2, idx)
    assert a2["dropped"].sum() == 0 and all(np.array_equal(a2[k], f2[k]) for k in f2)


def _reroute_logits(g):
    T, E = g["T"], g["E"]
    lg = np.zeros((T, E), np.float32)
    hot = [g["hot_tokens_stride"] * i for i in range(g["hot_tokens"])]
    j = 0
    for t in range(T):
        if t in hot:
            i = hot.index(t)
            lg[t, g["hot_expert"]] = 10.0
            lg[t, 1 + i % 5] = 5.0
        else:
            lg[t, 1 + j % 127] = 10.0
            lg[t, 1 + (j + 1) % 127] = 5.0
            j += 1
    return lg


def test_reroute_page_example():
    """[LN §3.2]: capacity 10 at C = 1.25, batch 1024, 128 experts; an expert
    chosen 15 times keeps 10 and its 5 excess tokens go to their next-best
    expert."""
    g = json.load(open(os.path.join(GOLDEN, "reroute_page_example.json")))
    L = oracle.layer(g["T"], 4, 4, g["E"], g["K"], renorm=False, capacity_factor=g["capacity_factor"])
    assert oracle.capacity(L) == g["capacity"]
    rt = oracle.route(L, None, None, policy="reroute", lg=_reroute_logits(g))
    ex = g["expect"]
    assert rt["counts"][g["hot_expert"]] == ex["counts_hot"]
    on_hot = np.nonzero((rt["idx"][:, 0] == g["hot_expert"]) & (rt["dest"] >= 0))[0]
    assert on_hot.tolist() == ex["kept_on_hot"]
    for t, e in ex["rerouted"].items():
        assert rt["idx"][int(t), 0] == e and rt["dest"][int(t)] >= 0
        assert rt["idx_first"][int(t), 0] == g["hot_expert"]
    assert int(rt["dropped"].sum()) == ex["dropped"]
    kept = np.bincount(rt["idx"][:, 0][rt["dest"] >= 0], minlength=g["E"])
    assert kept.max() <= g["capacity"]
    _perm_consistent(L, rt["idx"], rt)


def test_reroute_invariants_and_special_cases():
    r = rng(23)
    for K in (1, 2, 3):
        T, E = 400, 8
        lg = (r.standard_normal((T, E)) + np.linspace(0, 3, E)).astype(np.float32)
        L = oracle.layer(T, 4, 4, E, K, renorm=(K > 1), capacity_factor=1.0)
        cap = oracle.capacity(L)
        rt = oracle.route(L, None, None, policy="reroute", lg=lg)
        fc = oracle.route(L, None, None, policy="first_come", lg=lg)
        _perm_consistent(L, rt["idx"], rt)
        ranked, rw = oracle.select_ranked(L, lg, min(2 * K, E))
        first_kept = fc["dest"] >= 0
        # the first pass is the first-come rule
        assert np.array_equal(rt["counts"], fc["counts"])
        assert np.array_equal(rt["idx"].reshape(-1)[first_kept], fc["idx"].reshape(-1)[first_kept])
        assert np.all(rt["dest"][first_kept] >= 0)
        fin = rt["idx"].reshape(-1)
        kept_per = np.bincount(fin[rt["dest"] >= 0], minlength=E)
        assert kept_per.max() <= cap
        moved = np.nonzero(~first_kept)[0]
        assert len(moved) > 0
        for f in moved:
            t, k = divmod(f, K)
            j = int(np.sum(~first_kept[t * K:f]))          # earlier overflowing choices of t
            if K + j < min(2 * K, E):
                assert fin[f] == ranked[t, K + j] and rt["w"][t, k] == rw[t, K + j]
                if rt["dest"][f] < 0:
                    assert kept_per[fin[f]] == cap        # dropped only when the new expert is full
            else:
                assert rt["dest"][f] < 0 and fin[f] == fc["idx"].reshape(-1)[f]
        # flat-order priority among re-routed assignments of one expert
        for e in range(E):
            mv = moved[fin[moved] == e]
            k_ = mv[rt["dest"][mv] >= 0]
            d_ = mv[rt["dest"][mv] < 0]
            if len(k_) and len(d_):
                assert k_.max() < d_.min()
    # K == E: no alternates, so re-routing drops exactly what first-come drops
    L = oracle.layer(50, 4, 4, 3, 3, capacity_factor=0.5)
    lg = r.standard_normal((50, 3)).astype(np.float32)
    a, b = oracle.route(L, None, None, policy="reroute", lg=lg), oracle.route(L, None, None, lg=lg)
    for k in ("dest", "row_src", "dropped", "offsets", "idx"):
        assert np.array_equal(a[k], b[k]), k


def test_reroute_without_capacity_is_first_come():
    """With no capacity limit (capacity factor <= 0) nothing overflows, so
    re-routing moves nothing: the routing equals the first-come one [LN
    §3.2 re-routes only an expert's excess over its capacity], with offsets
    the exclusive scan of the demand and every assignment kept."""
    r = rng(25)
    for T, E, K, cf in ((6, 3, 1, 0.0), (300, 8, 2, 0.0), (120, 16, 3, -1.0), (64, 4, 4, 0.0)):
        L = oracle.layer(T, 4, 4, E, K, renorm=(K > 1), capacity_factor=cf)
        assert oracle.capacity(L) == -1
        lg = r.standard_normal((T, E)).astype(np.float32)
        a, b = oracle.route(L, None, None, policy="reroute", lg=lg), oracle.route(L, None, None, lg=lg)
        for k in ("idx", "w", "counts", "offsets", "dest", "row_src", "dropped"):
            assert np.array_equal(a[k], b[k]), (T, E, K, k)
        assert np.array_equal(a["offsets"], np.concatenate([[0], np.cumsum(np.bincount(b["idx"].reshape(-1),
                                                                                          minlength=E))]))
        assert not a["dropped"].any() and np.array_equal(np.sort(a["dest"]), np.arange(T * K))


def test_expert_choice_route_and_forward():
    """Expert choice in the K = E form: every expert holds exactly cap rows,
    rows list the chosen tokens in ascending order, and the layer output
    equals the direct sum over chosen (token, expert) pairs of g * E_e(x_t)
    [TD §3.3]; a token no expert chose gets zero (plus its shared expert)."""
    r = rng(24)
    T, d, F, E, K = 30, 8, 6, 5, 1
    L = oracle.layer(T, d, F, E, K, capacity_factor=1.4, n_shared=1, Fs=4)
    cap = oracle.ec_capacity(L)
    assert cap == int(np.floor(1.4 * T * K / E)) == 8
    assert oracle.ec_capacity(oracle.layer(T, d, F, E, 2)) == 12
    assert oracle.ec_capacity(oracle.layer(4, d, F, 2, 2, capacity_factor=9.0)) == 4   # at most T
    lg = r.standard_normal((T, E)).astype(np.float32)
    rt = oracle.route_expert_choice(L, lg=lg)
    dest = rt["dest"].reshape(T, E)
    for e in range(E):
        chosen = sorted(rt["tok"][e].tolist())
        assert np.nonzero(dest[:, e] >= 0)[0].tolist() == chosen
        assert dest[chosen, e].tolist() == list(range(e * cap, (e + 1) * cap))
    assert np.array_equal(rt["row_src"][dest[dest >= 0]], np.nonzero(rt["dest"] >= 0)[0])
    x = r.standard_normal((T, d)).astype(np.float32)
    W1, W3 = (r.standard_normal((E, F, d)).astype(np.float32) / 3 for _ in range(2))
    W2 = r.standard_normal((E, d, F)).astype(np.float32) / 3
    Ws1, Ws3 = (r.standard_normal((1, 4, d)).astype(np.float32) / 3 for _ in range(2))
    Ws2 = r.standard_normal((1, d, 4)).astype(np.float32) / 3
    y = oracle.forward_rows(oracle.ec_layer(L), x, rt["idx"], np.nan_to_num(rt["w"]), rt["dest"], W1, W3, W2,
                            Ws1, Ws3, Ws2)
    p = scipy.special.softmax(lg.astype(np.float64), axis=1)
    for t in range(T):
        want = torch_swiglu(Ws1[0], Ws3[0], Ws2[0], x[t].astype(np.float64))
        for e in range(E):
            if dest[t, e] >= 0:
                want = want + p[t, e] * torch_swiglu(W1[e], W3[e], W2[e], x[t].astype(np.float64))
        np.testing.assert_allclose(y[t], want, rtol=1e-12, atol=1e-13)
    assert (dest < 0).all(1).any()          # some token was chosen by no expert


# ---------------------------------------------------------- FP8 E4M3 weights --

def test_fp8_e4m3_decode():
    """Every code against torch's float8_e4m3fn, plus the format's landmarks."""
    codes = torch.arange(256, dtype=torch.uint8)
    want = codes.view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.fp8_e4m3(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(want)) and np.array_equal(got[~np.isnan(got)], want[~np.isnan(want)])
    assert oracle.fp8_e4m3(0x38) == 1.0 and oracle.fp8_e4m3(0x7E) == 448.0 and oracle.fp8_e4m3(0xFE) == -448.0
    assert oracle.fp8_e4m3(0x01) == 2.0 ** -9 and oracle.fp8_e4m3(0x08) == 2.0 ** -6
    assert np.isnan(oracle.fp8_e4m3(0x7F)) and np.isnan(oracle.fp8_e4m3(0xFF))


def _fp8_values(codes, scale_rows):
    return codes_to_f64(codes) * scale_rows.astype(np.float64)[..., None]


def codes_to_f64(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def test_swiglu_fp8_vs_torch():
    """Weight = decoded code * row scale, then the SwiGLU expert (torch on the
    dequantised weights)."""
    r = rng(33)
    d, F = 48, 80
    codes = [moe_synth.fp8_codes(7, t, s) for t, s in ((2, (F, d)), (3, (F, d)), (4, (d, F)))]
    sc = [r.uniform(0.01, 0.05, n).astype(np.float32) for n in (F, F, d)]
    x = r.standard_normal(d)
    want = torch_swiglu(*(_fp8_values(c, s) for c, s in zip(codes, sc)), x)
    got = oracle.swiglu(*codes, x, bf16=True, scales=sc)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_forward_rows_fp8_layer():
    """A whole FP8-weight layer (routed + shared expert) against the same
    layer with the dequantised weights given as fp32 (exact when the product
    code * scale is representable in fp32, which holds for these scales: 3
    mantissa bits times an fp32 value with few significant bits)."""
    r = rng(34)
    T, d, F, E, K, Fs = 12, 16, 8, 4, 2, 8
    wl = moe_synth.workload("mixtral_prefill", T=T, d=d, F=F, E=E, K=K, n_shared=1, Fs=Fs, wdtype="fp8")
    h = wl.gen_all()
    # scales with 8 significant bits: every code * scale is exact in fp32
    for k in ("S1", "S3", "S2", "Ss1", "Ss3", "Ss2"):
        h[k] = (np.round(h[k] * 2.0 ** 14) / 2.0 ** 14).astype(np.float32)
    assert oracle.layer_of(wl).w_fp8 == 1
    x = r.standard_normal((T, d)).astype(np.float32)
    L8 = oracle.layer(T, d, F, E, K, n_shared=1, Fs=Fs, w_fp8=True)
    rt = oracle.route(L8, x, h["Wg"])
    y8 = oracle.forward_rows(L8, x, rt["idx"], rt["w"], rt["dest"], h["W1"], h["W3"], h["W2"], h["Ws1"], h["Ws3"],
                             h["Ws2"], **{k: h[k] for k in ("S1", "S3", "S2", "Ss1", "Ss3", "Ss2")})
    deq = lambda c, s: _fp8_values(c, s).astype(np.float32)
    W1f = np.stack([deq(h["W1"][e], h["S1"][e]) for e in range(E)])
    W3f = np.stack([deq(h["W3"][e], h["S3"][e]) for e in range(E)])
    W2f = np.stack([deq(h["W2"][e], h["S2"][e]) for e in range(E)])
    Ws = [deq(h[a][0], h[b][0])[None] for a, b in (("Ws1", "Ss1"), ("Ws3", "Ss3"), ("Ws2", "Ss2"))]
    assert np.array_equal(W1f.astype(np.float64), np.stack([_fp8_values(h["W1"][e], h["S1"][e]) for e in range(E)]))
    Lf = oracle.layer(T, d, F, E, K, n_shared=1, Fs=Fs)
    yf = oracle.forward_rows(Lf, x, rt["idx"], rt["w"], rt["dest"], W1f, W3f, W2f, *Ws)
    np.testing.assert_allclose(y8, yf, rtol=1e-13, atol=1e-13)
