"""Pins for the CPU oracle, each against something other than the oracle.

Kinds of pin used here: the format's published value tables (golden file),
library routines on an independent code path (numpy / torch float64),
brute force (dense evaluation of every expert with a routing mask, Python
sorted() for the grouping), closed forms, and invariants the method's
definition implies.  A plausible slip in oracle.c (dropped term, wrong sign,
swapped nibble, transposed operand, wrong tie-break, missing eps) fails at
least one test below.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_gemm_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _formats():
    with open(os.path.join(GOLD, "mxfp4_formats.json")) as f:
        return json.load(f)


def _decode_independent(codes: np.ndarray, scales: np.ndarray, K: int) -> np.ndarray:
    """Decode MXFP4 rows with the golden value table and math.ldexp (not oracle.c)."""
    fm = _formats()
    table = np.array([fm["e2m1"][str(c)] for c in range(16)], dtype=np.float64)
    codes = codes.reshape(-1, K // 2)
    lo = codes & 15
    hi = codes >> 4
    el = np.empty((codes.shape[0], K), dtype=np.int64)
    el[:, 0::2] = lo
    el[:, 1::2] = hi
    sc = scales.reshape(-1, K // 32).astype(np.int64)
    mult = np.array([math.ldexp(1.0, int(s) - 127) for s in range(255)] + [np.nan])
    return table[el] * np.repeat(mult[sc], 32, axis=1)


# ---------------------------------------------------------------- formats

def test_e2m1_table_matches_format():
    fm = _formats()
    for c in range(16):
        v = oracle.e2m1(c)
        want = fm["e2m1"][str(c)]
        assert v == want and math.copysign(1, v) == math.copysign(1, want), c


def test_e8m0_matches_format():
    fm = _formats()
    for s, want in fm["e8m0_examples"].items():
        assert oracle.e8m0(int(s)) == want
    assert math.isnan(oracle.e8m0(fm["e8m0_nan"]))
    for s in range(255):
        assert oracle.e8m0(s) == math.ldexp(1.0, s - 127)


def test_dequant_exhaustive_codes_and_scales():
    # one 32-element row per scale byte; element i holds code i % 16
    K = 32
    codes = np.array([(((2 * b + 1) % 16) << 4) | ((2 * b) % 16) for b in range(K // 2)], np.uint8)
    rows = np.tile(codes, 255)
    scales = np.arange(255, dtype=np.uint8)
    got = oracle.dequant_rows(rows, scales, K)
    fm = _formats()
    for s in range(255):
        for i in range(K):
            want = fm["e2m1"][str(i % 16)] * math.ldexp(1.0, s - 127)
            assert got[s, i] == want, (s, i)


def test_dequant_nibble_order_and_block_scale():
    # element 0 = +6 (code 7, low nibble), element 1 = -0.5 (code 9, high nibble);
    # second block scaled differently from the first
    K = 64
    row = np.zeros(K // 2, np.uint8)
    row[0] = (9 << 4) | 7
    row[16] = (2 << 4) | 4          # elements 32 (2.0) and 33 (1.0)
    sc = np.array([127, 129], np.uint8)
    got = oracle.dequant_rows(row, sc, K)[0]
    assert got[0] == 6.0 and got[1] == -0.5
    assert got[32] == 8.0 and got[33] == 4.0
    assert np.all(got[2:32] == 0) and np.all(got[34:] == 0)


def test_dequant_random_rows_vs_independent_decode():
    rng = np.random.default_rng(5)
    K = 256
    codes = rng.integers(0, 256, size=(7, K // 2), dtype=np.uint8)
    scales = rng.integers(100, 150, size=(7, K // 32), dtype=np.uint8)
    np.testing.assert_array_equal(oracle.dequant_rows(codes, scales, K),
                                  _decode_independent(codes, scales, K))


def test_bf16_rounding_cases():
    # exact ties between neighbouring bf16 values go to the even mantissa
    assert oracle.double_to_bf16(1.0) == 0x3F80
    assert oracle.double_to_bf16(1.0 + 2.0 ** -8) == 0x3F80         # tie -> even (1.0)
    assert oracle.double_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82     # tie -> even (1+2^-6)
    assert oracle.double_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81
    assert oracle.double_to_bf16(-2.5) == 0xC020
    assert oracle.double_to_bf16(0.0) == 0 and oracle.double_to_bf16(-0.0) == 0x8000
    # agrees with an independent fp32 route on values that are exact in fp32
    rng = np.random.default_rng(1)
    v = rng.standard_normal(2000).astype(np.float32)
    np.testing.assert_array_equal(oracle.doubles_to_bf16(v.astype(np.float64)), synth.f32_to_bf16_bits(v))
    for b in [0x0001, 0x3F80, 0xC2F7, 0x7F7F, 0x0080]:
        assert oracle.double_to_bf16(oracle.bf16_to_double(b)) == b


# ---------------------------------------------------------------- router

def _tiny():
    return synth.make_layer("tiny")


def test_router_scores_vs_numpy_float64():
    L = _tiny()
    got = oracle.router_scores(L.x, L.router_w)
    ref = (synth.bf16_bits_to_f32(L.x).astype(np.float64) @ L.router_w.astype(np.float64).T)
    np.testing.assert_allclose(got.astype(np.float64), ref, rtol=2e-7, atol=1e-9)
    assert got.dtype == np.float32
    # full width: 2 tokens of the decode workload
    w = synth.WORKLOADS["decode4"]
    wr = synth.make_router(w)
    x = synth.make_tokens(w, wr)[:2]
    got = oracle.router_scores(x, wr)
    ref = synth.bf16_bits_to_f32(x).astype(np.float64) @ wr.astype(np.float64).T
    np.testing.assert_allclose(got.astype(np.float64), ref, rtol=2e-7, atol=1e-7)


def test_topk_equals_stable_full_sort():
    rng = np.random.default_rng(2)
    sc = rng.standard_normal((50, 40)).astype(np.float32)
    sc[3, [4, 9, 17]] = 5.0          # three-way tie at the top: ids ascending
    sc[7, :] = 0.25                  # everything tied
    for k in (1, 3, 8, 40):
        ids, _ = oracle.topk_softmax(sc, k)
        ref = np.argsort(-sc.astype(np.float64), axis=1, kind="stable")[:, :k]
        np.testing.assert_array_equal(ids, ref)
    ids, _ = oracle.topk_softmax(sc, 3)
    assert list(ids[3]) == [4, 9, 17]
    assert list(ids[7]) == [0, 1, 2]


def test_weights_softmax_properties():
    rng = np.random.default_rng(3)
    sc = (rng.standard_normal((200, 64)) * 2).astype(np.float32)
    for k in (1, 2, 5, 8):
        ids, w = oracle.topk_softmax(sc, k)
        assert np.all(np.abs(w.sum(1) - 1) <= 1e-12)
        assert np.all(w > 0)
        assert np.all(np.diff(w, axis=1) <= 0)
        picked = np.take_along_axis(sc, ids, axis=1).astype(np.float64)
        ref = torch.softmax(torch.from_numpy(picked), dim=1).numpy()
        np.testing.assert_allclose(w, ref, rtol=1e-13, atol=1e-15)
        if k == 1:
            assert np.all(w == 1.0)
        if k == 2:
            l0, l1 = picked[:, 0], picked[:, 1]
            np.testing.assert_allclose(w[:, 0], 1.0 / (1.0 + np.exp(l1 - l0)), rtol=1e-14)


# ---------------------------------------------------------------- grouping

def test_group_bruteforce_sorted():
    rng = np.random.default_rng(4)
    T, E, k = 97, 13, 4
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, inv = oracle.group(ids, E)
    slots = sorted(range(T * k), key=lambda s: (int(ids[s // k, s % k]), s // k))
    assert list(perm) == slots
    assert sorted(perm) == list(range(T * k))
    assert np.all(inv[perm] == np.arange(T * k))
    np.testing.assert_array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(ids.ravel()[seg] == e)
        assert np.all(np.diff(seg // k) > 0)


def test_group_degenerate():
    # every token to the same experts; empty experts keep zero-length segments
    T, E, k = 5, 6, 2
    ids = np.tile(np.array([[4, 1]], np.int32), (T, 1))
    counts, offsets, perm, inv = oracle.group(ids, E)
    assert list(counts) == [0, 5, 0, 0, 5, 0]
    assert list(offsets) == [0, 0, 5, 5, 5, 10, 10]
    assert list(perm) == [1, 3, 5, 7, 9, 0, 2, 4, 6, 8]


# ---------------------------------------------------------------- expert FFN

def _torch_dense_expert(Wg, Wu, Wd, X, eps):
    """Library path: SwiGLU MLP then RMSNorm, float64."""
    G = X @ Wg.T
    U = X @ Wu.T
    O = (torch.nn.functional.silu(G) * U) @ Wd.T
    N = torch.nn.functional.rms_norm(O, (O.shape[-1],), eps=eps)
    return O, N


def _split_expert(L, e):
    s = L.shape
    d, F = s.d, s.F
    wb = L.w_packed[e]
    sb = L.scales[e]
    g = _decode_independent(wb[: F * d // 2], sb[: F * d // 32], d)
    u = _decode_independent(wb[F * d // 2: F * d], sb[F * d // 32: F * d // 16], d)
    dn = _decode_independent(wb[F * d:], sb[F * d // 16:], F)
    return torch.from_numpy(g), torch.from_numpy(u), torch.from_numpy(dn)


def test_single_expert_is_dense_swiglu_rmsnorm():
    """E = k = 1, alpha = 0, beta = 1: the layer is one dense SwiGLU MLP + RMSNorm."""
    w = synth.custom_workload(T=9, d=128, E=1, k=1, F=96, seed=11)
    L = synth.make_layer(w, gap=0)
    zero = np.zeros(128, np.float32)
    one = np.ones(128, np.float32)
    s, ids, wt = oracle.moe_forward(L.x, L.router_w, L.w_packed, L.scales, zero, one, 1)
    assert np.all(ids == 0) and np.all(wt == 1.0)
    Wg, Wu, Wd = _split_expert(L, 0)
    X = torch.from_numpy(synth.bf16_bits_to_f32(L.x).astype(np.float64))
    _, N = _torch_dense_expert(Wg, Wu, Wd, X, 1e-6)
    np.testing.assert_allclose(s, N.numpy(), rtol=1e-12, atol=1e-12)


def test_expert_outputs_vs_torch():
    L = _tiny()
    s = L.shape
    Wg, Wu, Wd = _split_expert(L, 3)
    X = torch.from_numpy(synth.bf16_bits_to_f32(L.x[:5]).astype(np.float64))
    O, N = _torch_dense_expert(Wg, Wu, Wd, X, 1e-6)
    for t in range(5):
        o, n, ms = oracle.expert(L.w_packed[3], L.scales[3], X[t].numpy(), s.d, s.F)
        np.testing.assert_allclose(o, O[t].numpy(), rtol=1e-11, atol=1e-9)
        np.testing.assert_allclose(n, N[t].numpy(), rtol=1e-11, atol=1e-12)
        assert abs(ms - float((O[t] ** 2).mean())) <= 1e-10 * ms


def test_rmsnorm_closed_form():
    L = _tiny()
    s = L.shape
    x = synth.bf16_bits_to_f32(L.x[0]).astype(np.float64)
    for eps in (1e-6, 1.0, 1e3):
        o, n, ms = oracle.expert(L.w_packed[1], L.scales[1], x, s.d, s.F, eps)
        assert abs(ms - np.mean(o ** 2)) <= 1e-12 * ms
        assert abs(np.mean(n ** 2) - ms / (ms + eps)) <= 1e-12


# ---------------------------------------------------------------- whole layer

def _dense_bruteforce(L):
    """Every expert on every token, then a routing mask (independent of oracle.c)."""
    s = L.shape
    X = torch.from_numpy(synth.bf16_bits_to_f32(L.x).astype(np.float64))
    scores = (X @ torch.from_numpy(L.router_w.astype(np.float64)).T).to(torch.float32)
    order = np.argsort(-scores.numpy().astype(np.float64), axis=1, kind="stable")[:, : s.k]
    picked = torch.gather(scores.to(torch.float64), 1, torch.from_numpy(order))
    wts = torch.softmax(picked, dim=1)
    mask = torch.zeros(s.T, s.E, dtype=torch.float64)
    mask.scatter_(1, torch.from_numpy(order), wts)
    Y = torch.zeros(s.T, s.d, dtype=torch.float64)
    for e in range(s.E):
        Wg, Wu, Wd = _split_expert(L, e)
        _, N = _torch_dense_expert(Wg, Wu, Wd, X, L.eps)
        Y += mask[:, e:e + 1] * N
    S = torch.from_numpy(L.alpha.astype(np.float64)) * X + torch.from_numpy(L.beta.astype(np.float64)) * Y
    return S.numpy(), order


def test_layer_equals_dense_bruteforce():
    L = _tiny()
    s, ids, _ = oracle.moe_forward(L.x, L.router_w, L.w_packed, L.scales, L.alpha, L.beta, L.k)
    ref, order = _dense_bruteforce(L)
    np.testing.assert_array_equal(ids, order)
    err = np.abs(s - ref).max() / np.abs(ref).max()
    assert err <= 1e-12, err


def test_layer_token_subset_and_permutation():
    L = _tiny()
    full, ids, w = oracle.moe_forward(L.x, L.router_w, L.w_packed, L.scales, L.alpha, L.beta, L.k)
    sel = np.array([5, 0, 63, 17], np.int32)
    sub, ids2, w2 = oracle.moe_forward(L.x, L.router_w, L.w_packed, L.scales, L.alpha, L.beta, L.k,
                                       tokens=sel)
    np.testing.assert_array_equal(sub, full[sel])
    np.testing.assert_array_equal(ids2, ids[sel])
    p = np.random.default_rng(0).permutation(L.shape.T)
    permd, _, _ = oracle.moe_forward(L.x[p], L.router_w, L.w_packed, L.scales, L.alpha, L.beta, L.k)
    np.testing.assert_array_equal(permd, full[p])


def test_layer_expert_relabelling_invariance():
    L = _tiny()
    full, ids, _ = oracle.moe_forward(L.x, L.router_w, L.w_packed, L.scales, L.alpha, L.beta, L.k)
    q = np.array([3, 7, 0, 5, 1, 6, 2, 4])
    s2, ids2, _ = oracle.moe_forward(L.x, L.router_w[q], L.w_packed[q], L.scales[q], L.alpha, L.beta, L.k)
    np.testing.assert_array_equal(q[ids2], ids)
    np.testing.assert_allclose(s2, full, rtol=0, atol=1e-13)


def test_gate_special_cases():
    L = _tiny()
    d = L.shape.d
    one = np.ones(d, np.float32)
    zero = np.zeros(d, np.float32)
    s, _, _ = oracle.moe_forward(L.x, L.router_w, L.w_packed, L.scales, one, zero, L.k)
    np.testing.assert_array_equal(s, synth.bf16_bits_to_f32(L.x).astype(np.float64))
    s, _, _ = oracle.moe_forward(L.x, L.router_w, L.w_packed, L.scales, zero, one, L.k)
    # convex combination of unit-RMS (less eps) vectors
    assert np.all(np.sqrt(np.mean(s ** 2, axis=1)) <= 1.0 + 1e-12)
    assert np.all(np.sqrt(np.mean(s ** 2, axis=1)) > 0.3)


def test_scale_invariance_of_expert_norm():
    """+1 on an expert's E8M0 bytes for down (or up) rows doubles o; RMSNorm removes it."""
    L = _tiny()
    d, F = L.shape.d, L.shape.F
    fw = lambda sc, eps: oracle.moe_forward(L.x, L.router_w, L.w_packed, sc, L.alpha, L.beta, L.k,
                                            eps=eps)[0]
    s0 = fw(L.scales, 1e-6)
    z0 = fw(L.scales, 0.0)
    for lo, hi in ((F * d // 16, 3 * d * F // 32), (F * d // 32, F * d // 16)):
        sc = L.scales.copy()
        sc[2, lo:hi] += 1
        # eps = 0: doubling is exact in binary floating point, so bit-identical
        np.testing.assert_array_equal(fw(sc, 0.0), z0)
        # eps > 0: n moves by at most 3/8 * eps / ms relative (ms >= 0.1 here)
        np.testing.assert_allclose(fw(sc, 1e-6), s0, rtol=0, atol=1e-5)
    # while the gate rows are not scale-free: the layer output must move
    sc = L.scales.copy()
    sc[2, : F * d // 32] += 1
    s2, _, _ = oracle.moe_forward(L.x, L.router_w, L.w_packed, sc, L.alpha, L.beta, L.k)
    assert np.abs(s2 - s0).max() > 1e-3


def test_eps_inside_sqrt():
    """A huge eps shrinks every normalised expert output toward zero."""
    L = _tiny()
    d = L.shape.d
    zero = np.zeros(d, np.float32)
    one = np.ones(d, np.float32)
    s_small, _, _ = oracle.moe_forward(L.x, L.router_w, L.w_packed, L.scales, zero, one, L.k, eps=1e-6)
    s_big, _, _ = oracle.moe_forward(L.x, L.router_w, L.w_packed, L.scales, zero, one, L.k, eps=1e12)
    assert np.abs(s_big).max() < 1e-3 * np.abs(s_small).max()


# ------------------------------------------------- latent-width variant (L1-L5)

def _latent_experts_view(L):
    """The experts of a latent layer in the shape _split_expert expects (width d)."""
    from types import SimpleNamespace
    return SimpleNamespace(shape=SimpleNamespace(d=L.w.d, F=L.w.F), w_packed=L.w_packed,
                           scales=L.scales)


def test_latent_equals_dense_bruteforce():
    """torch float64 matmuls for the two shared matrices, every expert on every
    token (golden-table decode), a routing mask on the full-width scores."""
    L = synth.make_latent_layer("latent_tiny")
    w = L.w
    s, ids, _ = oracle.latent_forward(L.x, L.router_w, L.wc, L.w_packed, L.scales, L.we, L.alpha,
                                      L.beta, w.k)
    f64 = lambda b: torch.from_numpy(synth.bf16_bits_to_f32(b).astype(np.float64))
    X, Wc, We = f64(L.x), f64(L.wc), f64(L.we)
    scores = (X @ torch.from_numpy(L.router_w.astype(np.float64)).T).to(torch.float32)
    order = np.argsort(-scores.numpy().astype(np.float64), axis=1, kind="stable")[:, : w.k]
    wts = torch.softmax(torch.gather(scores.to(torch.float64), 1, torch.from_numpy(order)), dim=1)
    mask = torch.zeros(w.T, w.E, dtype=torch.float64)
    mask.scatter_(1, torch.from_numpy(order), wts)
    Z = X @ Wc.T
    V = _latent_experts_view(L)
    Y = torch.zeros(w.T, w.d, dtype=torch.float64)
    for e in range(w.E):
        Wg, Wu, Wd = _split_expert(V, e)
        _, N = _torch_dense_expert(Wg, Wu, Wd, Z, L.eps)
        Y += mask[:, e:e + 1] * N
    ref = torch.from_numpy(L.alpha.astype(np.float64)) * X + \
        torch.from_numpy(L.beta.astype(np.float64)) * (Y @ We.T)
    np.testing.assert_array_equal(ids, order)
    err = np.abs(s - ref.numpy()).max() / np.abs(ref.numpy()).max()
    assert err <= 1e-12, err


def test_latent_with_selection_matrices_is_the_full_width_layer():
    """Wc picks d of the D input channels in a scrambled order, We puts the d
    sums on d scrambled output channels and the router ignores the other
    channels: the variant is then the full-width layer (O1-O8) at width d on
    the picked channels, plus alpha * x on every channel.  A transposed shared
    matrix or a swapped width moves values to the wrong channels."""
    L = synth.make_latent_layer("latent_tiny")
    w = L.w
    rng = np.random.default_rng(5)
    pick = rng.permutation(w.D)[: w.d]   # latent j reads input channel pick[j]
    put = rng.permutation(w.D)[: w.d]    # latent j lands on output channel put[j]
    one = np.uint16(0x3F80)
    wc = np.zeros((w.d, w.D), np.uint16)
    wc[np.arange(w.d), pick] = one
    we = np.zeros((w.D, w.d), np.uint16)
    we[put, np.arange(w.d)] = one
    wr = np.zeros_like(L.router_w)
    wr[:, pick] = L.router_w[:, pick]
    s, ids, wt = oracle.latent_forward(L.x, wr, wc, L.w_packed, L.scales, we, L.alpha, L.beta, w.k)
    y, ids2, wt2 = oracle.moe_forward(np.ascontiguousarray(L.x[:, pick]),
                                      np.ascontiguousarray(wr[:, pick]), L.w_packed, L.scales,
                                      np.zeros(w.d, np.float32), np.ones(w.d, np.float32), w.k)
    np.testing.assert_array_equal(ids, ids2)
    np.testing.assert_array_equal(wt, wt2)
    expect = L.alpha.astype(np.float64) * synth.bf16_bits_to_f32(L.x).astype(np.float64)
    expect[:, put] += L.beta[put].astype(np.float64) * y
    np.testing.assert_allclose(s, expect, rtol=1e-13, atol=1e-13)


def test_latent_token_subset():
    L = synth.make_latent_layer("latent_tiny")
    full, ids, _ = oracle.latent_forward(L.x, L.router_w, L.wc, L.w_packed, L.scales, L.we,
                                         L.alpha, L.beta, L.w.k)
    sel = np.array([9, 0, 63], np.int32)
    sub, ids2, _ = oracle.latent_forward(L.x, L.router_w, L.wc, L.w_packed, L.scales, L.we,
                                         L.alpha, L.beta, L.w.k, tokens=sel)
    np.testing.assert_array_equal(sub, full[sel])
    np.testing.assert_array_equal(ids2, ids[sel])


# ------------------------------------------------- block with stream norms (B1-B3)

def _block_inputs(name="tiny"):
    L = synth.make_layer(name)
    g_pre, g_post = synth.make_norm_gains(synth.WORKLOADS[name])
    return L, g_pre, g_post


def test_block_is_norm_layer_norm_composition():
    """torch float64 rms_norm for both stream norms, the pinned bf16 rounding
    and the pinned full-width layer (alpha = 0, beta = 1 gives y) between them."""
    L, g_pre, g_post = _block_inputs()
    s, ids, w = oracle.block_forward(L.x, g_pre, L.router_w, L.w_packed, L.scales, g_post, L.alpha,
                                     L.beta, L.k)
    X = torch.from_numpy(synth.bf16_bits_to_f32(L.x).astype(np.float64))
    Xn = torch.nn.functional.rms_norm(X, (X.shape[-1],), eps=L.eps) * \
        torch.from_numpy(g_pre.astype(np.float64))
    xn_bits = oracle.doubles_to_bf16(Xn.numpy())
    d = L.shape.d
    y, ids2, w2 = oracle.moe_forward(xn_bits, L.router_w, L.w_packed, L.scales,
                                     np.zeros(d, np.float32), np.ones(d, np.float32), L.k)
    np.testing.assert_array_equal(ids, ids2)
    Y = torch.from_numpy(y)
    P = torch.nn.functional.rms_norm(Y, (d,), eps=L.eps) * torch.from_numpy(g_post.astype(np.float64))
    ref = torch.from_numpy(L.alpha.astype(np.float64)) * X + torch.from_numpy(L.beta.astype(np.float64)) * P
    err = np.abs(s - ref.numpy()).max() / np.abs(ref.numpy()).max()
    assert err <= 1e-12, err


def test_block_stream_scale_invariance():
    """With eps = 0 both norms remove the scale of the stream: doubling s (exact
    in bf16) leaves the block's contribution unchanged, so s_out moves by
    exactly alpha * s.  A dropped or misplaced pre-norm fails this."""
    L, g_pre, g_post = _block_inputs()
    s1, ids1, _ = oracle.block_forward(L.x, g_pre, L.router_w, L.w_packed, L.scales, g_post,
                                       L.alpha, L.beta, L.k, eps=0.0)
    x2 = synth.f32_to_bf16_bits(2.0 * synth.bf16_bits_to_f32(L.x))
    s2, ids2, _ = oracle.block_forward(x2, g_pre, L.router_w, L.w_packed, L.scales, g_post,
                                       L.alpha, L.beta, L.k, eps=0.0)
    np.testing.assert_array_equal(ids1, ids2)
    ax = L.alpha.astype(np.float64) * synth.bf16_bits_to_f32(L.x).astype(np.float64)
    np.testing.assert_allclose(s2 - s1, ax, rtol=0, atol=1e-12)


def test_block_post_gain_linearity():
    """The block's contribution is linear in the post-norm gain (doubling is
    exact in fp32)."""
    L, g_pre, g_post = _block_inputs()
    ax = L.alpha.astype(np.float64) * synth.bf16_bits_to_f32(L.x).astype(np.float64)
    s1, _, _ = oracle.block_forward(L.x, g_pre, L.router_w, L.w_packed, L.scales, g_post, L.alpha,
                                    L.beta, L.k)
    s3, _, _ = oracle.block_forward(L.x, g_pre, L.router_w, L.w_packed, L.scales,
                                    (2.0 * g_post).astype(np.float32), L.alpha, L.beta, L.k)
    np.testing.assert_allclose(s3 - ax, 2.0 * (s1 - ax), rtol=1e-12, atol=1e-12)


def test_block_token_subset():
    L, g_pre, g_post = _block_inputs()
    full, ids, _ = oracle.block_forward(L.x, g_pre, L.router_w, L.w_packed, L.scales, g_post,
                                        L.alpha, L.beta, L.k)
    sel = np.array([7, 0, 63, 31], np.int32)
    sub, ids2, _ = oracle.block_forward(L.x, g_pre, L.router_w, L.w_packed, L.scales, g_post,
                                        L.alpha, L.beta, L.k, tokens=sel)
    np.testing.assert_array_equal(sub, full[sel])
    np.testing.assert_array_equal(ids2, ids[sel])


def test_block_prenorm_is_rms_norm_rounded():
    """B1 alone: torch float64 rms_norm times the gain, rounded by the pinned
    bf16 rounding, bit for bit."""
    L, g_pre, _ = _block_inputs()
    xn = oracle.block_prenorm(L.x, g_pre, eps=L.eps)
    X = torch.from_numpy(synth.bf16_bits_to_f32(L.x).astype(np.float64))
    Xn = torch.nn.functional.rms_norm(X, (X.shape[-1],), eps=L.eps) * \
        torch.from_numpy(g_pre.astype(np.float64))
    np.testing.assert_array_equal(xn, oracle.doubles_to_bf16(Xn.numpy()))
    sel = np.array([5, 0, 40], np.int32)
    np.testing.assert_array_equal(oracle.block_prenorm(L.x, g_pre, eps=L.eps, tokens=sel), xn[sel])


def test_block_given_normalised_rows():
    """B2-B3 on given normalised rows: B1's own rows give the same result bit
    for bit; other rows (B1's doubled, exact in bf16) give the composition of
    the pinned layer on those rows (alpha = 0, beta = 1 gives y) with torch
    float64 rms_norm, while the residual still takes the stream s."""
    L, g_pre, g_post = _block_inputs()
    sel = np.array([3, 17, 60], np.int32)
    ref, ids, _ = oracle.block_forward(L.x, g_pre, L.router_w, L.w_packed, L.scales, g_post,
                                       L.alpha, L.beta, L.k, tokens=sel)
    xn = oracle.block_prenorm(L.x, g_pre, eps=L.eps, tokens=sel)
    got, ids2, _ = oracle.block_forward(L.x, g_pre, L.router_w, L.w_packed, L.scales, g_post,
                                        L.alpha, L.beta, L.k, tokens=sel, xn=xn)
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(ids2, ids)
    xn2 = synth.f32_to_bf16_bits(2.0 * synth.bf16_bits_to_f32(xn))
    s2, _, _ = oracle.block_forward(L.x, g_pre, L.router_w, L.w_packed, L.scales, g_post,
                                    L.alpha, L.beta, L.k, tokens=sel, xn=xn2)
    d = L.shape.d
    y, _, _ = oracle.moe_forward(xn2, L.router_w, L.w_packed, L.scales, np.zeros(d, np.float32),
                                 np.ones(d, np.float32), L.k)
    P = torch.nn.functional.rms_norm(torch.from_numpy(y), (d,), eps=L.eps) * \
        torch.from_numpy(g_post.astype(np.float64))
    X = synth.bf16_bits_to_f32(L.x[sel]).astype(np.float64)
    want = L.alpha.astype(np.float64) * X + L.beta.astype(np.float64) * P.numpy()
    assert np.abs(s2 - want).max() / np.abs(want).max() <= 1e-12
    assert np.abs(s2 - ref).max() > 1e-3  # the given rows are the ones used
