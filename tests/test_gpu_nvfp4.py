"""GPU parity of the 16-block weight format (one E4M3 scale per 16 values,
fp32 matrix scales) against the CPU oracle, through the C ABI.

Same bar as the MXFP4 layer: routing bit for bit, weights to 1e-5, s_out
within rel_max 2e-2 / normwise 5e-3 (tests/helpers.py).  The generator puts
subnormal, zero and negative scale bytes in every workload.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_gemm_amd import synth

from helpers import (WEIGHT_TOL, assert_close, bf16_bits, parity_tokens, run_nv, upload_nv,
                     weight_tol)

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-case]", *a, flush=True)


def _check_routing(L, dbg, label):
    r = oracle.route(L.x, L.router_w, L.k)
    np.testing.assert_array_equal(dbg["ids"], r["ids"], err_msg=label)
    np.testing.assert_array_equal(dbg["offsets"], r["offsets"], err_msg=label)
    np.testing.assert_array_equal(dbg["perm"], r["perm"], err_msg=label)
    np.testing.assert_array_equal(dbg["inv"], r["inv"], err_msg=label)
    assert np.all(np.abs(dbg["weights"] - r["w"]) <= weight_tol(L.x)), label
    return r


def _check_tokens(L, out_bits, tokens, label):
    ref, _, _ = oracle.moe_forward_nv(L.x, L.router_w, L.w_packed, L.scales16, L.gscale, L.alpha,
                                      L.beta, L.k, eps=L.eps, tokens=np.asarray(tokens, np.int32))
    got = synth.bf16_bits_to_f32(out_bits[tokens]).astype(np.float64)
    m = assert_close(got, ref, label)
    _say(label, "tokens", len(tokens), m)
    return m


def _sample(T, n, seed):
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(T, size=min(n, T), replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(pick), np.int32)


def _pack_reference_nv(codes, s16, d, F):
    """The packed scale tiles of include/moe.h (moe_pack_weights_nvfp4) with
    numpy index arrays; the code tiles are those of moe_pack_weights."""
    E = codes.shape[0]
    r = np.arange(256)
    out = np.empty_like(s16)

    def tiles(mat_s, rows_of_tile, ntiles, K):
        parts = []
        for nt in range(ntiles):
            rows = rows_of_tile(nt)
            for kc in range(K // 128):
                parts.append(mat_s[rows, kc * 8:(kc + 1) * 8].reshape(-1))
        return np.concatenate(parts)

    for e in range(E):
        w1s = s16[e, :d * F // 8].reshape(2 * F, d // 16)
        w2s = s16[e, d * F // 8:].reshape(d, F // 16)
        f_of = lambda nt: nt * 128 + (r // 128) * 64 + (r % 64) + np.where((r // 64) % 2 == 1, F, 0)
        out[e] = np.concatenate([tiles(w1s, f_of, F // 128, d),
                                 tiles(w2s, lambda nt: nt * 256 + r, d // 256, F)])
    return out


@pytest.mark.parametrize("E,d,F", [(3, 512, 256), (2, 256, 384)])
def test_pack_nv_layout(E, d, F):
    from mixture_experts_gemm_amd import binding as B
    rng = np.random.default_rng(31)
    codes = rng.integers(0, 256, size=(E, 3 * d * F // 2), dtype=np.uint8)
    s16 = rng.integers(0, 256, size=(E, 3 * d * F // 16), dtype=np.uint8)
    _say("pack nv", E, d, F)
    wp, sp = B.moe_pack_weights_nvfp4(torch.from_numpy(codes).cuda(), torch.from_numpy(s16).cuda(), d, F)
    wp_mx, _ = B.moe_pack_weights(torch.from_numpy(codes).cuda(),
                                  torch.zeros(E, 3 * d * F // 32, dtype=torch.uint8, device="cuda"), d, F)
    np.testing.assert_array_equal(wp.cpu().numpy(), wp_mx.cpu().numpy())
    np.testing.assert_array_equal(sp.cpu().numpy(), _pack_reference_nv(codes, s16, d, F))


@pytest.mark.parametrize("T", [64, 37, 1, 200])
def test_nv_tiny_all_tokens(T):
    # T = 1, 37: 16-row tiles; T = 64, 200: 128-row tiles (2 rows a slot per expert and up)
    L = synth.make_layer_nv("tiny", T=T)
    _say("nv tiny", T)
    out, dbg = run_nv(L)
    _check_routing(L, dbg, f"nv tiny T={T}")
    _check_tokens(L, out, np.arange(T), f"nv tiny T={T}")


@pytest.mark.parametrize("T,k", [(50, 1), (50, 8), (32, 8)])
def test_nv_k_extremes(T, k):
    w = synth.custom_workload(T=T, d=256, E=8, k=k, F=512, seed=41)
    L = synth.make_layer_nv(w)
    _say("nv T k", T, k)
    out, dbg = run_nv(L)
    _check_routing(L, dbg, f"nv T={T} k={k}")
    _check_tokens(L, out, np.arange(T), f"nv T={T} k={k}")


def test_nv_all_tokens_to_one_expert():
    # a 300-row segment (three 128-row tiles, the last ragged) next to empty experts
    w = synth.custom_workload(T=300, d=256, E=16, k=2, F=256, seed=42, zipf=True)
    L = synth.make_layer_nv(w, with_tokens=False)
    L.router_w[:, 0] = 0.0
    L.router_w[[0, 11, 12, 13, 14, 15], 0] = -50.0
    L.router_w[5, 0] = 50.0
    L.x = synth.make_tokens(w, L.router_w)
    _say("nv one hot expert")
    out, dbg = run_nv(L)
    r = _check_routing(L, dbg, "nv hot expert")
    assert np.all(dbg["ids"][:, 0] == 5) and (r["counts"] == 0).sum() >= 6
    _check_tokens(L, out, np.arange(300), "nv hot expert")


@pytest.mark.parametrize("name", ["decode1", "decode4"])
def test_nv_decode_all_tokens(name):
    L = synth.make_layer_nv(name)
    _say("nv", name)
    out, dbg = run_nv(L)
    _check_routing(L, dbg, "nv " + name)
    _check_tokens(L, out, np.arange(L.shape.T), "nv " + name)


def test_nv_deterministic_and_in_place():
    L = synth.make_layer_nv("tiny", T=200)
    dev = upload_nv(L)
    a, _ = run_nv(L, dev=dev, debug=False)
    b, _ = run_nv(L, dev=dev, debug=False)
    assert np.array_equal(a, b)
    x = dev["x"].clone()
    from mixture_experts_gemm_amd import binding as B
    B.moe_layer_forward_nvfp4(x, dev["router_w"], dev["w"], dev["s"], dev["gs"], dev["alpha"],
                              dev["beta"], L.k, s_out=x)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(x), a)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["prefill", "ep753", "ep3012"])
def test_nv_full_size(name):
    """Routing on every token; outputs on 512 seeded tokens (every token at
    the expert-parallel shares) plus the tokens behind the first and last row
    of every 192-row tile."""
    L = synth.make_layer_nv(name, threads=16)
    _say("nv", name, "T", L.shape.T)
    out, dbg = run_nv(L)
    r = _check_routing(L, dbg, "nv " + name)
    assert int(r["counts"].sum()) == L.shape.T * L.shape.k
    n = 512 if name == "prefill" else L.shape.T
    _check_tokens(L, out, parity_tokens(L.shape.T, dbg, L.shape.k, 192, n=n, seed=7), "nv " + name)


# (T, d, E, k, F): E = 16 runs the 16-feature streaming kernel; E = 256,
# k = 8 the whole-column kernel (712 and 256 column items; F/128 odd)
@pytest.mark.parametrize("T,d,E,k,F", [(3, 2048, 16, 4, 256), (8, 4096, 16, 4, 256),
                                       (6, 2048, 256, 8, 2048), (3, 4096, 256, 8, 1408)])
def test_nv_few_tokens_hot_expert(T, d, E, k, F):
    # every token picks expert 3 first: on the streaming gate/up kernels its
    # segment is cut into several 2-row tiles
    w = synth.custom_workload(T=T, d=d, E=E, k=k, F=F, seed=43 + T, zipf=True)
    L = synth.make_layer_nv(w, with_tokens=False)
    L.router_w[:, 0] = 0.0
    L.router_w[3, 0] = 50.0
    L.x = synth.make_tokens(w, L.router_w)
    _say("nv few tokens hot expert", T, d)
    out, dbg = run_nv(L)
    _check_routing(L, dbg, f"nv hot T={T} d={d}")
    assert np.all(dbg["ids"][:, 0] == 3)
    _check_tokens(L, out, np.arange(T), f"nv hot T={T} d={d}")


@pytest.mark.timeout(900)
def test_nv_skewed_full_size():
    """Zipf-biased routing: the hottest expert's segment spans dozens of
    192-row tiles; 512 seeded tokens plus every tile's first and last row."""
    L = synth.make_layer_nv("skewed", threads=16)
    _say("nv skewed T", L.shape.T)
    out, dbg = run_nv(L)
    _check_routing(L, dbg, "nv skewed")
    _say("nv skewed largest segment", int(np.diff(dbg["offsets"]).max()))
    _check_tokens(L, out, parity_tokens(L.shape.T, dbg, L.shape.k, 192, n=512, seed=9), "nv skewed")


@pytest.mark.parametrize("T,d,E,k,F", [(512, 768, 8, 2, 1408), (4, 768, 16, 4, 384),
                                       (6, 2048, 64, 6, 1408)])
def test_nv_other_shapes(T, d, E, k, F):
    """d = 768 and F = 1408 on the tiled, 16-row and streaming kernels."""
    w = synth.custom_workload(T=T, d=d, E=E, k=k, F=F, seed=80 + T)
    L = synth.make_layer_nv(w)
    _say("nv shape", (T, d, E, k, F))
    out, dbg = run_nv(L)
    _check_routing(L, dbg, f"nv {(T, d, E, k, F)}")
    _check_tokens(L, out, np.arange(T), f"nv {(T, d, E, k, F)}")


@pytest.mark.parametrize("name,T", [("tiny", 64), ("decode4", None), ("prefill", 512)])
def test_nv_outlier_activation_blocks(name, T):
    """One channel per 32-block at 2^8..2^12 times the rest and blocks with
    half their values 2^-14 below, alpha = 0: the fp16 row scaling keeps every
    bf16 value down to 2^-32 of the row's largest exact."""
    L = synth.make_layer_nv(name, T=T, outliers=True)
    L.alpha[:] = 0.0
    _say("nv outliers", name, L.shape.T)
    out, dbg = run_nv(L)
    _check_routing(L, dbg, f"nv outliers {name}")
    _check_tokens(L, out, np.arange(L.shape.T), f"nv outliers {name}")


@pytest.mark.parametrize("name,T", [("tiny", 64), ("decode4", None), ("prefill", 512)])
def test_nv_workspace_contents_do_not_matter(name, T):
    """A workspace of 0xFF bytes gives bit-for-bit the zeroed workspace's output."""
    from mixture_experts_gemm_amd import binding as B
    L = synth.make_layer_nv(name, T=T)
    dev = upload_nv(L)
    s = L.shape
    n = B.moe_layer_workspace_size(s.T, s.d, s.E, s.F, s.k)
    _say("nv poisoned workspace", name, s.T)
    outs = []
    for fill in (0x00, 0xFF):
        ws = torch.full((n,), fill, dtype=torch.uint8, device="cuda")
        outs.append(run_nv(L, dev=dev, debug=False, workspace=ws)[0])
        del ws
    assert np.array_equal(outs[0], outs[1]), int((outs[0] != outs[1]).sum())


def _scaled_rows(L):
    """Rows of x multiplied by 1, 2^6, 2^13, 2^20 in turn (exact in bf16;
    scaling up only widens the router margins), alpha = 0 so the output is
    beta * y alone.  Returns the layer and the row scales."""
    f = synth.bf16_bits_to_f32(L.x).astype(np.float32)
    scale = np.array([1.0, 2.0 ** 6, 2.0 ** 13, 2.0 ** 20], np.float32)[np.arange(L.x.shape[0]) % 4]
    L.x = synth.f32_to_bf16_bits(f * scale[:, None])
    L.alpha[:] = 0.0
    return L, scale


def _check_scaled_routing(L, dbg, scale, label):
    """Routing bit-exact; weights to 1e-5 on the unscaled rows (the fp32
    scores and their rounding differences grow with the row)."""
    r = oracle.route(L.x, L.router_w, L.k)
    for n in ("ids", "offsets", "perm", "inv"):
        np.testing.assert_array_equal(dbg[n], r[n], err_msg=label)
    assert np.all(np.abs(dbg["weights"] - r["w"])[scale == 1.0] <= WEIGHT_TOL), label


def test_nv_rows_of_very_different_magnitude():
    for name, T in (("tiny", 64), ("prefill", 256), ("decode4", None)):
        L, scale = _scaled_rows(synth.make_layer_nv(name, T=T))
        _say("nv scaled rows", name, L.shape.T)
        out, dbg = run_nv(L)
        _check_scaled_routing(L, dbg, scale, f"nv scaled rows {name}")
        _check_tokens(L, out, np.arange(L.shape.T), f"nv scaled rows {name}")
