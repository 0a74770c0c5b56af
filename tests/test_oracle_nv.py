"""Pins for the oracle's 16-block weight format (NV1-NV3 in oracle.c).

"Muse Spark Open を段階的に分解する" (animemo.app), section ⑪: the released
expert weights share one small scale per 16 values, about 4.5 bits a value;
section ⑬: about 28 MB per 4-bit expert, read in about 5.9 us.  The scale
encoding is a reading (one E4M3 byte per 16 values and one fp32 scale per
matrix, as in the published NVFP4 format), so every pin here is against
something other than oracle.c: torch's float8_e4m3fn decode, the MXFP4
oracle (pinned in test_oracle.py) on weights that both formats hold exactly,
numpy float64 products, and the pages' byte and time figures.
"""
import json
import os

import numpy as np
import torch

import oracle
from mixture_experts_gemm_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3(b: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_e4m3_matches_torch_for_every_byte():
    bytes_ = np.arange(256, dtype=np.uint8)
    ref = _torch_e4m3(bytes_)
    got = np.array([oracle.e4m3(int(b)) for b in bytes_])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m])
    # a few landmarks of the format: 1.0, the largest, the smallest subnormal / normal
    assert oracle.e4m3(0x38) == 1.0 and oracle.e4m3(0x7E) == 448.0
    assert oracle.e4m3(0x01) == 2.0 ** -9 and oracle.e4m3(0x08) == 2.0 ** -6
    assert oracle.e4m3(0xB8) == -1.0


def test_bytes_per_expert_match_the_page():
    with open(os.path.join(GOLD, "costmodel_muse.json")) as f:
        cm = json.load(f)
    d, F = 8192, 2048  # the layer shape used throughout (same 50.3M weights per expert)
    per_expert = 3 * d * F // 2 + 3 * d * F // 16 + 3 * 4  # codes + E4M3 bytes + matrix scales
    want, tol = cm["expect"]["nvfp4_bytes_per_expert"]
    assert abs(per_expert / want - 1) <= tol
    us = per_expert / cm["h200_hbm_bytes_per_s"] * 1e6
    want_us, tol_us = cm["expect"]["read_us_per_expert"]
    assert abs(us / want_us - 1) <= tol_us
    assert abs(per_expert * 8 / (3 * d * F) - cm["nvfp4_bits_per_value"]) < 1e-5


def _pow2_pair(rng, rows, K):
    """E8M0 bytes for 32-blocks and the E4M3 bytes of the same powers of two
    (both 16-blocks of a 32-block alike): exponents 2^-6 .. 2^8."""
    e = rng.integers(-6, 9, size=(rows, K // 32))
    s8 = (e + 127).astype(np.uint8)
    s16 = np.repeat(((e + 7) << 3).astype(np.uint8), 2, axis=1)
    return s8, s16


def test_dequant_reduces_to_mxfp4_on_power_of_two_scales():
    rng = np.random.default_rng(11)
    rows, K = 40, 256
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    s8, s16 = _pow2_pair(rng, rows, K)
    assert np.array_equal(oracle.dequant_rows_nv(codes, s16, K, 1.0), oracle.dequant_rows(codes, s8, K))


def test_dequant_is_code_times_block_scale_times_matrix_scale():
    rng = np.random.default_rng(12)
    rows, K = 24, 192
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    s16 = rng.integers(0, 256, size=(rows, K // 16), dtype=np.uint8)
    s16[(s16 & 0x7F) == 0x7F] = 0x38  # no NaN bytes
    g = 0.0372
    # E2M1 values from the (pinned) MXFP4 decode at unit scale, E4M3 from torch
    e2m1 = oracle.dequant_rows(codes, np.full((rows, K // 32), 127, np.uint8), K)
    sc = np.repeat(_torch_e4m3(s16), 16, axis=1)
    ref = e2m1 * sc * g
    got = oracle.dequant_rows_nv(codes, s16, K, g)
    assert np.array_equal(got, ref)
    # block boundaries: element 15 and 16 of a row take different scale bytes
    assert got[0, 16] == e2m1[0, 16] * _torch_e4m3(s16[0, 1:2])[0] * g


def test_expert_vs_numpy_float64():
    rng = np.random.default_rng(13)
    d, F = 256, 128
    w = rng.integers(0, 256, size=3 * d * F // 2, dtype=np.uint8)
    s16 = synth._expert_scales16(0, 0, 0, 3 * d * F // 16)
    gs = np.array([0.031, 0.027, 0.044], np.float32)
    x = rng.standard_normal(d)
    o, n, ms = oracle.expert_nv(w, s16, gs, x, d, F, eps=1e-6)
    nb, ns = F * d // 2, F * d // 16
    Wg = oracle.dequant_rows_nv(w[:nb], s16[:ns], d, float(gs[0]))
    Wu = oracle.dequant_rows_nv(w[nb:2 * nb], s16[ns:2 * ns], d, float(gs[1]))
    Wd = oracle.dequant_rows_nv(w[2 * nb:], s16[2 * ns:], F, float(gs[2]))
    g = Wg @ x
    a = g / (1 + np.exp(-g)) * (Wu @ x)
    o_ref = Wd @ a
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12 * np.abs(o_ref).max())
    ms_ref = np.mean(o_ref ** 2)
    assert abs(ms / ms_ref - 1) < 1e-12
    np.testing.assert_allclose(n, o_ref / np.sqrt(ms_ref + 1e-6), rtol=1e-11)
    # the gate's matrix scale enters inside silu: doubling it is not a rescale of o
    o2, _, _ = oracle.expert_nv(w, s16, gs * np.array([2, 1, 1], np.float32), x, d, F)
    assert not np.allclose(o2, 2 * o)


def test_layer_reduces_to_mxfp4_layer():
    L = synth.make_layer("tiny")
    s = L.shape
    # the MXFP4 draw's E8M0 bytes (2^-8 .. 2^-4) as E4M3 powers of two
    # 2^-2 .. 2^2 times a matrix scale 2^-6: the same weights exactly
    s8 = L.scales
    s16 = np.repeat(((s8.astype(np.int64) - 121 + 7) << 3).astype(np.uint8), 2, axis=1)
    gs = np.full((s.E, 3), 2.0 ** -6, np.float32)
    mx, ids_mx, w_mx = oracle.moe_forward(L.x, L.router_w, L.w_packed, s8, L.alpha, L.beta, L.k)
    nv, ids_nv, w_nv = oracle.moe_forward_nv(L.x, L.router_w, L.w_packed, s16, gs, L.alpha, L.beta, L.k)
    assert np.array_equal(ids_mx, ids_nv) and np.array_equal(w_mx, w_nv)
    assert np.array_equal(mx, nv)


def test_layer_matrix_scales_of_up_and_down_cancel_in_the_norm():
    # o is linear in the up and down matrices' scales and the per-expert norm
    # removes any positive factor (eps = 0): the output does not move
    L = synth.make_layer_nv("tiny", T=16)
    base, _, _ = oracle.moe_forward_nv(L.x, L.router_w, L.w_packed, L.scales16, L.gscale, L.alpha,
                                       L.beta, L.k, eps=0.0)
    g2 = L.gscale * np.array([1, 4, 0.5], np.float32)
    moved, _, _ = oracle.moe_forward_nv(L.x, L.router_w, L.w_packed, L.scales16, g2, L.alpha,
                                        L.beta, L.k, eps=0.0)
    np.testing.assert_allclose(moved, base, rtol=1e-12, atol=1e-12 * np.abs(base).max())
    g3 = L.gscale * np.array([4, 1, 1], np.float32)
    gate, _, _ = oracle.moe_forward_nv(L.x, L.router_w, L.w_packed, L.scales16, g3, L.alpha,
                                       L.beta, L.k, eps=0.0)
    assert np.abs(gate - base).max() > 1e-3 * np.abs(base).max()


def test_layer_token_subset():
    L = synth.make_layer_nv("tiny", T=24)
    full, ids, w = oracle.moe_forward_nv(L.x, L.router_w, L.w_packed, L.scales16, L.gscale, L.alpha,
                                         L.beta, L.k)
    sel = np.array([5, 0, 17], np.int32)
    sub, ids_s, w_s = oracle.moe_forward_nv(L.x, L.router_w, L.w_packed, L.scales16, L.gscale,
                                            L.alpha, L.beta, L.k, tokens=sel)
    assert np.array_equal(sub, full[sel]) and np.array_equal(ids_s, ids[sel])
