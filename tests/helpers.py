"""Shared test helpers: device upload of generated inputs, the GPU call through
the C ABI, and the floating-point comparison metrics.

Tolerances for the layer output s (bf16) against the oracle's float64 s_ref:
  rel_max  = max |a - b| / max(|b|, rms of b's row)   <= 2e-2
  normwise = ||a - b||_F / ||b||_F                     <= 5e-3
Routing ids, offsets, perm and inv must match exactly; weights to 1e-5.
"""
import numpy as np
import torch

REL_MAX_TOL = 2e-2
NORMWISE_TOL = 5e-3
WEIGHT_TOL = 1e-5


def weight_tol(x_bits):
    """Per-token bound on |w_gpu - w_ref|: 1e-5 for rows of unit RMS (the
    generator's N(0,1) tokens), growing with the row's RMS: the fp32 scores,
    and the rounding by which two summation orders differ, scale with the
    row, and the softmax weights' differences with them."""
    from mixture_experts_gemm_amd import synth
    x = synth.bf16_bits_to_f32(x_bits).astype(np.float64)
    rms = np.sqrt(np.mean(x * x, axis=1))
    return WEIGHT_TOL * np.maximum(rms, 1.0)[:, None]


def metrics(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    rms = np.sqrt(np.mean(b * b, axis=-1, keepdims=True))
    rel = np.abs(a - b) / np.maximum(np.abs(b), rms)
    return dict(rel_max=float(rel.max()),
                normwise=float(np.linalg.norm(a - b) / np.linalg.norm(b)),
                plain=float(np.abs(a - b).max() / np.abs(b).max()))


def assert_close(a, b, label=""):
    m = metrics(a, b)
    assert m["rel_max"] <= REL_MAX_TOL and m["normwise"] <= NORMWISE_TOL, (label, m)
    return m


def bf16_tensor(bits: np.ndarray, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def upload(L, device="cuda"):
    """Device copies of a generated layer; the expert weights go through the
    library's packing entry point (natural rows -> packed tiles)."""
    from mixture_experts_gemm_amd import binding as B
    w_nat = torch.from_numpy(L.w_packed).to(device)
    s_nat = torch.from_numpy(L.scales).to(device)
    w, s = B.moe_pack_weights(w_nat, s_nat, L.shape.d, L.shape.F)
    torch.cuda.synchronize()
    del w_nat, s_nat
    return dict(
        x=bf16_tensor(L.x, device),
        router_w=torch.from_numpy(L.router_w).to(device),
        w=w,
        s=s,
        alpha=torch.from_numpy(L.alpha).to(device),
        beta=torch.from_numpy(L.beta).to(device),
    )


def tile_edge_rows(offsets, R):
    """Grouped rows at the first and the last row of every tile the library's
    tiled expert kernels cut the segments into: an expert with c rows gets
    nt = ceil(c / R) tiles of `per` rows each (the last one ragged), per =
    ceil(c / nt) rounded up to a multiple of 16 (the MFMA row block) and at
    most R (R = 128 for MXFP4 weights, 192 for the 16-block format)."""
    rows = []
    for e in range(len(offsets) - 1):
        a, c = int(offsets[e]), int(offsets[e + 1] - offsets[e])
        if c == 0:
            continue
        nt = -(-c // R)
        per = min(R, ((-(-c // nt)) + 15) // 16 * 16)
        for i in range(nt):
            r0 = i * per
            rows += [a + r0, a + min(c, r0 + per) - 1]
    return np.unique(np.asarray(rows, np.int64))


def parity_tokens(T, dbg, k, R, n=512, seed=0):
    """Tokens to compare at full size: n seeded tokens (all when T <= n),
    token 0 and T-1, and the tokens behind the first and last row of every
    tile (tile_edge_rows)."""
    rng = np.random.default_rng(seed)
    pick = set(range(T)) if T <= n else set(rng.choice(T, size=n, replace=False).tolist())
    pick |= {0, T - 1}
    rows = tile_edge_rows(dbg["offsets"], R)
    pick |= set((dbg["perm"][rows] // k).tolist())
    return np.array(sorted(pick), np.int32)


def debug_buffers(T, E, k, device="cuda"):
    S = T * k
    return dict(ids=torch.empty(S, dtype=torch.int32, device=device),
                weights=torch.empty(S, dtype=torch.float32, device=device),
                offsets=torch.empty(E + 1, dtype=torch.int32, device=device),
                perm=torch.empty(S, dtype=torch.int32, device=device),
                inv=torch.empty(S, dtype=torch.int32, device=device))


def run_layer(L, dev=None, debug=True, x=None, **kw):
    """GPU layer through the C ABI.  Returns (s_out bits [T][d], debug numpy dict)."""
    from mixture_experts_gemm_amd import binding as B
    dev = dev or upload(L)
    s = L.shape
    xin = dev["x"] if x is None else x
    T = xin.shape[0]
    dbg = debug_buffers(T, s.E, s.k) if debug else None
    out = B.moe_layer_forward(xin, dev["router_w"], dev["w"], dev["s"], dev["alpha"], dev["beta"],
                              s.k, F=s.F, eps=L.eps, debug=dbg, **kw)
    torch.cuda.synchronize()
    res = None
    if debug:
        res = {n: t.cpu().numpy() for n, t in dbg.items()}
        res["ids"] = res["ids"].reshape(T, s.k)
        res["weights"] = res["weights"].reshape(T, s.k)
    return bf16_bits(out), res


def upload_latent(L, device="cuda"):
    """Device copies of a generated latent-width layer (experts packed for width d)."""
    from mixture_experts_gemm_amd import binding as B
    w_nat = torch.from_numpy(L.w_packed).to(device)
    s_nat = torch.from_numpy(L.scales).to(device)
    w, s = B.moe_pack_weights(w_nat, s_nat, L.w.d, L.w.F)
    torch.cuda.synchronize()
    del w_nat, s_nat
    return dict(
        x=bf16_tensor(L.x, device),
        router_w=torch.from_numpy(L.router_w).to(device),
        wc=bf16_tensor(L.wc, device),
        w=w,
        s=s,
        we=bf16_tensor(L.we, device),
        alpha=torch.from_numpy(L.alpha).to(device),
        beta=torch.from_numpy(L.beta).to(device),
    )


def run_latent(L, dev=None, debug=True, **kw):
    """GPU latent-width layer through the C ABI.  Returns (s_out bits [T][D], debug dict)."""
    from mixture_experts_gemm_amd import binding as B
    dev = dev or upload_latent(L)
    w = L.w
    dbg = debug_buffers(w.T, w.E, w.k) if debug else None
    out = B.moe_latent_forward(dev["x"], dev["router_w"], dev["wc"], dev["w"], dev["s"], dev["we"],
                               dev["alpha"], dev["beta"], w.k, F=w.F, eps=L.eps, debug=dbg, **kw)
    torch.cuda.synchronize()
    res = None
    if debug:
        res = {n: t.cpu().numpy() for n, t in dbg.items()}
        res["ids"] = res["ids"].reshape(w.T, w.k)
        res["weights"] = res["weights"].reshape(w.T, w.k)
    return bf16_bits(out), res


def upload_nv(L, device="cuda"):
    """Device copies of a generated layer in the 16-block format, packed by the
    library's entry point."""
    from mixture_experts_gemm_amd import binding as B
    w_nat = torch.from_numpy(L.w_packed).to(device)
    s_nat = torch.from_numpy(L.scales16).to(device)
    w, s = B.moe_pack_weights_nvfp4(w_nat, s_nat, L.shape.d, L.shape.F)
    torch.cuda.synchronize()
    del w_nat, s_nat
    return dict(
        x=bf16_tensor(L.x, device),
        router_w=torch.from_numpy(L.router_w).to(device),
        w=w,
        s=s,
        gs=torch.from_numpy(L.gscale).to(device),
        alpha=torch.from_numpy(L.alpha).to(device),
        beta=torch.from_numpy(L.beta).to(device),
    )


def run_nv(L, dev=None, debug=True, **kw):
    """GPU layer on 16-block weights through the C ABI: (s_out bits, debug dict)."""
    from mixture_experts_gemm_amd import binding as B
    dev = dev or upload_nv(L)
    s = L.shape
    T = dev["x"].shape[0]
    dbg = debug_buffers(T, s.E, s.k) if debug else None
    out = B.moe_layer_forward_nvfp4(dev["x"], dev["router_w"], dev["w"], dev["s"], dev["gs"],
                                    dev["alpha"], dev["beta"], s.k, F=s.F, eps=L.eps, debug=dbg, **kw)
    torch.cuda.synchronize()
    res = None
    if debug:
        res = {n: t.cpu().numpy() for n, t in dbg.items()}
        res["ids"] = res["ids"].reshape(T, s.k)
        res["weights"] = res["weights"].reshape(T, s.k)
    return bf16_bits(out), res
