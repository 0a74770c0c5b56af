#!/usr/bin/env python3
"""Throughput of the MoE expert layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload decode4|decode1|prefill|skewed|stack|...]

One step = one moe_layer_forward call (router, top-k, grouping, gate/up +
SwiGLU, down + row sums of squares, RMSNorm/combine/gate) over one batch of
synthetic tokens whose inputs already sit in HBM; for the `stack` workload
one step is four chained calls on four weight sets.  Decode steps rotate
over four independent weight sets (27 GB) and a pool of token rows, so the
256 MB Infinity Cache cannot serve the expert weights.

Prints ONE JSON line: tokens/s for the named workload, the roofline of the
dominant kernel (gate/up), measured live with HIP events recorded by the
library on the benchmark's stream, beside the whole layer's fraction; the
CPU oracle on a bounded sample; and the other shapes under "also", each with
its own roofline, oracle baseline and three-rerun determinism flag.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s (T=1/4 decode, T=4096 prefill) + % HBM / MFMA roofline"
WORKLOAD_TEXT = {
    "decode4": "Muse-shaped decode, 4 concurrent requests (T=4, d=8192, E=256, top-8, F=2048, MXFP4)",
    "decode1": "Muse-shaped decode, single request (T=1, d=8192, E=256, top-8, F=2048, MXFP4)",
    "prefill": "Muse-shaped prefill micro-batch (T=4096, d=8192, E=256, top-8, F=2048, MXFP4, uniform routing)",
    "skewed": "Skewed-routing prefill (T=16384, d=8192, E=256, top-8, F=2048, MXFP4, Zipf(1.2) router "
              "bias, top-8 experts ~40% of slots)",
    "stack": "Stack of 4 chained MoE layers with independent weights (T=8192, d=8192, E=256, top-8, "
             "F=2048, MXFP4, per-expert RMSNorm + alpha/beta gated residual between layers)",
    "ep753": "One GPU's share under 8-way expert parallelism, 753-token batch (E=32 local experts, "
             "753 routed rows, k=1, d=8192, F=2048, MXFP4)",
    "ep3012": "One GPU's share under 8-way expert parallelism, 3012-token batch (E=32 local experts, "
              "3012 routed rows, k=1, d=8192, F=2048, MXFP4)",
    "latent4": "Latent-width variant, 4 concurrent requests (T=4, token width 8192 narrowed to 4096 by a "
               "shared bf16 matrix, E=256, top-8, 4096x4096 MXFP4 experts, widened back by a second one)",
    "latent_prefill": "Latent-width variant, prefill micro-batch (T=4096, 8192 -> 4096 -> 8192 shared bf16 "
                      "matrices, E=256, top-8, 4096x4096 MXFP4 experts)",
    "block4": "MoE block with its stream norms (RMSNorm + gain in front, on the output before the gate), "
              "4 concurrent requests (T=4, d=8192, E=256, top-8, F=2048, MXFP4)",
    "block_prefill": "MoE block with its stream norms, prefill micro-batch (T=4096, d=8192, E=256, top-8, "
                     "F=2048, MXFP4)",
    "nv4": "Muse-shaped decode, 4 concurrent requests, expert weights in the 16-block format "
           "(T=4, d=8192, E=256, top-8, F=2048, E2M1 + E4M3 per 16 + fp32 per matrix)",
    "nv_prefill": "Muse-shaped prefill micro-batch, expert weights in the 16-block format "
                  "(T=4096, d=8192, E=256, top-8, F=2048, E2M1 + E4M3 per 16 + fp32 per matrix)",
}
LATENT = ("latent4", "latent_prefill")
# the block with its stream norms runs on the full-width workloads' inputs
BLOCK = {"block4": "decode4", "block_prefill": "prefill"}
# the 16-block weight format on the full-width workloads' tokens and router
NV = {"nv4": "decode4", "nv_prefill": "prefill"}
DECODE_LIKE = ("latent4", "block4", "nv4")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode4", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--also", default="decode1,prefill,skewed,stack,ep753,ep3012,latent4,latent_prefill,"
                                      "block4,block_prefill,nv4,nv_prefill",
                    help="comma list of extra workloads timed after the main one ('' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle time on the main workload")
    ap.add_argument("--cpu-also-seconds", type=float, default=3.0,
                    help="oracle time on each extra workload and each one-thread run")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the copy / GEMM peak probes")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (a known-size kernel "
                         "to scale hardware byte counters against)")
    return ap.parse_args()


def make_sets(name, nsets, device):
    """Weight sets (layer 0 from the shared generator, the rest drawn on the GPU)."""
    import numpy as np
    import torch

    from mixture_experts_gemm_amd import binding as B
    from mixture_experts_gemm_amd import synth

    w = synth.WORKLOADS[name]
    s = w.shape
    pool = 256 if s.T < 64 else s.T  # decode: a pool of token rows, 64 or more batches
    host = synth.make_layer(w, layer=0, T=pool, threads=16)
    sets = []
    for i in range(nsets):
        if i == 0:
            W = torch.from_numpy(host.w_packed).to(device)
            S = torch.from_numpy(host.scales).to(device)
            wr = torch.from_numpy(host.router_w).to(device)
            a = torch.from_numpy(host.alpha).to(device)
            b = torch.from_numpy(host.beta).to(device)
        else:
            g = torch.Generator(device=device)
            g.manual_seed(1000 * w.seed + i)
            W = torch.randint(0, 256, (s.E, s.expert_bytes), dtype=torch.uint8, device=device, generator=g)
            S = torch.randint(synth.SCALE_LO, synth.SCALE_HI + 1, (s.E, s.expert_scale_bytes),
                              dtype=torch.uint8, device=device, generator=g)
            wr = torch.from_numpy(synth.make_router(w, layer=i)).to(device)
            a, b = (torch.from_numpy(v).to(device) for v in synth.make_gates(w, layer=i))
        # the layer reads the packed weight layout; packing is a one-time load step
        Wp, Sp = B.moe_pack_weights(W, S, s.d, s.F)
        torch.cuda.synchronize()
        del W, S
        sets.append(dict(w=Wp, s=Sp, wr=wr, alpha=a, beta=b))
    x = torch.from_numpy(host.x.view(np.int16)).to(device).view(torch.bfloat16)
    return w, host, sets, x


def make_nv_sets(name, nsets, device):
    """Weight sets in the 16-block format (set 0 from the shared generator,
    the rest drawn on the GPU with the same distributions)."""
    import numpy as np
    import torch

    from mixture_experts_gemm_amd import binding as B
    from mixture_experts_gemm_amd import synth

    w = synth.WORKLOADS[NV[name]]
    s = w.shape
    pool = 256 if s.T < 64 else s.T
    host = synth.make_layer_nv(w, layer=0, T=pool, threads=16)
    ns = 3 * s.d * s.F // 16
    sets = []
    for i in range(nsets):
        if i == 0:
            W = torch.from_numpy(host.w_packed).to(device)
            S = torch.from_numpy(host.scales16).to(device)
            G = torch.from_numpy(host.gscale).to(device)
            wr = torch.from_numpy(host.router_w).to(device)
            a = torch.from_numpy(host.alpha).to(device)
            b = torch.from_numpy(host.beta).to(device)
        else:
            g = torch.Generator(device=device)
            g.manual_seed(1000 * w.seed + 500 + i)
            W = torch.randint(0, 256, (s.E, s.expert_bytes), dtype=torch.uint8, device=device, generator=g)
            ex = torch.randint(synth.NV_EXP_LO, synth.NV_EXP_HI + 1, (s.E, ns), dtype=torch.uint8,
                               device=device, generator=g)
            mt = torch.randint(0, 8, (s.E, ns), dtype=torch.uint8, device=device, generator=g)
            S = (ex << 3) | mt
            G = (torch.rand(s.E, 3, device=device, generator=g) * 0.5 + 0.75) * 2.0 ** -5
            wr = torch.from_numpy(synth.make_router(w, layer=i)).to(device)
            a, b = (torch.from_numpy(v).to(device) for v in synth.make_gates(w, layer=i))
        Wp, Sp = B.moe_pack_weights_nvfp4(W, S, s.d, s.F)
        torch.cuda.synchronize()
        del W, S
        sets.append(dict(w=Wp, s=Sp, gs=G.contiguous(), wr=wr, alpha=a, beta=b))
    x = torch.from_numpy(host.x.view(np.int16)).to(device).view(torch.bfloat16)
    return w, host, sets, x


def make_latent_sets(name, nsets, device):
    """Weight sets of the latent-width variant (set 0 from the shared
    generator, the others' experts drawn on the GPU)."""
    import numpy as np
    import torch

    from mixture_experts_gemm_amd import binding as B
    from mixture_experts_gemm_amd import synth

    w = synth.LATENT_WORKLOADS[name]
    ev = w.expert_view().shape
    pool = 256 if w.T < 64 else w.T
    host = synth.make_latent_layer(w, layer=0, T=pool, threads=16)
    bf16 = lambda a: torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    sets = []
    for i in range(nsets):
        if i == 0:
            W = torch.from_numpy(host.w_packed).to(device)
            S = torch.from_numpy(host.scales).to(device)
            wr = torch.from_numpy(host.router_w).to(device)
            a = torch.from_numpy(host.alpha).to(device)
            b = torch.from_numpy(host.beta).to(device)
            wc, we = bf16(host.wc), bf16(host.we)
        else:
            g = torch.Generator(device=device)
            g.manual_seed(1000 * w.seed + i)
            W = torch.randint(0, 256, (ev.E, ev.expert_bytes), dtype=torch.uint8, device=device, generator=g)
            S = torch.randint(synth.SCALE_LO, synth.SCALE_HI + 1, (ev.E, ev.expert_scale_bytes),
                              dtype=torch.uint8, device=device, generator=g)
            wr = torch.from_numpy(synth.make_router(w.token_view(), layer=i)).to(device)
            a, b = (torch.from_numpy(v).to(device) for v in synth.make_gates(w.token_view(), layer=i))
            wc, we = (bf16(m) for m in synth.make_shared(w, layer=i))
        Wp, Sp = B.moe_pack_weights(W, S, w.d, w.F)
        torch.cuda.synchronize()
        del W, S
        sets.append(dict(w=Wp, s=Sp, wr=wr, alpha=a, beta=b, wc=wc, we=we))
    x = bf16(host.x)
    return w, host, sets, x


# the gate/up kernel each workload runs (the dominant kernel of the layer)
GATE_UP_KERNEL = {
    "decode1": "gemm1_stream_kernel (routing prologue + gate/up + SwiGLU, persistent, MX MFMA)",
    "decode4": "gemm1_col_kernel (gate/up + SwiGLU, persistent, whole 128-feature tile columns, MX MFMA)",
    "prefill": "gemm_mxw_kernel<true, 128> (gate/up + SwiGLU, 128x512 tiles, MX MFMA)",
    "skewed": "gemm_mxw_kernel<true, 128> (gate/up + SwiGLU, 128x512 tiles, MX MFMA)",
    "stack": "gemm_mxw_kernel<true, 128> (gate/up + SwiGLU, 128x512 tiles, MX MFMA)",
    "ep753": "gemm_mxw_kernel<true, 64> (gate/up + SwiGLU, 64x512 tiles, three stages, MX MFMA)",
    "ep3012": "gemm_mxw_kernel<true, 128> (gate/up + SwiGLU, 128x512 tiles, MX MFMA)",
    "latent4": "gemm1_col_kernel (gate/up + SwiGLU, persistent, whole 128-feature tile columns, MX MFMA)",
    "latent_prefill": "gemm_mxw_kernel<true, 128> (gate/up + SwiGLU, 128x512 tiles, MX MFMA)",
    "block4": "gemm1_col_kernel (gate/up + SwiGLU, persistent, whole 128-feature tile columns, MX MFMA)",
    "block_prefill": "gemm_mxw_kernel<true, 128> (gate/up + SwiGLU, 128x512 tiles, MX MFMA)",
    "nv4": "gemm1_col_kernel<false, true> (gate/up + SwiGLU, persistent, whole 128-feature tile columns, fp16 MFMA, 16-block weights)",
    "nv_prefill": "gemm_nv_kernel<true> (gate/up + SwiGLU, 192x256 tiles, fp16 MFMA, 16-block weights)",
}
# How the gate/up kernel issues one bf16 x FP4 product on the matrix cores:
# (MFMAs per product, operand types, that instruction's dense peak in
# TFLOP/s).  The streaming decode kernels split x into two FP8 parts, the
# wide prefill kernel into three FP6 parts; the 16-block kernels run fp16.
MX_ISSUE = {
    "gemm1_stream_kernel": (2, "fp8 x fp4 (two FP8 parts of x)", 5000.0),
    "gemm1_col_kernel": (2, "fp8 x fp4 (two FP8 parts of x)", 5000.0),
    "gemm_mxw_kernel": (3, "fp6 x fp4 (three FP6 parts of x)", 10100.0),
    "gemm_nv_kernel": (1, "fp16 x fp16 (weights widened)", 2500.0),
}


EVENT_EVERY = 8  # timed steps between two gate/up kernel timings


def counter_summary(name):
    """Committed HBM byte-counter summary of the gate/up kernel on this workload."""
    return os.path.join(ROOT, "profiles", f"gate_up_{name}_hbm_counters.md")


def _pct(vals, q):
    v = sorted(vals)
    return v[min(len(v) - 1, int(round(q * (len(v) - 1))))]


def _roofline(name, nbytes, flops, g1_ms, R):
    """The gate/up kernel against the bound of its shape (the larger of the
    byte time at the HBM peak and the flop time at the bf16 peak)."""
    hbm_bound = nbytes / R.MI355X_HBM_BYTES_PER_S >= flops / R.MI355X_BF16_FLOPS_PER_S
    kern = GATE_UP_KERNEL[name]
    out = dict(kernel=kern, traffic=R.recorded_traffic(counter_summary(name)),
               kernel_us_per_launch=g1_ms * 1e3)
    if hbm_bound:
        achieved = nbytes / (g1_ms * 1e-3)
        out.update(bound="hbm", achieved=achieved / 1e9, peak=R.MI355X_HBM_BYTES_PER_S / 1e9, unit="GB/s",
                   frac=achieved / R.MI355X_HBM_BYTES_PER_S, algorithmic_bytes_per_launch=nbytes)
    else:
        achieved = flops / (g1_ms * 1e-3)
        out.update(bound="mfma", achieved=achieved / 1e12, peak=R.MI355X_BF16_FLOPS_PER_S / 1e12,
                   unit="TFLOP/s", frac=achieved / R.MI355X_BF16_FLOPS_PER_S,
                   algorithmic_flops_per_launch=flops)
        parts, what, peak = MX_ISSUE[kern.split(" ")[0].split("<")[0]]
        issued = parts * flops / (g1_ms * 1e-3)
        out["mx_issue"] = dict(mfma_per_product=parts, operands=what, issued_TFLOPs=issued / 1e12,
                               peak_TFLOPs=peak, frac=issued / (peak * 1e12))
    return out


def time_workload(name, steps, warmup, device):
    import torch

    from mixture_experts_gemm_amd import binding as B
    from mixture_experts_gemm_amd import roofline as R

    latent = name in LATENT
    block = name in BLOCK
    nv = name in NV
    decode = name.startswith("decode") or name in DECODE_LIKE
    nsets = 4 if decode else 1
    log(f"generating {name}: {nsets} weight set(s)")
    if latent:
        # the experts' view (width d) drives the expert accounting below; the
        # token width D enters through the shared matrices and the router
        w, host, sets, xpool = make_latent_sets(name, nsets, device)
        s = w.expert_view().shape
        D = w.D
    elif nv:
        w, host, sets, xpool = make_nv_sets(name, nsets, device)
        s = w.shape
        D = s.d
    else:
        w, host, sets, xpool = make_sets(BLOCK.get(name, name), nsets, device)
        s = w.shape
        D = s.d
        if block:
            from mixture_experts_gemm_amd import synth
            for i, st in enumerate(sets):
                st["g_pre"], st["g_post"] = (torch.from_numpy(v).to(device)
                                             for v in synth.make_norm_gains(w, layer=i))
            host.g_pre, host.g_post = sets[0]["g_pre"].cpu().numpy(), sets[0]["g_post"].cpu().numpy()
    T = s.T
    npool = xpool.shape[0] // T
    if latent:
        nws = B.moe_latent_workspace_size(T, D, s.d, s.E, s.F, s.k)
        ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=device)
    elif block:
        nws = B.moe_block_workspace_size(T, s.d, s.E, s.F, s.k)
        ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=device)
    else:
        ws = B.workspace_for(T, s.d, s.E, s.F, s.k, device=device)
    out = torch.empty(T, D, dtype=torch.bfloat16, device=device)
    offsets = torch.empty(s.E + 1, dtype=torch.int32, device=device)

    def call(i, debug=None, dst=out):
        st = sets[i % nsets]
        xb = xpool[(i % npool) * T:(i % npool + 1) * T]
        if latent:
            B.moe_latent_forward(xb, st["wr"], st["wc"], st["w"], st["s"], st["we"], st["alpha"],
                                 st["beta"], s.k, F=s.F, s_out=dst, workspace=ws, debug=debug)
        elif block:
            B.moe_block_forward(xb, st["g_pre"], st["wr"], st["w"], st["s"], st["g_post"], st["alpha"],
                                st["beta"], s.k, F=s.F, s_out=dst, workspace=ws, debug=debug)
        elif nv:
            B.moe_layer_forward_nvfp4(xb, st["wr"], st["w"], st["s"], st["gs"], st["alpha"], st["beta"],
                                      s.k, F=s.F, s_out=dst, workspace=ws, debug=debug)
        else:
            B.moe_layer_forward(xb, st["wr"], st["w"], st["s"], st["alpha"], st["beta"], s.k, F=s.F,
                                s_out=dst, workspace=ws, debug=debug)

    # accounting pass (untimed): distinct experts per step, from the library's own grouping
    U = []
    for i in range(steps):
        call(i, debug=dict(offsets=offsets))
        off = offsets.cpu()
        U.append(int(((off[1:] - off[:-1]) > 0).sum()))
    assert torch.isfinite(out.float()).all(), "non-finite layer output"
    # determinism: the same step three times, outputs compared bit for bit
    reruns = [torch.empty_like(out) for _ in range(3)]
    for r in reruns:
        call(0, dst=r)
    torch.cuda.synchronize()
    deterministic = all(torch.equal(reruns[0], r) for r in reruns[1:])
    del reruns
    for i in range(warmup):
        call(i)
    # The gate/up kernel is timed by the HIP events its own dispatch records,
    # on every EVENT_EVERY-th step of the timed region: recording timestamps
    # stalls the queue for a few microseconds, so timing every step would
    # charge that stall to the throughput.
    timed = list(range(0, steps, EVENT_EVERY))
    evs = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for i in timed}
    for a, b in evs.values():  # create the underlying HIP events before handing them over
        a.record()
        b.record()
    torch.cuda.synchronize()
    log(f"timing {name}: {steps} steps after {warmup} warmup")
    t0 = time.perf_counter()
    for i in range(steps):
        call(i, debug=dict(events={"gemm1": evs[i]}) if i in evs else None)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    g1_ms = sum(a.elapsed_time(b) for a, b in evs.values()) / len(evs)
    out_ok = bool(torch.isfinite(out.float()).all())
    S = T * s.k
    u_mean = sum(U) / len(U)
    # Per-step latency distribution, in a separate pass after the timed
    # region (events around every call stall the queue a little, so these
    # steps are not part of `value`): p10, median and p90 over n steps.
    n_lat = min(steps, 50)
    lat = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_lat)]
    for i, (a, b) in enumerate(lat):
        a.record()
        call(i)
        b.record()
    torch.cuda.synchronize()
    step_us = [a.elapsed_time(b) * 1e3 for a, b in lat]
    res = dict(
        T=T, steps=steps, ms_per_step=elapsed / steps * 1e3, tokens_per_s=T * steps / elapsed,
        gemm1_ms=g1_ms, gemm1_timed_launches=len(timed), distinct_experts_mean=u_mean, finite=out_ok,
        bitwise_identical_3_reruns=deterministic,
        step_us_p10_p50_p90=[_pct(step_us, 0.1), _pct(step_us, 0.5), _pct(step_us, 0.9)],
        step_us_samples=n_lat,
    )
    # the gate/up kernel's algorithmic bytes (over the timed launches: U, the
    # distinct experts, differs per step) and flops
    w1b = R.nvfp4_w1_bytes(s.d, s.F) if nv else R.mxfp4_w1_bytes(s.d, s.F)
    nbytes = sum(w1b * U[i] + T * s.d * 2 + S * s.F * 2 for i in timed) / len(timed)
    res["roofline"] = _roofline(name, nbytes, R.gemm1_flops(S, s.d, s.F), g1_ms, R)
    # the whole layer against both peaks (algorithmic bytes with the realized U)
    if latent:
        lb = sum(R.latent_layer_bytes(T, D, s.d, s.E, s.F, u) for u in U) / len(U)
        lf = R.latent_layer_flops(T, D, s.d, s.k, s.F)
    else:
        lb = sum(R.layer_bytes(T, s.d, s.E, s.F, u, nv=nv) for u in U) / len(U)
        lf = R.layer_flops(T, s.d, s.k, s.F)
    res["layer_hbm_frac"] = lb / (elapsed / steps) / R.MI355X_HBM_BYTES_PER_S
    res["layer_mfma_frac"] = lf / (elapsed / steps) / R.MI355X_BF16_FLOPS_PER_S
    res["layer_bytes"] = lb
    res["layer_flops"] = lf
    log(json.dumps(res))
    return res, host, T


def make_stack_sets(device):
    """The four layers of the stack workload from the shared generator (host
    copies kept for the oracle's chain), packed on the GPU."""
    import numpy as np
    import torch

    from mixture_experts_gemm_amd import binding as B
    from mixture_experts_gemm_amd import synth

    w = synth.WORKLOADS["stack"]
    s = w.shape
    hosts, sets = [], []
    for layer in range(w.layers):
        h = synth.make_layer(w, layer=layer, with_tokens=(layer == 0), threads=16)
        Wp, Sp = B.moe_pack_weights(torch.from_numpy(h.w_packed).to(device),
                                    torch.from_numpy(h.scales).to(device), s.d, s.F)
        torch.cuda.synchronize()
        sets.append(dict(w=Wp, s=Sp, wr=torch.from_numpy(h.router_w).to(device),
                         alpha=torch.from_numpy(h.alpha).to(device),
                         beta=torch.from_numpy(h.beta).to(device)))
        hosts.append(h)
    x = torch.from_numpy(hosts[0].x.view(np.int16)).to(device).view(torch.bfloat16)
    return w, hosts, sets, x


def time_stack(steps, warmup, device, sample=32):
    """Four chained layers per step (each layer's bf16 output is the next
    one's input).  Also reports, on `sample` seeded tokens, each layer's
    error against the oracle run on the GPU's own layer input
    (teacher-forced) and against the oracle's own free-running chain (the
    error growth through the gated residual)."""
    import numpy as np
    import torch

    import oracle
    from mixture_experts_gemm_amd import binding as B
    from mixture_experts_gemm_amd import roofline as R
    from mixture_experts_gemm_amd import synth

    log("generating stack: 4 layers")
    w, hosts, sets, x = make_stack_sets(device)
    s = w.shape
    T = s.T
    ws = B.workspace_for(T, s.d, s.E, s.F, s.k, device=device)
    bufs = [torch.empty(T, s.d, dtype=torch.bfloat16, device=device) for _ in range(2)]

    def step(keep=None, ev=None):
        cur = x
        for layer, st in enumerate(sets):
            dst = keep[layer] if keep is not None else bufs[layer % 2]
            dbg = dict(events={"gemm1": ev[layer]}) if ev is not None else None
            B.moe_layer_forward(cur, st["wr"], st["w"], st["s"], st["alpha"], st["beta"], s.k, F=s.F,
                                s_out=dst, workspace=ws, debug=dbg)
            cur = dst
        return cur

    # every layer's output of one step, then the determinism reruns
    outs = [torch.empty(T, s.d, dtype=torch.bfloat16, device=device) for _ in range(4)]
    step(keep=outs)
    reruns = []
    for _ in range(2):
        o2 = [torch.empty_like(o) for o in outs]
        step(keep=o2)
        reruns.append(o2)
    torch.cuda.synchronize()
    deterministic = all(torch.equal(a, b) for r in reruns for a, b in zip(outs, r))
    del reruns
    for _ in range(warmup):
        step()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4)]
    for a, b in ev:
        a.record()
        b.record()
    torch.cuda.synchronize()
    log(f"timing stack: {steps} steps after {warmup} warmup")
    t0 = time.perf_counter()
    for i in range(steps):
        step(ev=ev if i == steps - 1 else None)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    g1_ms = sum(a.elapsed_time(b) for a, b in ev) / 4
    S = T * s.k
    flops = 4 * R.layer_flops(T, s.d, s.k, s.F)
    res = dict(T=T, layers=4, steps=steps, ms_per_step=elapsed / steps * 1e3,
               tokens_per_s=T * steps / elapsed, gemm1_ms=g1_ms, bitwise_identical_3_reruns=deterministic,
               layer_mfma_frac=flops / (elapsed / steps) / R.MI355X_BF16_FLOPS_PER_S)
    res["roofline"] = _roofline("stack", 0, R.gemm1_flops(S, s.d, s.F), g1_ms, R)
    # per-layer error on a token sample
    tok = np.sort(np.random.default_rng(4).choice(T, size=sample, replace=False)).astype(np.int32)
    got = [synth.bf16_bits_to_f32(o.view(torch.int16).cpu().numpy().view(np.uint16)[tok]).astype(np.float64)
           for o in outs]
    gin = [hosts[0].x] + [o.view(torch.int16).cpu().numpy().view(np.uint16) for o in outs[:-1]]
    ref_chain = hosts[0].x[tok]
    err = []
    for layer, h in enumerate(hosts):
        tf, _, _ = oracle.moe_forward(gin[layer], h.router_w, h.w_packed, h.scales, h.alpha, h.beta, h.k,
                                      eps=h.eps, tokens=tok)
        fr, _, _ = oracle.moe_forward(ref_chain, h.router_w, h.w_packed, h.scales, h.alpha, h.beta, h.k,
                                      eps=h.eps)
        m_tf, m_fr = _metrics(got[layer], tf), _metrics(got[layer], fr)
        err.append(dict(layer=layer, teacher_forced=m_tf, free_running=m_fr))
        ref_chain = oracle.doubles_to_bf16(fr)
    res["per_layer_error"] = err
    res["error_sample_tokens"] = sample
    log(json.dumps(res))
    return res, hosts, T


def _metrics(a, b):
    import numpy as np
    rms = np.sqrt(np.mean(b * b, axis=-1, keepdims=True))
    return dict(rel_max=float((np.abs(a - b) / np.maximum(np.abs(b), rms)).max()),
                normwise=float(np.linalg.norm(a - b) / np.linalg.norm(b)))


def cpu_baseline(host, T, seconds, name, threads=None):
    """The oracle as it is, on the host cores, timed on a bounded sample of
    the same workload: whole steps for few-token workloads, else seeded
    token subsets (the layer is token-separable), scaled to tokens/s."""
    import numpy as np

    import oracle

    full = T <= 64
    if threads is not None:
        prev = oracle.max_threads()
        oracle.set_num_threads(threads)
    cores = oracle.max_threads()
    rng = np.random.default_rng(17)
    n = 0
    t0 = time.perf_counter()
    while True:
        tok = None if full else rng.choice(T, size=min(16, T), replace=False).astype(np.int32)
        nt = T if full else len(tok)
        if name == "stack":
            xin = host[0].x if tok is None else host[0].x[tok]
            for h in host:
                y, _, _ = oracle.moe_forward(xin, h.router_w, h.w_packed, h.scales, h.alpha, h.beta, h.k,
                                             eps=h.eps)
                xin = oracle.doubles_to_bf16(y)
        elif hasattr(host, "scales16"):  # 16-block weight format
            oracle.moe_forward_nv(host.x[:T], host.router_w, host.w_packed, host.scales16, host.gscale,
                                  host.alpha, host.beta, host.k, eps=host.eps, tokens=tok)
        elif hasattr(host, "wc"):  # latent-width variant
            oracle.latent_forward(host.x[:T], host.router_w, host.wc, host.w_packed, host.scales,
                                  host.we, host.alpha, host.beta, host.k, eps=host.eps, tokens=tok)
        elif hasattr(host, "g_pre"):  # the block with its stream norms
            oracle.block_forward(host.x[:T], host.g_pre, host.router_w, host.w_packed, host.scales,
                                 host.g_post, host.alpha, host.beta, host.k, eps=host.eps, tokens=tok)
        else:
            oracle.moe_forward(host.x[:T], host.router_w, host.w_packed, host.scales, host.alpha,
                               host.beta, host.k, eps=host.eps, tokens=tok)
        n += nt
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    if threads is not None:
        oracle.set_num_threads(prev)
    what = "whole steps" if full else "seeded 16-token subsets"
    return dict(value=n / el, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{n} tokens in {what} of the workload (weight set 0), {el:.1f} s")


def measured_peaks(device):
    """What this GPU reaches on plain library work, as context for the
    fractions: a 2 GiB device copy (bytes read + written per second) and a
    bf16 8192^3 matrix product (torch.matmul)."""
    import torch

    n = 2 << 30
    a = torch.empty(n, dtype=torch.uint8, device=device)
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(2):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_bps = 5 * 2 * n / (e0.elapsed_time(e1) * 1e-3)
    del a, b
    m = 8192
    x = torch.randn(m, m, dtype=torch.bfloat16, device=device)
    y = torch.randn(m, m, dtype=torch.bfloat16, device=device)
    for _ in range(2):
        torch.matmul(x, y)
    e0.record()
    for _ in range(5):
        torch.matmul(x, y)
    e1.record()
    torch.cuda.synchronize()
    gemm = 5 * 2 * m ** 3 / (e0.elapsed_time(e1) * 1e-3)
    del x, y
    torch.cuda.empty_cache()
    return dict(copy_GBps=copy_bps / 1e9, bf16_gemm_TFLOPs=gemm / 1e12,
                note="2 GiB torch device copy (read + write bytes); torch.matmul bf16 8192^3")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the layer runs on one GPU only (asked for --gpus {args.gpus}); "
              "sharding it over several GPUs is not implemented", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    device = "cuda:0"
    torch.cuda.set_device(0)
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=device)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {n} bytes read, {n} bytes written")
        del src, dst

    def run(name, steps=None, warmup=None):
        d = name.startswith("decode") or name in DECODE_LIKE
        st = steps or (200 if d else (5 if name == "stack" else 20))
        wu = warmup if warmup is not None else (10 if d else 2)
        if name == "stack":
            return time_stack(st, wu, device) + (st, wu)
        return time_workload(name, st, wu, device) + (st, wu)

    main_res, host, T, steps, warmup = run(args.workload, args.steps, args.warmup)
    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle")
        cpu = cpu_baseline(host, T, args.cpu_seconds, args.workload)
    also = {}
    hosts = {args.workload: (host, T)}
    for extra in [e for e in args.also.split(",") if e and e != args.workload]:
        r, h, t, _, _ = run(extra, None if extra != "stack" else 5)
        if not args.no_cpu:
            log(f"timing the CPU oracle on {extra}")
            r["cpu_baseline"] = cpu_baseline(h, t, args.cpu_also_seconds, extra)
        if extra in ("decode1", "decode4"):  # kept for the one-thread oracle runs
            hosts.setdefault(extra, (h, t))
        also[extra] = r
        del h
        torch.cuda.empty_cache()
    single = None
    if not args.no_cpu:
        # the oracle on one host thread, for the tiny and the decode workloads
        from mixture_experts_gemm_amd import synth
        single = {"tiny": cpu_baseline(synth.make_layer("tiny"), 64, args.cpu_also_seconds, "tiny", threads=1)}
        for name in ("decode1", "decode4"):
            if name in hosts:
                h, t = hosts[name]
                single[name] = cpu_baseline(h, t, args.cpu_also_seconds, name, threads=1)
    peaks = None if args.no_peaks else measured_peaks(device)
    s = (host[0].shape if args.workload == "stack" else
         host.w.expert_view().shape if args.workload in LATENT else host.shape)
    roof = main_res["roofline"]
    layer_bound = "hbm" if roof["bound"] == "hbm" else "mfma"
    layer = dict(bound=layer_bound,
                 frac=main_res["layer_hbm_frac"] if layer_bound == "hbm" else main_res["layer_mfma_frac"],
                 note="the whole layer (all kernels, host launch gaps included) over ms_per_step: "
                      "algorithmic bytes (hbm) or flops (mfma) at the same peak")
    if peaks:
        if roof["bound"] == "hbm":
            roof["frac_of_measured_copy_rate"] = roof["achieved"] / peaks["copy_GBps"]
        else:
            roof["frac_of_measured_bf16_gemm_rate"] = roof["achieved"] / peaks["bf16_gemm_TFLOPs"]
    line = {
        "metric": METRIC,
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 x bf16",
        "dtype_note": ("MXFP4 weights (E2M1 + E8M0 per 32) times bf16 activations, fp32 accumulation; on the "
                       "matrix cores the bf16 activations enter as exact block-scaled FP8 (two parts) or "
                       "FP6 (three parts) splits"),
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "T": T, "d": s.d, "E": s.E,
                   **({"D": host.w.D} if args.workload in LATENT else {}),
                   "k": s.k, "F": s.F,
                   "weights": ("E2M1 + E4M3 per 16 + fp32 per matrix" if args.workload in NV
                               else "MXFP4 (E2M1 + E8M0 per 32)"),
                   "weight_sets": 4 if (args.workload.startswith("decode") or args.workload in DECODE_LIKE)
                   else 1,
                   "distinct_experts_mean": main_res.get("distinct_experts_mean")},
        "roofline": {**{k: v for k, v in roof.items()
                        if k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "kernel",
                                 "kernel_us_per_launch", "algorithmic_bytes_per_launch",
                                 "algorithmic_flops_per_launch",
                                 "frac_of_measured_copy_rate", "frac_of_measured_bf16_gemm_rate",
                                 "mx_issue")},
                     "layer": layer},
        "step_us_p10_p50_p90": main_res.get("step_us_p10_p50_p90"),
        "bitwise_identical_3_reruns": main_res["bitwise_identical_3_reruns"],
        "cpu_baseline": cpu,
        "cpu_baseline_1_thread": single,
        "measured_peaks": peaks,
        "also": also,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
