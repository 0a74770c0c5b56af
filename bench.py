#!/usr/bin/env python3
"""Throughput of the MoE expert layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload decode4|decode1|prefill|skewed]

One step = one moe_layer_forward call (router, top-k, grouping, gate/up +
SwiGLU, down + row sums of squares, RMSNorm/combine/gate) over one batch of
synthetic tokens whose inputs already sit in HBM.  Decode steps rotate over
four independent weight sets (27 GB) and a pool of token rows, so the 256 MB
Infinity Cache cannot serve the expert weights.

Prints ONE JSON line: tokens/s for the named workload, the roofline of the
dominant kernel (gate/up), measured live with HIP events recorded by the
library on the benchmark's stream, the CPU oracle on a bounded sample, and
the other shapes under "also".
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
    "skewed": "Skewed-routing prefill (T=16384, Zipf(1.2) router bias, top-8 experts ~40% of slots)",
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
    ap.add_argument("--also", default="decode1,prefill,ep753,ep3012,latent4,latent_prefill,block4,"
                                      "block_prefill,nv4,nv_prefill",
                    help="comma list of extra workloads timed after the main one ('' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
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
    "decode1": "gemm1_stream_kernel (gate/up + SwiGLU, persistent, MX MFMA)",
    "decode4": "gemm1_stream_kernel (gate/up + SwiGLU, persistent, MX MFMA)",
    "prefill": "gemm_mxw_kernel<true> (gate/up + SwiGLU, 128x512 tiles, MX MFMA)",
    "skewed": "gemm_mxw_kernel<true> (gate/up + SwiGLU, 128x512 tiles, MX MFMA)",
    "ep753": "gemm_mxw_kernel<true> (gate/up + SwiGLU, 128x512 tiles, MX MFMA)",
    "ep3012": "gemm_mxw_kernel<true> (gate/up + SwiGLU, 128x512 tiles, MX MFMA)",
    "latent4": "gemm1_stream_kernel (gate/up + SwiGLU, persistent, MX MFMA)",
    "latent_prefill": "gemm_mxw_kernel<true> (gate/up + SwiGLU, 128x512 tiles, MX MFMA)",
    "block4": "gemm1_stream_kernel (gate/up + SwiGLU, persistent, MX MFMA)",
    "block_prefill": "gemm_mxw_kernel<true> (gate/up + SwiGLU, 128x512 tiles, MX MFMA)",
    "nv4": "gemm1_stream_kernel<4, true> (gate/up + SwiGLU, persistent, fp16 MFMA, 16-block weights)",
    "nv_prefill": "gemm_nv_kernel<true, 192> (gate/up + SwiGLU, 192x256 tiles, fp16 MFMA, 16-block weights)",
}


EVENT_EVERY = 8  # timed steps between two gate/up kernel timings


def counter_summary(name):
    """Committed HBM byte-counter summary of the gate/up kernel on this workload."""
    return os.path.join(ROOT, "profiles", f"gate_up_{name}_hbm_counters.md")


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

    def call(i, debug=None):
        st = sets[i % nsets]
        xb = xpool[(i % npool) * T:(i % npool + 1) * T]
        if latent:
            B.moe_latent_forward(xb, st["wr"], st["wc"], st["w"], st["s"], st["we"], st["alpha"],
                                 st["beta"], s.k, F=s.F, s_out=out, workspace=ws, debug=debug)
        elif block:
            B.moe_block_forward(xb, st["g_pre"], st["wr"], st["w"], st["s"], st["g_post"], st["alpha"],
                                st["beta"], s.k, F=s.F, s_out=out, workspace=ws, debug=debug)
        elif nv:
            B.moe_layer_forward_nvfp4(xb, st["wr"], st["w"], st["s"], st["gs"], st["alpha"], st["beta"],
                                      s.k, F=s.F, s_out=out, workspace=ws, debug=debug)
        else:
            B.moe_layer_forward(xb, st["wr"], st["w"], st["s"], st["alpha"], st["beta"], s.k, F=s.F,
                                s_out=out, workspace=ws, debug=debug)

    # accounting pass (untimed): distinct experts per step, from the library's own grouping
    U = []
    for i in range(steps):
        call(i, debug=dict(offsets=offsets))
        off = offsets.cpu()
        U.append(int(((off[1:] - off[:-1]) > 0).sum()))
    assert torch.isfinite(out.float()).all(), "non-finite layer output"
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
    step_us = sorted(a.elapsed_time(b) * 1e3 for a, b in lat)
    pct = lambda q: step_us[min(len(step_us) - 1, int(round(q * (len(step_us) - 1))))]
    res = dict(
        T=T, steps=steps, ms_per_step=elapsed / steps * 1e3, tokens_per_s=T * steps / elapsed,
        gemm1_ms=g1_ms, gemm1_timed_launches=len(timed), distinct_experts_mean=u_mean, finite=out_ok,
        step_us_p10_p50_p90=[pct(0.1), pct(0.5), pct(0.9)], step_us_samples=n_lat,
    )
    # the gate/up kernel's algorithmic bytes (over the timed launches: U, the
    # distinct experts, differs per step) and flops; its bound is the larger
    # of the two times at the peaks
    w1b = R.nvfp4_w1_bytes(s.d, s.F) if nv else R.mxfp4_w1_bytes(s.d, s.F)
    nbytes = sum(w1b * U[i] + T * s.d * 2 + S * s.F * 2 for i in timed) / len(timed)
    flops = R.gemm1_flops(S, s.d, s.F)
    hbm_bound = nbytes / R.MI355X_HBM_BYTES_PER_S >= flops / R.MI355X_BF16_FLOPS_PER_S
    if hbm_bound:
        achieved = nbytes / (g1_ms * 1e-3)
        res["roofline"] = dict(bound="hbm", achieved=achieved / 1e9, peak=R.MI355X_HBM_BYTES_PER_S / 1e9,
                               unit="GB/s", frac=achieved / R.MI355X_HBM_BYTES_PER_S,
                               traffic=R.recorded_traffic(counter_summary(name)),
                               kernel=GATE_UP_KERNEL[name],
                               algorithmic_bytes_per_launch=nbytes)
    else:
        achieved = flops / (g1_ms * 1e-3)
        res["roofline"] = dict(bound="mfma", achieved=achieved / 1e12, peak=R.MI355X_BF16_FLOPS_PER_S / 1e12,
                               unit="TFLOP/s", frac=achieved / R.MI355X_BF16_FLOPS_PER_S,
                               traffic=R.recorded_traffic(counter_summary(name)),
                               kernel=GATE_UP_KERNEL[name],
                               algorithmic_flops_per_launch=flops)
    # the whole layer against both peaks (algorithmic bytes with the realized U)
    if latent:
        lb = sum(R.latent_layer_bytes(T, D, s.d, s.E, s.F, u) for u in U) / len(U)
        lf = R.latent_layer_flops(T, D, s.d, s.k, s.F)
    else:
        lb = sum(R.layer_bytes(T, s.d, s.E, s.F, u, nv=nv) for u in U) / len(U)
        lf = R.layer_flops(T, s.d, s.k, s.F)
    res["layer_hbm_frac"] = lb / (elapsed / steps) / R.MI355X_HBM_BYTES_PER_S
    res["layer_mfma_frac"] = lf / (elapsed / steps) / R.MI355X_BF16_FLOPS_PER_S
    log(json.dumps(res))
    return res, host, T


def cpu_baseline(host, T, seconds):
    """The oracle as it is, on the host cores, over whole steps of the same workload."""
    import oracle

    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    n = 0
    t0 = time.perf_counter()
    while True:
        if hasattr(host, "scales16"):  # 16-block weight format
            oracle.moe_forward_nv(host.x[:T], host.router_w, host.w_packed, host.scales16, host.gscale,
                                  host.alpha, host.beta, host.k, eps=host.eps)
        elif hasattr(host, "wc"):  # latent-width variant
            oracle.latent_forward(host.x[:T], host.router_w, host.wc, host.w_packed, host.scales,
                                  host.we, host.alpha, host.beta, host.k, eps=host.eps)
        else:
            oracle.moe_forward(host.x[:T], host.router_w, host.w_packed, host.scales, host.alpha,
                               host.beta, host.k, eps=host.eps)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return dict(value=n * T / el, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{n} full steps of the workload ({n * T} tokens, weight set 0), {el:.1f} s")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the layer's multi-GPU sharding is described in DESIGN.md but not built", file=sys.stderr)
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
    decode = args.workload.startswith("decode") or args.workload in DECODE_LIKE
    steps = args.steps or (200 if decode else 20)
    warmup = args.warmup if args.warmup is not None else (10 if decode else 3)
    main_res, host, T = time_workload(args.workload, steps, warmup, device)
    also = {}
    for extra in [e for e in args.also.split(",") if e and e != args.workload]:
        d2 = extra.startswith("decode") or extra in DECODE_LIKE
        r, _, _ = time_workload(extra, 200 if d2 else 10, 10 if d2 else 2, device)
        also[extra] = r
        torch.cuda.empty_cache()
    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle")
        cpu = cpu_baseline(host, T, args.cpu_seconds)
    s = host.w.expert_view().shape if args.workload in LATENT else host.shape
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
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "T": T, "d": s.d, "E": s.E,
                   **({"D": host.w.D} if args.workload in LATENT else {}),
                   "k": s.k, "F": s.F,
                   "weights": ("E2M1 + E4M3 per 16 + fp32 per matrix" if args.workload in NV
                               else "MXFP4 (E2M1 + E8M0 per 32)"),
                   "weight_sets": 4 if decode else 1,
                   "distinct_experts_mean": main_res["distinct_experts_mean"]},
        "roofline": {k: v for k, v in main_res["roofline"].items()
                     if k in ("bound", "achieved", "peak", "unit", "frac", "traffic")},
        "step_us_p10_p50_p90": main_res["step_us_p10_p50_p90"],
        "cpu_baseline": cpu,
        "also": {k: {kk: vv for kk, vv in v.items()} for k, v in also.items()},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
