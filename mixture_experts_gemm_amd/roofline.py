"""Algorithmic byte / flop accounting for the MoE expert layer.

Only what the method must move or compute is counted: the chosen experts'
weights once, the router matrix, tokens in and out, the gate vectors, and
T*k*6*d*F flops for the expert FFNs (2 flops per multiply-add, three
d x F matrices per expert).  Intermediates (h, o, permutation) and the
dense work that sparse routing avoids are excluded.

The read-versus-compute model follows "Muse Spark Open を段階的に分解する"
(animemo.app), section ⑬: an expert's time is the larger of reading its
weights and computing its tokens, the weight read does not depend on the
token count, and the two are equal at the crossover token count.
"""
from __future__ import annotations

import hashlib
import math
import os
import re

# MI355X published peaks
MI355X_HBM_BYTES_PER_S = 8.0e12
MI355X_BF16_FLOPS_PER_S = 2.5e15      # dense MFMA
MI355X_FP32_MFMA_FLOPS_PER_S = 157.3e12


def expert_params(d: int, F: int) -> int:
    """gate, up (F x d each) and down (d x F)."""
    return 3 * d * F


def block_scaled_bits(value_bits: int, block: int, scale_bits: int = 8) -> float:
    """Storage bits per value of a block-scaled format (4-bit values, one scale per block)."""
    return value_bits + scale_bits / block


def expert_bytes(d: int, F: int, bits_per_value: float) -> float:
    return expert_params(d, F) * bits_per_value / 8


def mxfp4_expert_bytes(d: int, F: int) -> int:
    """Packed bytes + E8M0 scales of one expert (32 values per scale)."""
    p = expert_params(d, F)
    return p // 2 + p // 32


def mxfp4_w1_bytes(d: int, F: int) -> int:
    """gate + up part of one expert (2F rows of d values)."""
    return 2 * F * d // 2 + 2 * F * d // 32


def mxfp4_w2_bytes(d: int, F: int) -> int:
    """down part of one expert (d rows of F values)."""
    return d * F // 2 + d * F // 32


def nvfp4_expert_bytes(d: int, F: int) -> int:
    """16-block format: codes + E4M3 scales (16 values per scale) + three fp32 matrix scales."""
    p = expert_params(d, F)
    return p // 2 + p // 16 + 12


def nvfp4_w1_bytes(d: int, F: int) -> int:
    """gate + up part of one expert in the 16-block format."""
    return 2 * F * d // 2 + 2 * F * d // 16 + 8


def flops_per_slot(d: int, F: int) -> int:
    return 2 * expert_params(d, F)


def read_time(nbytes: float, bw: float) -> float:
    return nbytes / bw


def compute_time(flops: float, rate: float) -> float:
    return flops / rate


def crossover_tokens(d: int, F: int, bits_per_value: float, bw: float, rate: float) -> float:
    """Tokens per expert at which computing equals reading the expert's weights."""
    return read_time(expert_bytes(d, F, bits_per_value), bw) / compute_time(flops_per_slot(d, F), rate)


def layer_bytes(T: int, d: int, E: int, F: int, U: int, nv: bool = False) -> int:
    """Whole-layer algorithmic bytes with U distinct experts used (nv: 16-block weights)."""
    per_expert = nvfp4_expert_bytes(d, F) if nv else mxfp4_expert_bytes(d, F)
    return (U * per_expert + E * d * 4                 # experts + fp32 router
            + 2 * d * 4                                # alpha, beta
            + 2 * T * d * 2)                           # x in, s_out out (bf16)


def layer_flops(T: int, d: int, k: int, F: int) -> int:
    return T * k * flops_per_slot(d, F)


def latent_layer_bytes(T: int, D: int, d: int, E: int, F: int, U: int) -> int:
    """Latent-width variant: experts at width d, router and gate at width D,
    plus the two shared bf16 matrices (d x D and D x d)."""
    return (U * mxfp4_expert_bytes(d, F) + E * D * 4 + 2 * D * 4 + 2 * T * D * 2
            + 2 * d * D * 2)


def latent_layer_flops(T: int, D: int, d: int, k: int, F: int) -> int:
    """Experts at width d plus the two shared products (2 T d D flops each)."""
    return T * k * flops_per_slot(d, F) + 2 * (2 * T * d * D)


def router_flops(T: int, d: int, E: int) -> int:
    return 2 * T * d * E


def gemm1_bytes(U: int, d: int, F: int, S: int) -> int:
    """gate/up kernel: chosen experts' W1, gathered token rows in, h out (bf16)."""
    return U * mxfp4_w1_bytes(d, F) + S * d * 2 + S * F * 2


def gemm1_flops(S: int, d: int, F: int) -> int:
    return 2 * S * (2 * F) * d


def gemm2_bytes(U: int, d: int, F: int, S: int) -> int:
    """down kernel: chosen experts' W2, h in, o out (bf16)."""
    return U * mxfp4_w2_bytes(d, F) + S * F * 2 + S * d * 2


def gemm2_flops(S: int, d: int, F: int) -> int:
    return 2 * S * F * d


def combinations(n: int, r: int) -> int:
    return math.comb(n, r)


# ---- recorded HBM traffic (hardware byte counters) ---------------------------

KERNEL_SOURCES = ("csrc/expert.hip", "csrc/layout.h", "csrc/device.h", "csrc/internal.h")


def kernel_source_digest() -> str:
    """sha256 over the sources of the expert kernels (the counters are only
    valid for the code they were taken on)."""
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(here, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def recorded_traffic(path: str) -> float | None:
    """HBM bytes per launch from a committed counter summary, or None when
    the summary is missing or was taken on different kernel sources.

    The summary holds lines 'traffic_bytes_per_launch: N' and
    'source_sha256: H'."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        text = f.read()
    mt = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    mh = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    if not mt or not mh or mh.group(1) != kernel_source_digest():
        return None
    return float(mt.group(1))
