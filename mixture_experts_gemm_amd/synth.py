"""Seeded synthetic inputs for the MoE expert layer.

This module is shared by the GPU path's tests/benchmark and by the CPU
oracle's tests.  It only draws random numbers and lays them out in the
layer's input formats; it holds none of the layer's arithmetic (no router
selection, no expert FFN, no normalisation, no combine).

The one check it makes on the numbers it draws is an input precondition:
every token's five-and-up largest router scores must be separated by a
margin (1e-4 by default), so that the top-k choice is decided the same way
by any summation order of the fp32 score.  The scores for that check are
a float64 library matmul followed by a library sort; tokens that violate
the margin are redrawn from their own substream.

Workloads (the page "Muse Spark Open を段階的に分解する" (animemo.app) gives
the model shape: token width 8,192 (section ①), 256 experts with top-8
routing (section ⑧), 4-bit block-scaled expert weights (section ⑪)):

  tiny      T=64,    d=256,  E=8,   k=2, F=512,  seed 0
  decode    T=1 / 4, d=8192, E=256, k=8, F=2048, seed 1
  prefill   T=4096,  same shape, uniform routing, seed 2
  skewed    T=16384, same shape, Zipf(1.2)-biased routing, seed 3
  stack     4 chained layers, T=8192, same shape, seed 4 (substream per layer)
  ep753     one GPU's share under 8-way expert parallelism (section ⑫: the 256
  ep3012    experts spread over 8 GPUs, 32 each; section ⑭: 753- and
            3,012-token batches): E=32 local experts, each routed (token,
            expert) pair one row, so k=1 and T = 753 / 3,012 rows (about 24 /
            94 rows per expert); seeds 5 / 6

The latent-width variant's workloads (latent_tiny, latent1/4, latent_prefill)
are described with LATENT_WORKLOADS below.

Value distributions: x = bf16(N(0,1)); router weights fp32 N(0, 0.02^2);
expert weight bytes uniform over 0..255 (so both FP4 E2M1 nibbles are
uniform over the 16 codes, -0 included); E8M0 scale bytes uniform over
119..123 (2^-8 .. 2^-4); alpha, beta fp32 U(0.5, 1.5).

Every array is drawn from numpy PCG64 seeded with
SeedSequence([seed, layer, tag, index]) so that any part (one expert's
weights, one token's redraw) can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# substream tags
(_TAG_X, _TAG_WR, _TAG_W, _TAG_S, _TAG_AB, _TAG_ZIPF, _TAG_REDRAW, _TAG_WC, _TAG_WE,
 _TAG_GAIN, _TAG_S16, _TAG_GS, _TAG_OUTLIER) = range(13)

SCALE_LO, SCALE_HI = 119, 123          # E8M0 bytes: 2^-8 .. 2^-4
GAP_DEFAULT = 1e-4
ZIPF_S = 1.2
# Gain on the Zipf bias channel; with it the 8 most-loaded experts of the
# skewed workload hold about 40% of the token slots (checked by a test).
ZIPF_GAIN = 0.95


@dataclasses.dataclass(frozen=True)
class Shape:
    T: int
    d: int
    E: int
    k: int
    F: int

    @property
    def S(self) -> int:
        return self.T * self.k

    @property
    def expert_bytes(self) -> int:
        """Packed FP4 bytes of one expert: gate, up ([F][d/2] each), down [d][F/2]."""
        return 3 * self.d * self.F // 2

    @property
    def expert_scale_bytes(self) -> int:
        """E8M0 bytes of one expert: gate, up ([F][d/32] each), down [d][F/32]."""
        return 3 * self.d * self.F // 32


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: Shape
    seed: int
    layers: int = 1
    zipf: bool = False


WORKLOADS = {
    "tiny": Workload("tiny", Shape(64, 256, 8, 2, 512), 0),
    "decode1": Workload("decode1", Shape(1, 8192, 256, 8, 2048), 1),
    "decode4": Workload("decode4", Shape(4, 8192, 256, 8, 2048), 1),
    "prefill": Workload("prefill", Shape(4096, 8192, 256, 8, 2048), 2),
    "skewed": Workload("skewed", Shape(16384, 8192, 256, 8, 2048), 3, zipf=True),
    "stack": Workload("stack", Shape(8192, 8192, 256, 8, 2048), 4, layers=4),
    "ep753": Workload("ep753", Shape(753, 8192, 32, 1, 2048), 5),
    "ep3012": Workload("ep3012", Shape(3012, 8192, 32, 1, 2048), 6),
}


def _rng(*entropy: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(entropy))))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _draw_x_rows(seed: int, layer: int, d: int, tokens: np.ndarray, attempt: np.ndarray | None,
                 base: np.ndarray | None = None) -> np.ndarray:
    """x rows as bf16 bits; row t drawn from its own redraw substream when attempt[t] > 0."""
    out = np.empty((len(tokens), d), dtype=np.uint16)
    for r, t in enumerate(tokens):
        a = 0 if attempt is None else int(attempt[r])
        if a == 0 and base is not None:
            out[r] = base[r]
            continue
        g = _rng(seed, layer, _TAG_REDRAW, int(t), a)
        out[r] = f32_to_bf16_bits(g.standard_normal(d, dtype=np.float32))
    return out


def _gap_violations(x_bits: np.ndarray, wr: np.ndarray, k: int, gap: float) -> np.ndarray:
    """Precondition check: rows whose sorted float64 scores of ranks 1..k+1 are closer than gap."""
    E = wr.shape[0]
    scores = bf16_bits_to_f32(x_bits).astype(np.float64) @ wr.astype(np.float64).T
    m = min(k + 1, E)
    if m < 2:
        return np.zeros(len(x_bits), dtype=bool)
    top = -np.sort(-scores, axis=1)[:, :m]
    return np.any(top[:, :-1] - top[:, 1:] < gap, axis=1)


def zipf_rank_of_expert(seed: int, layer: int, E: int) -> np.ndarray:
    """Seeded permutation: rank (1..E) of each expert in the Zipf popularity order."""
    return _rng(seed, layer, _TAG_ZIPF, 0).permutation(E) + 1


def make_router(w: Workload, layer: int = 0) -> np.ndarray:
    s = w.shape
    wr = _rng(w.seed, layer, _TAG_WR, 0).standard_normal((s.E, s.d), dtype=np.float32)
    wr *= np.float32(0.02)
    if w.zipf:
        # bias channel 0: the token side carries 1.0 there, so expert e's
        # score gains gain * log(r_e^-s), a Zipf(s) prior over experts
        r = zipf_rank_of_expert(w.seed, layer, s.E).astype(np.float64)
        wr[:, 0] = (ZIPF_GAIN * (-ZIPF_S) * np.log(r)).astype(np.float32)
    return wr


def outlier_rows(x_bits: np.ndarray, seed: int, layer: int, tokens: np.ndarray,
                 attempt: int = 0) -> np.ndarray:
    """Hard activation blocks for the block-scaled activation splits, applied
    to bf16 rows (powers of two only, so every value stays exact):
      * in every 32-value block one seeded channel is multiplied by 2^u,
        u uniform over 8..12 (one large value per block, as in activation
        outlier channels);
      * in a seeded quarter of the blocks, half of the other values are
        multiplied by 2^-14 (values far below the block maximum).
    Row r is transformed from its own substream (seed, layer, token, attempt)."""
    out = x_bits.copy()
    T, d = out.shape
    nb = d // 32
    for r in range(T):
        g = _rng(seed, layer, _TAG_OUTLIER, int(tokens[r]), attempt)
        f = bf16_bits_to_f32(out[r]).reshape(nb, 32).astype(np.float32)
        ch = g.integers(0, 32, size=nb)
        up = g.integers(8, 13, size=nb)
        f[np.arange(nb), ch] *= np.exp2(up).astype(np.float32)
        low = g.random(nb) < 0.25
        half = g.random((nb, 32)) < 0.5
        half[np.arange(nb), ch] = False
        f[low[:, None] & half] *= np.float32(2.0 ** -14)
        out[r] = f32_to_bf16_bits(f.reshape(d))
    return out


def make_tokens(w: Workload, wr: np.ndarray, layer: int = 0, T: int | None = None,
                gap: float = GAP_DEFAULT, max_attempts: int = 64,
                outliers: bool = False) -> np.ndarray:
    """x as bf16 bits [T][d], every row meeting the router margin precondition
    (with outliers=True, after outlier_rows; redrawn rows are transformed too)."""
    s = w.shape
    T = s.T if T is None else T
    g = _rng(w.seed, layer, _TAG_X, 0)
    x = f32_to_bf16_bits(g.standard_normal((T, s.d), dtype=np.float32))
    if outliers:
        x = outlier_rows(x, w.seed, layer, np.arange(T))
    if w.zipf:
        x[:, 0] = 0x3F80  # 1.0: the bias channel
    if gap <= 0:
        return x
    bad = np.nonzero(_gap_violations(x, wr, s.k, gap))[0]
    attempt = 0
    while len(bad) and attempt < max_attempts:
        attempt += 1
        rows = _draw_x_rows(w.seed, layer, s.d, bad, np.full(len(bad), attempt))
        if outliers:
            rows = outlier_rows(rows, w.seed, layer, bad, attempt)
        if w.zipf:
            rows[:, 0] = 0x3F80
        x[bad] = rows
        still = _gap_violations(x[bad], wr, s.k, gap)
        bad = bad[still]
    if len(bad):
        raise RuntimeError(f"could not meet the router margin for {len(bad)} tokens")
    return x


def _expert_bytes(seed: int, layer: int, e: int, n: int) -> np.ndarray:
    g = _rng(seed, layer, _TAG_W, e)
    words = g.integers(0, 2**64 - 1, size=(n + 7) // 8, dtype=np.uint64, endpoint=True)
    return words.view(np.uint8)[:n]


def _expert_scales(seed: int, layer: int, e: int, n: int) -> np.ndarray:
    return _rng(seed, layer, _TAG_S, e).integers(SCALE_LO, SCALE_HI + 1, size=n, dtype=np.uint8)


def make_experts(w: Workload, layer: int = 0, threads: int = 8,
                 out_w: np.ndarray | None = None, out_s: np.ndarray | None = None):
    """Packed FP4 weights uint8 [E][3dF/2] and E8M0 scales uint8 [E][3dF/32]."""
    s = w.shape
    nb, ns = s.expert_bytes, s.expert_scale_bytes
    W = np.empty((s.E, nb), dtype=np.uint8) if out_w is None else out_w
    S = np.empty((s.E, ns), dtype=np.uint8) if out_s is None else out_s

    def one(e):
        W[e] = _expert_bytes(w.seed, layer, e, nb)
        S[e] = _expert_scales(w.seed, layer, e, ns)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(one, range(s.E)))
    return W, S


# ---------------------------------------------------------------------------
# The 16-block format ("Muse Spark Open を段階的に分解する", section ⑪: one
# small scale shared by 16 values, about 4.5 bits a value), read as one E4M3
# byte per 16 values and one fp32 scale per matrix.  Any workload above can
# be drawn in it: x, the router, alpha / beta and the code bytes are the
# workload's own; the scales are drawn instead of the E8M0 bytes:
#   E4M3 bytes: exponent field uniform over 4..8 (2^-3 .. 2^1), mantissa
#     uniform over 0..7, positive; with probability 1/32 a subnormal byte
#     (0x00..0x07, 0x00 a zero block) and, independently, with probability
#     1/32 the sign bit set;
#   matrix scales: fp32 U(0.75, 1.25) * 2^-5,
# so the weight magnitudes match the MXFP4 draw's (2^-8 .. 2^-4 per block).
# ---------------------------------------------------------------------------
NV_EXP_LO, NV_EXP_HI = 4, 8


def _expert_scales16(seed: int, layer: int, e: int, n: int) -> np.ndarray:
    g = _rng(seed, layer, _TAG_S16, e)
    ex = g.integers(NV_EXP_LO, NV_EXP_HI + 1, size=n, dtype=np.uint8)
    mt = g.integers(0, 8, size=n, dtype=np.uint8)
    b = (ex << 3) | mt
    sub = g.random(n) < 1.0 / 32
    b[sub] = mt[sub]
    neg = g.random(n) < 1.0 / 32
    b[neg] |= 0x80
    return b.astype(np.uint8)


def make_experts_nv(w: Workload, layer: int = 0, threads: int = 8):
    """Codes uint8 [E][3dF/2] (the workload's own), E4M3 scales uint8 [E][3dF/16],
    matrix scales fp32 [E][3] (gate, up, down)."""
    s = w.shape
    nb, ns = s.expert_bytes, 3 * s.d * s.F // 16
    W = np.empty((s.E, nb), dtype=np.uint8)
    S = np.empty((s.E, ns), dtype=np.uint8)

    def one(e):
        W[e] = _expert_bytes(w.seed, layer, e, nb)
        S[e] = _expert_scales16(w.seed, layer, e, ns)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(one, range(s.E)))
    g = _rng(w.seed, layer, _TAG_GS, 0)
    G = ((g.random((s.E, 3)) * 0.5 + 0.75) * 2.0 ** -5).astype(np.float32)
    return W, S, G


def make_gates(w: Workload, layer: int = 0):
    g = _rng(w.seed, layer, _TAG_AB, 0)
    alpha = (g.random(w.shape.d, dtype=np.float32) + np.float32(0.5)).astype(np.float32)
    beta = (g.random(w.shape.d, dtype=np.float32) + np.float32(0.5)).astype(np.float32)
    return alpha, beta


def make_norm_gains(w: Workload, layer: int = 0):
    """Learned gains of the block's two stream norms, fp32 [d] each, U(0.5, 1.5)."""
    g = _rng(w.seed, layer, _TAG_GAIN, 0)
    pre = (g.random(w.shape.d, dtype=np.float32) + np.float32(0.5)).astype(np.float32)
    post = (g.random(w.shape.d, dtype=np.float32) + np.float32(0.5)).astype(np.float32)
    return pre, post


@dataclasses.dataclass
class LayerInputs:
    shape: Shape
    x: np.ndarray          # uint16 bf16 bits [T][d]
    router_w: np.ndarray   # float32 [E][d]
    w_packed: np.ndarray   # uint8 [E][3dF/2]
    scales: np.ndarray     # uint8 [E][3dF/32]
    alpha: np.ndarray      # float32 [d]
    beta: np.ndarray       # float32 [d]
    k: int
    eps: float = 1e-6


def make_layer(name_or_w, layer: int = 0, T: int | None = None, gap: float = GAP_DEFAULT,
               threads: int = 8, with_tokens: bool = True, outliers: bool = False) -> LayerInputs:
    w = WORKLOADS[name_or_w] if isinstance(name_or_w, str) else name_or_w
    s = w.shape
    if T is not None:
        s = dataclasses.replace(s, T=T)
        w = dataclasses.replace(w, shape=s)
    wr = make_router(w, layer)
    x = (make_tokens(w, wr, layer, gap=gap, outliers=outliers) if with_tokens
         else np.zeros((0, s.d), np.uint16))
    W, S = make_experts(w, layer, threads=threads)
    a, b = make_gates(w, layer)
    return LayerInputs(s, x, wr, W, S, a, b, s.k)


@dataclasses.dataclass
class NvLayerInputs:
    shape: Shape
    x: np.ndarray          # uint16 bf16 bits [T][d]
    router_w: np.ndarray   # float32 [E][d]
    w_packed: np.ndarray   # uint8 [E][3dF/2] codes
    scales16: np.ndarray   # uint8 [E][3dF/16] E4M3
    gscale: np.ndarray     # float32 [E][3]
    alpha: np.ndarray
    beta: np.ndarray
    k: int
    eps: float = 1e-6


def make_layer_nv(name_or_w, layer: int = 0, T: int | None = None, gap: float = GAP_DEFAULT,
                  threads: int = 8, with_tokens: bool = True, outliers: bool = False) -> NvLayerInputs:
    """A workload's layer with its expert weights drawn in the 16-block format."""
    w = WORKLOADS[name_or_w] if isinstance(name_or_w, str) else name_or_w
    s = w.shape
    if T is not None:
        s = dataclasses.replace(s, T=T)
        w = dataclasses.replace(w, shape=s)
    wr = make_router(w, layer)
    x = (make_tokens(w, wr, layer, gap=gap, outliers=outliers) if with_tokens
         else np.zeros((0, s.d), np.uint16))
    W, S, G = make_experts_nv(w, layer, threads=threads)
    a, b = make_gates(w, layer)
    return NvLayerInputs(s, x, wr, W, S, G, a, b, s.k)


def custom_workload(T: int, d: int, E: int, k: int, F: int, seed: int, zipf: bool = False) -> Workload:
    return Workload(f"custom_T{T}_d{d}_E{E}_k{k}_F{F}_s{seed}", Shape(T, d, E, k, F), seed, zipf=zipf)


# ---------------------------------------------------------------------------
# Latent-width variant ("Muse Spark Open を段階的に分解する", section ⑨): the
# token (width D) is narrowed by a shared matrix to the experts' width d,
# the experts run at d, and a second shared matrix widens their weighted
# sum back to D.  The page gives D = 8,192, d = 4,096 and 4,096 x 4,096
# gate / up / down matrices.
#
#   latent_tiny     T=64,   D=512,  d=256,  E=8,   k=2, F=256,  seed 7
#   latent1/4       T=1/4,  D=8192, d=4096, E=256, k=8, F=4096, seed 8
#   latent_prefill  T=4096, same, seed 9
#
# Shared matrices bf16: Wc [d][D] = bf16(N(0, 1/D)), We [D][d] = bf16(N(0, 1/d)),
# so the narrowed token and the widened sum stay near unit scale.  x, the
# router and the experts are drawn as for the full-width workloads (the
# router and the margin precondition at width D, the experts at width d).
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class LatentWorkload:
    name: str
    T: int
    D: int
    d: int
    E: int
    k: int
    F: int
    seed: int

    def token_view(self) -> Workload:
        """The full-width view: token width D (router, tokens, gate vectors)."""
        return Workload(self.name, Shape(self.T, self.D, self.E, self.k, self.F), self.seed)

    def expert_view(self) -> Workload:
        """The experts' view: width d (expert weights)."""
        return Workload(self.name, Shape(self.T, self.d, self.E, self.k, self.F), self.seed)


LATENT_WORKLOADS = {
    "latent_tiny": LatentWorkload("latent_tiny", 64, 512, 256, 8, 2, 256, 7),
    "latent1": LatentWorkload("latent1", 1, 8192, 4096, 256, 8, 4096, 8),
    "latent4": LatentWorkload("latent4", 4, 8192, 4096, 256, 8, 4096, 8),
    "latent_prefill": LatentWorkload("latent_prefill", 4096, 8192, 4096, 256, 8, 4096, 9),
}


@dataclasses.dataclass
class LatentInputs:
    w: LatentWorkload
    x: np.ndarray          # uint16 bf16 bits [T][D]
    router_w: np.ndarray   # float32 [E][D]
    wc: np.ndarray         # uint16 bf16 bits [d][D]
    w_packed: np.ndarray   # uint8 [E][3dF/2] (natural layout, width d)
    scales: np.ndarray     # uint8 [E][3dF/32]
    we: np.ndarray         # uint16 bf16 bits [D][d]
    alpha: np.ndarray      # float32 [D]
    beta: np.ndarray       # float32 [D]
    k: int
    eps: float = 1e-6


def make_shared(w: LatentWorkload, layer: int = 0):
    """The two shared matrices as bf16 bits: Wc [d][D] and We [D][d]."""
    gc = _rng(w.seed, layer, _TAG_WC, 0)
    wc = gc.standard_normal((w.d, w.D), dtype=np.float32) * np.float32(1.0 / math.sqrt(w.D))
    ge = _rng(w.seed, layer, _TAG_WE, 0)
    we = ge.standard_normal((w.D, w.d), dtype=np.float32) * np.float32(1.0 / math.sqrt(w.d))
    return f32_to_bf16_bits(wc), f32_to_bf16_bits(we)


def make_latent_layer(name_or_w, layer: int = 0, T: int | None = None, gap: float = GAP_DEFAULT,
                      threads: int = 8) -> LatentInputs:
    w = LATENT_WORKLOADS[name_or_w] if isinstance(name_or_w, str) else name_or_w
    if T is not None:
        w = dataclasses.replace(w, T=T)
    tv, ev = w.token_view(), w.expert_view()
    wr = make_router(tv, layer)
    x = make_tokens(tv, wr, layer, gap=gap)
    W, S = make_experts(ev, layer, threads=threads)
    a, b = make_gates(tv, layer)
    wc, we = make_shared(w, layer)
    return LatentInputs(w, x, wr, wc, W, S, we, a, b, w.k)
