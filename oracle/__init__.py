"""CPU oracle for the MoE expert layer -- TEST INFRASTRUCTURE ONLY.

Plain C (oracle.c, built by oracle/build.py into liboracle.so) wrapped with
ctypes.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import this package; the product library never does.

Each wrapper names the step of oracle.c it runs (O1-O8 there).  Every
function here is pinned by a CPU test to something other than itself.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_P = C.c_void_p
_I = C.c_int
_I64 = C.c_int64


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            from . import build as _b
            _b.build()
        L = C.CDLL(_LIB)
        L.oracle_bf16_to_double.argtypes = [C.c_uint16]
        L.oracle_bf16_to_double.restype = C.c_double
        L.oracle_double_to_bf16.argtypes = [C.c_double]
        L.oracle_double_to_bf16.restype = C.c_uint16
        L.oracle_e2m1.argtypes = [C.c_uint]
        L.oracle_e2m1.restype = C.c_double
        L.oracle_e8m0.argtypes = [C.c_uint]
        L.oracle_e8m0.restype = C.c_double
        L.oracle_dequant_rows.argtypes = [_I64, _I64, _P, _P, _P]
        L.oracle_dequant_rows.restype = None
        L.oracle_e4m3.argtypes = [C.c_uint]
        L.oracle_e4m3.restype = C.c_double
        L.oracle_dequant_rows_nv.argtypes = [_I64, _I64, _P, _P, C.c_double, _P]
        L.oracle_dequant_rows_nv.restype = None
        L.oracle_expert_nv.argtypes = [_I, _I, _P, _P, _P, _P, C.c_double, _P, _P]
        L.oracle_expert_nv.restype = C.c_double
        L.oracle_moe_forward_nv.argtypes = [_I, _I, _I, _I, _I, C.c_double, _P, _P, _P, _P, _P,
                                            _P, _P, _I, _P, _P, _P, _P]
        L.oracle_moe_forward_nv.restype = _I
        L.oracle_router_scores.argtypes = [_I, _I, _I, _P, _P, _P]
        L.oracle_router_scores.restype = None
        L.oracle_topk_softmax.argtypes = [_I, _I, _I, _P, _P, _P]
        L.oracle_topk_softmax.restype = None
        L.oracle_group.argtypes = [_I, _I, _I, _P, _P, _P, _P, _P]
        L.oracle_group.restype = None
        L.oracle_expert.argtypes = [_I, _I, _P, _P, _P, C.c_double, _P, _P]
        L.oracle_expert.restype = C.c_double
        L.oracle_moe_forward.argtypes = [_I, _I, _I, _I, _I, C.c_double, _P, _P, _P, _P, _P, _P,
                                         _I, _P, _P, _P, _P]
        L.oracle_moe_forward.restype = _I
        L.oracle_latent_forward.argtypes = [_I, _I, _I, _I, _I, _I, C.c_double, _P, _P, _P, _P, _P,
                                            _P, _P, _P, _I, _P, _P, _P, _P]
        L.oracle_latent_forward.restype = _I
        L.oracle_block_forward.argtypes = [_I, _I, _I, _I, _I, C.c_double, _P, _P, _P, _P, _P, _P,
                                           _P, _P, _I, _P, _P, _P, _P, _P]
        L.oracle_block_forward.restype = _I
        L.oracle_block_prenorm.argtypes = [_I, _I, C.c_double, _P, _P, _I, _P, _P]
        L.oracle_block_prenorm.restype = _I
        L.oracle_set_num_threads.argtypes = [_I]
        L.oracle_set_num_threads.restype = None
        L.oracle_max_threads.argtypes = []
        L.oracle_max_threads.restype = _I
        _lib = L
    return _lib


def set_num_threads(n: int) -> None:
    """Host threads of the oracle's parallel loops from now on."""
    lib().oracle_set_num_threads(int(n))


def max_threads() -> int:
    """Host threads the oracle's parallel loops use."""
    return int(lib().oracle_max_threads())


def _p(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def bf16_to_double(bits: int) -> float:
    return lib().oracle_bf16_to_double(int(bits))


def double_to_bf16(v: float) -> int:
    return int(lib().oracle_double_to_bf16(float(v)))


def doubles_to_bf16(a: np.ndarray) -> np.ndarray:
    f = lib().oracle_double_to_bf16
    flat = np.asarray(a, dtype=np.float64).ravel()
    return np.fromiter((f(float(v)) for v in flat), dtype=np.uint16, count=flat.size).reshape(np.shape(a))


def e2m1(code: int) -> float:
    return lib().oracle_e2m1(int(code))


def e8m0(s: int) -> float:
    return lib().oracle_e8m0(int(s))


def dequant_rows(codes: np.ndarray, scales: np.ndarray, K: int) -> np.ndarray:
    """O6 decode: rows of K MXFP4 elements -> float64 [rows][K]."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    rows = codes.size // (K // 2)
    assert codes.size == rows * K // 2 and scales.size == rows * K // 32
    out = np.empty((rows, K), dtype=np.float64)
    lib().oracle_dequant_rows(rows, K, _p(codes), _p(scales), _p(out))
    return out


def e4m3(b: int) -> float:
    """NV1: one E4M3 scale byte -> its value."""
    return lib().oracle_e4m3(int(b))


def dequant_rows_nv(codes: np.ndarray, scales16: np.ndarray, K: int, g: float = 1.0) -> np.ndarray:
    """NV2 decode: rows of K elements in the 16-block format -> float64 [rows][K]."""
    codes = _c(codes, np.uint8)
    scales16 = _c(scales16, np.uint8)
    rows = codes.size // (K // 2)
    assert codes.size == rows * K // 2 and scales16.size == rows * K // 16
    out = np.empty((rows, K), dtype=np.float64)
    lib().oracle_dequant_rows_nv(rows, K, _p(codes), _p(scales16), float(g), _p(out))
    return out


def expert_nv(w_e, s16_e, gs_e, x, d: int, F: int, eps: float = 1e-6):
    """NV3 (O6/O7 in the 16-block format) for one expert on one token: (o, n, ms)."""
    w_e = _c(w_e, np.uint8)
    s16_e = _c(s16_e, np.uint8)
    gs_e = _c(gs_e, np.float32)
    x = _c(x, np.float64)
    assert gs_e.size == 3
    o = np.empty(d, np.float64)
    n = np.empty(d, np.float64)
    ms = lib().oracle_expert_nv(d, F, _p(w_e), _p(s16_e), _p(gs_e), _p(x), eps, _p(o), _p(n))
    return o, n, ms


def router_scores(x_bits: np.ndarray, wr: np.ndarray) -> np.ndarray:
    """O2: fp32 scores [T][E]."""
    x_bits = _c(x_bits, np.uint16)
    wr = _c(wr, np.float32)
    T, d = x_bits.shape
    E = wr.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    lib().oracle_router_scores(T, d, E, _p(x_bits), _p(wr), _p(out))
    return out


def topk_softmax(scores: np.ndarray, k: int):
    """O3/O4: ids int32 [T][k], weights float64 [T][k]."""
    scores = _c(scores, np.float32)
    T, E = scores.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    lib().oracle_topk_softmax(T, E, k, _p(scores), _p(ids), _p(w))
    return ids, w


def group(ids: np.ndarray, E: int):
    """O5: counts [E], offsets [E+1], perm [S], inv [S]."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    inv = np.empty(T * k, np.int32)
    lib().oracle_group(T, E, k, _p(ids), _p(counts), _p(offsets), _p(perm), _p(inv))
    return counts, offsets, perm, inv


def expert(w_e: np.ndarray, s_e: np.ndarray, x: np.ndarray, d: int, F: int, eps: float = 1e-6):
    """O6/O7 for one expert on one token: (o, n, mean square of o)."""
    w_e = _c(w_e, np.uint8)
    s_e = _c(s_e, np.uint8)
    x = _c(x, np.float64)
    o = np.empty(d, np.float64)
    n = np.empty(d, np.float64)
    ms = lib().oracle_expert(d, F, _p(w_e), _p(s_e), _p(x), eps, _p(o), _p(n))
    return o, n, ms


def route(x_bits: np.ndarray, wr: np.ndarray, k: int):
    """O2-O5 on all tokens: dict with scores, ids, w, counts, offsets, perm, inv."""
    sc = router_scores(x_bits, wr)
    ids, w = topk_softmax(sc, k)
    counts, offsets, perm, inv = group(ids, wr.shape[0])
    return dict(scores=sc, ids=ids, w=w, counts=counts, offsets=offsets, perm=perm, inv=inv)


def moe_forward(x_bits, wr, w_packed, scales, alpha, beta, k, eps=1e-6, F=None, tokens=None):
    """O1-O8 on the listed tokens (all when None): (s float64 [n][d], ids, w)."""
    x_bits = _c(x_bits, np.uint16)
    wr = _c(wr, np.float32)
    w_packed = _c(w_packed, np.uint8)
    scales = _c(scales, np.uint8)
    alpha = _c(alpha, np.float32)
    beta = _c(beta, np.float32)
    T, d = x_bits.shape
    E = wr.shape[0]
    if F is None:
        F = w_packed.size // E * 2 // (3 * d)
    assert w_packed.size == E * 3 * d * F // 2 and scales.size == E * 3 * d * F // 32
    if tokens is None:
        sel = None
        n = T
    else:
        sel = _c(tokens, np.int32)
        n = sel.size
    s = np.empty((n, d), np.float64)
    ids = np.empty((n, k), np.int32)
    w = np.empty((n, k), np.float64)
    rc = lib().oracle_moe_forward(T, d, E, F, k, eps, _p(x_bits), _p(wr), _p(w_packed), _p(scales),
                                  _p(alpha), _p(beta), n, None if sel is None else _p(sel),
                                  _p(s), _p(ids), _p(w))
    if rc != 0:
        raise ValueError("oracle_moe_forward: bad arguments")
    return s, ids, w


def moe_forward_nv(x_bits, wr, w_packed, scales16, gscale, alpha, beta, k, eps=1e-6, tokens=None):
    """O1-O8 with 16-block expert weights (NV1-NV3): (s float64 [n][d], ids, w).

    scales16: E4M3 bytes, expert e at e*(3dF/16); gscale fp32 [E][3].
    """
    x_bits = _c(x_bits, np.uint16)
    wr = _c(wr, np.float32)
    w_packed = _c(w_packed, np.uint8)
    scales16 = _c(scales16, np.uint8)
    gscale = _c(gscale, np.float32)
    alpha = _c(alpha, np.float32)
    beta = _c(beta, np.float32)
    T, d = x_bits.shape
    E = wr.shape[0]
    F = w_packed.size // E * 2 // (3 * d)
    assert w_packed.size == E * 3 * d * F // 2 and scales16.size == E * 3 * d * F // 16
    assert gscale.size == 3 * E
    if tokens is None:
        sel = None
        n = T
    else:
        sel = _c(tokens, np.int32)
        n = sel.size
    s = np.empty((n, d), np.float64)
    ids = np.empty((n, k), np.int32)
    w = np.empty((n, k), np.float64)
    rc = lib().oracle_moe_forward_nv(T, d, E, F, k, eps, _p(x_bits), _p(wr), _p(w_packed),
                                     _p(scales16), _p(gscale), _p(alpha), _p(beta), n,
                                     None if sel is None else _p(sel), _p(s), _p(ids), _p(w))
    if rc != 0:
        raise ValueError("oracle_moe_forward_nv: bad arguments")
    return s, ids, w


def latent_forward(x_bits, wr, wc_bits, w_packed, scales, we_bits, alpha, beta, k, eps=1e-6,
                   tokens=None):
    """L1-L5 (latent-width variant) on the listed tokens: (s float64 [n][D], ids, w).

    x bf16 bits [T][D]; wr fp32 [E][D]; wc bf16 bits [d][D]; experts packed for
    width d; we bf16 bits [D][d]; alpha, beta fp32 [D].
    """
    x_bits = _c(x_bits, np.uint16)
    wr = _c(wr, np.float32)
    wc_bits = _c(wc_bits, np.uint16)
    we_bits = _c(we_bits, np.uint16)
    w_packed = _c(w_packed, np.uint8)
    scales = _c(scales, np.uint8)
    alpha = _c(alpha, np.float32)
    beta = _c(beta, np.float32)
    T, D = x_bits.shape
    d = wc_bits.shape[0]
    E = wr.shape[0]
    assert wc_bits.shape == (d, D) and we_bits.shape == (D, d) and wr.shape == (E, D)
    F = w_packed.size // E * 2 // (3 * d)
    assert w_packed.size == E * 3 * d * F // 2 and scales.size == E * 3 * d * F // 32
    if tokens is None:
        sel = None
        n = T
    else:
        sel = _c(tokens, np.int32)
        n = sel.size
    s = np.empty((n, D), np.float64)
    ids = np.empty((n, k), np.int32)
    w = np.empty((n, k), np.float64)
    rc = lib().oracle_latent_forward(T, D, d, E, F, k, eps, _p(x_bits), _p(wr), _p(wc_bits),
                                     _p(w_packed), _p(scales), _p(we_bits), _p(alpha), _p(beta),
                                     n, None if sel is None else _p(sel), _p(s), _p(ids), _p(w))
    if rc != 0:
        raise ValueError("oracle_latent_forward: bad arguments")
    return s, ids, w


def block_prenorm(x_bits, gamma_pre, eps=1e-6, tokens=None):
    """B1 on the listed tokens (all when None): the normalised rows as bf16 bits [n][d]."""
    x_bits = _c(x_bits, np.uint16)
    gamma_pre = _c(gamma_pre, np.float32)
    T, d = x_bits.shape
    sel = None if tokens is None else _c(tokens, np.int32)
    n = T if sel is None else sel.size
    xn = np.empty((n, d), np.uint16)
    rc = lib().oracle_block_prenorm(T, d, eps, _p(x_bits), _p(gamma_pre), n,
                                    None if sel is None else _p(sel), _p(xn))
    if rc != 0:
        raise ValueError("oracle_block_prenorm: bad arguments")
    return xn


def block_forward(x_bits, gamma_pre, wr, w_packed, scales, gamma_post, alpha, beta, k, eps=1e-6,
                  tokens=None, xn=None):
    """B1-B3 (the block with its stream norms) on the listed tokens: (s float64 [n][d], ids, w).

    xn: optional normalised rows (bf16 bits [n][d], one per listed token) used
    in place of B1's own, to check B2-B3 on exactly the rows another
    implementation computed."""
    x_bits = _c(x_bits, np.uint16)
    gamma_pre = _c(gamma_pre, np.float32)
    gamma_post = _c(gamma_post, np.float32)
    wr = _c(wr, np.float32)
    w_packed = _c(w_packed, np.uint8)
    scales = _c(scales, np.uint8)
    alpha = _c(alpha, np.float32)
    beta = _c(beta, np.float32)
    T, d = x_bits.shape
    E = wr.shape[0]
    F = w_packed.size // E * 2 // (3 * d)
    assert w_packed.size == E * 3 * d * F // 2 and scales.size == E * 3 * d * F // 32
    if tokens is None:
        sel = None
        n = T
    else:
        sel = _c(tokens, np.int32)
        n = sel.size
    s = np.empty((n, d), np.float64)
    ids = np.empty((n, k), np.int32)
    w = np.empty((n, k), np.float64)
    if xn is not None:
        xn = _c(xn, np.uint16)
        assert xn.shape == (n, d)
    rc = lib().oracle_block_forward(T, d, E, F, k, eps, _p(x_bits), _p(gamma_pre), _p(wr),
                                    _p(w_packed), _p(scales), _p(gamma_post), _p(alpha), _p(beta),
                                    n, None if sel is None else _p(sel),
                                    None if xn is None else _p(xn), _p(s), _p(ids), _p(w))
    if rc != 0:
        raise ValueError("oracle_block_forward: bad arguments")
    return s, ids, w
