"""ctypes binding of libmoe.so (C ABI in include/moe.h), argument marshalling only.

The functions keep the C names.  Device buffers are torch tensors on the
current HIP device (torch supplies memory and the stream); every step of the
layer runs in the library's HIP kernels.  There is no fallback: if libmoe.so
is missing this module raises on first use.
"""
from __future__ import annotations

import ctypes as C
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "moe.h")

MOE_OK = 0
MOE_ERR_NULL = -1
MOE_ERR_SHAPE = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_ARCH = -4
MOE_ERR_HIP = -5
MOE_ERR_ALIGN = -6
MOE_ERR_SCRATCH = -7
MOE_STATIC_SCRATCH_BYTES = 32 << 20


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {moe_status_string(code)} (status {code})")
        self.code = code


class moe_dims_t(C.Structure):
    _fields_ = [("T", C.c_int32), ("d", C.c_int32), ("E", C.c_int32), ("F", C.c_int32),
                ("eps", C.c_float)]


class moe_latent_dims_t(C.Structure):
    _fields_ = [("T", C.c_int32), ("D", C.c_int32), ("d", C.c_int32), ("E", C.c_int32),
                ("F", C.c_int32), ("eps", C.c_float)]


MOE_NUM_STAGES = 6
STAGES = ("router", "topk", "group", "gemm1", "gemm2", "combine")


class moe_debug_t(C.Structure):
    _fields_ = [("ids", C.c_void_p), ("weights", C.c_void_p), ("offsets", C.c_void_p),
                ("perm", C.c_void_p), ("inv", C.c_void_p),
                ("stage_begin", C.c_void_p * MOE_NUM_STAGES),
                ("stage_end", C.c_void_p * MOE_NUM_STAGES),
                ("xn", C.c_void_p)]


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run mixture_experts_gemm_amd.build")
        L = C.CDLL(LIB_PATH)
        P = C.c_void_p
        L.moe_layer_workspace_size.argtypes = [C.POINTER(moe_dims_t), C.c_int32]
        L.moe_layer_workspace_size.restype = C.c_size_t
        L.moe_layer_forward.argtypes = [C.POINTER(moe_dims_t), P, P, P, P, P, P, C.c_int32, P, P,
                                        C.c_size_t, P, C.POINTER(moe_debug_t)]
        L.moe_layer_forward.restype = C.c_int
        L.moe_layer_forward_noalloc.argtypes = [C.POINTER(moe_dims_t), P, P, P, P, P, P, C.c_int32,
                                                P, P, C.POINTER(moe_debug_t)]
        L.moe_layer_forward_noalloc.restype = C.c_int
        L.moe_pack_weights.argtypes = [C.POINTER(moe_dims_t), P, P, P, P, P]
        L.moe_pack_weights.restype = C.c_int
        L.moe_dequant_mxfp4.argtypes = [P, P, C.c_int64, C.c_int32, P, P]
        L.moe_dequant_mxfp4.restype = C.c_int
        L.moe_latent_workspace_size.argtypes = [C.POINTER(moe_latent_dims_t), C.c_int32]
        L.moe_latent_workspace_size.restype = C.c_size_t
        L.moe_latent_forward.argtypes = [C.POINTER(moe_latent_dims_t), P, P, P, P, P, P, P, P,
                                         C.c_int32, P, P, C.c_size_t, P, C.POINTER(moe_debug_t)]
        L.moe_latent_forward.restype = C.c_int
        L.moe_block_workspace_size.argtypes = [C.POINTER(moe_dims_t), C.c_int32]
        L.moe_block_workspace_size.restype = C.c_size_t
        L.moe_block_forward.argtypes = [C.POINTER(moe_dims_t), P, P, P, P, P, P, P, P, C.c_int32, P,
                                        P, C.c_size_t, P, C.POINTER(moe_debug_t)]
        L.moe_block_forward.restype = C.c_int
        L.moe_pack_weights_nvfp4.argtypes = [C.POINTER(moe_dims_t), P, P, P, P, P]
        L.moe_pack_weights_nvfp4.restype = C.c_int
        L.moe_layer_forward_nvfp4.argtypes = [C.POINTER(moe_dims_t), P, P, P, P, P, P, P,
                                              C.c_int32, P, P, C.c_size_t, P,
                                              C.POINTER(moe_debug_t)]
        L.moe_layer_forward_nvfp4.restype = C.c_int
        L.moe_status_string.argtypes = [C.c_int]
        L.moe_status_string.restype = C.c_char_p
        _lib = L
    return _lib


def declared_functions() -> list[str]:
    """Names of the functions include/moe.h declares."""
    with open(HEADER) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)


def moe_status_string(code: int) -> str:
    return lib().moe_status_string(int(code)).decode()


def _dims(T, d, E, F, eps) -> moe_dims_t:
    return moe_dims_t(int(T), int(d), int(E), int(F), float(eps))


def moe_layer_workspace_size(T: int, d: int, E: int, F: int, k: int, eps: float = 1e-6) -> int:
    return int(lib().moe_layer_workspace_size(C.byref(_dims(T, d, E, F, eps)), int(k)))


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _check(t, name, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")


def workspace_for(T, d, E, F, k, eps=1e-6, device=None) -> torch.Tensor:
    n = moe_layer_workspace_size(T, d, E, F, k, eps)
    if n == 0 and T != 0:
        raise MoeError(MOE_ERR_SHAPE, "moe_layer_workspace_size")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device or "cuda")


def moe_pack_weights(codes, scales, d, F, *, codes_packed=None, scales_packed=None, stream=None):
    """Natural MXFP4 expert weights -> the packed layout moe_layer_forward reads.

    codes uint8 [E][3dF/2], scales uint8 [E][3dF/32] (natural row-major
    matrices gate | up | down per expert); returns (codes_packed, scales_packed)
    of the same shapes.
    """
    E = codes.shape[0]
    _check(codes, "codes", torch.uint8, (E, 3 * d * F // 2))
    _check(scales, "scales", torch.uint8, (E, 3 * d * F // 32))
    if codes_packed is None:
        codes_packed = torch.empty_like(codes)
    if scales_packed is None:
        scales_packed = torch.empty_like(scales)
    _check(codes_packed, "codes_packed", torch.uint8, (E, 3 * d * F // 2))
    _check(scales_packed, "scales_packed", torch.uint8, (E, 3 * d * F // 32))
    rc = lib().moe_pack_weights(C.byref(_dims(0, d, E, F, 1e-6)), _ptr(codes), _ptr(scales),
                                _ptr(codes_packed), _ptr(scales_packed), _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_pack_weights")
    return codes_packed, scales_packed


def moe_layer_forward(x, router_w, expert_w_packed, scales, alpha, beta, k, *, F=None,
                      eps=1e-6, s_out=None, workspace=None, stream=None, debug=None):
    """Runs the layer; returns s_out (bf16 [T][d]).

    x bf16 [T][d]; router_w fp32 [E][d]; expert_w_packed uint8 [E][3dF/2] and
    scales uint8 [E][3dF/32], both as written by moe_pack_weights; alpha,
    beta fp32 [d].  debug: optional dict of preallocated device tensors among
    ids/weights/offsets/perm/inv, and "events": {stage: (begin, end)}.
    """
    T, d = x.shape
    E = router_w.shape[0]
    if F is None:
        F = expert_w_packed.shape[1] * 2 // (3 * d)
    _check(x, "x", torch.bfloat16, (T, d))
    _check(router_w, "router_w", torch.float32, (E, d))
    _check(expert_w_packed, "expert_w_packed", torch.uint8, (E, 3 * d * F // 2))
    _check(scales, "scales", torch.uint8, (E, 3 * d * F // 32))
    _check(alpha, "alpha", torch.float32, (d,))
    _check(beta, "beta", torch.float32, (d,))
    if s_out is None:
        s_out = torch.empty_like(x)
    _check(s_out, "s_out", torch.bfloat16, (T, d))
    if workspace is None:
        workspace = workspace_for(T, d, E, F, k, eps, device=x.device)
    dbg = _debug_struct(debug)
    rc = lib().moe_layer_forward(C.byref(_dims(T, d, E, F, eps)), _ptr(x), _ptr(router_w),
                                 _ptr(expert_w_packed), _ptr(scales), _ptr(alpha), _ptr(beta),
                                 int(k), _ptr(s_out), _ptr(workspace), workspace.numel(),
                                 _stream(stream), C.byref(dbg) if dbg is not None else None)
    if rc != MOE_OK:
        raise MoeError(rc, "moe_layer_forward")
    return s_out


def moe_layer_forward_noalloc(x, router_w, expert_w_packed, scales, alpha, beta, k, *, F=None,
                              eps=1e-6, s_out=None, stream=None, debug=None):
    """moe_layer_forward on the library's static scratch (no workspace, no
    allocation in the call; sizes up to MOE_STATIC_SCRATCH_BYTES of
    workspace).  Returns s_out (bf16 [T][d])."""
    T, d = x.shape
    E = router_w.shape[0]
    if F is None:
        F = expert_w_packed.shape[1] * 2 // (3 * d)
    _check(x, "x", torch.bfloat16, (T, d))
    _check(router_w, "router_w", torch.float32, (E, d))
    _check(expert_w_packed, "expert_w_packed", torch.uint8, (E, 3 * d * F // 2))
    _check(scales, "scales", torch.uint8, (E, 3 * d * F // 32))
    _check(alpha, "alpha", torch.float32, (d,))
    _check(beta, "beta", torch.float32, (d,))
    if s_out is None:
        s_out = torch.empty_like(x)
    _check(s_out, "s_out", torch.bfloat16, (T, d))
    dbg = _debug_struct(debug)
    rc = lib().moe_layer_forward_noalloc(C.byref(_dims(T, d, E, F, eps)), _ptr(x), _ptr(router_w),
                                         _ptr(expert_w_packed), _ptr(scales), _ptr(alpha),
                                         _ptr(beta), int(k), _ptr(s_out), _stream(stream),
                                         C.byref(dbg) if dbg is not None else None)
    if rc != MOE_OK:
        raise MoeError(rc, "moe_layer_forward_noalloc")
    return s_out


def moe_pack_weights_nvfp4(codes, scales16, d, F, *, codes_packed=None, scales_packed=None,
                           stream=None):
    """Natural 16-block expert weights -> the packed layout moe_layer_forward_nvfp4 reads.

    codes uint8 [E][3dF/2] (as for moe_pack_weights), scales16 uint8 E4M3
    [E][3dF/16]; returns (codes_packed, scales_packed) of the same shapes.
    """
    E = codes.shape[0]
    _check(codes, "codes", torch.uint8, (E, 3 * d * F // 2))
    _check(scales16, "scales16", torch.uint8, (E, 3 * d * F // 16))
    if codes_packed is None:
        codes_packed = torch.empty_like(codes)
    if scales_packed is None:
        scales_packed = torch.empty_like(scales16)
    _check(codes_packed, "codes_packed", torch.uint8, (E, 3 * d * F // 2))
    _check(scales_packed, "scales_packed", torch.uint8, (E, 3 * d * F // 16))
    rc = lib().moe_pack_weights_nvfp4(C.byref(_dims(0, d, E, F, 1e-6)), _ptr(codes), _ptr(scales16),
                                      _ptr(codes_packed), _ptr(scales_packed), _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_pack_weights_nvfp4")
    return codes_packed, scales_packed


def moe_layer_forward_nvfp4(x, router_w, expert_w_packed, scales16, gscale, alpha, beta, k, *,
                            F=None, eps=1e-6, s_out=None, workspace=None, stream=None, debug=None):
    """The layer on 16-block weights; returns s_out (bf16 [T][d]).

    As moe_layer_forward, with scales16 uint8 [E][3dF/16] from
    moe_pack_weights_nvfp4 and gscale fp32 [E][3] (gate, up, down).
    """
    T, d = x.shape
    E = router_w.shape[0]
    if F is None:
        F = expert_w_packed.shape[1] * 2 // (3 * d)
    _check(x, "x", torch.bfloat16, (T, d))
    _check(router_w, "router_w", torch.float32, (E, d))
    _check(expert_w_packed, "expert_w_packed", torch.uint8, (E, 3 * d * F // 2))
    _check(scales16, "scales16", torch.uint8, (E, 3 * d * F // 16))
    _check(gscale, "gscale", torch.float32, (E, 3))
    _check(alpha, "alpha", torch.float32, (d,))
    _check(beta, "beta", torch.float32, (d,))
    if s_out is None:
        s_out = torch.empty_like(x)
    _check(s_out, "s_out", torch.bfloat16, (T, d))
    if workspace is None:
        workspace = workspace_for(T, d, E, F, k, eps, device=x.device)
    dbg = _debug_struct(debug)
    rc = lib().moe_layer_forward_nvfp4(C.byref(_dims(T, d, E, F, eps)), _ptr(x), _ptr(router_w),
                                       _ptr(expert_w_packed), _ptr(scales16), _ptr(gscale),
                                       _ptr(alpha), _ptr(beta), int(k), _ptr(s_out),
                                       _ptr(workspace), workspace.numel(), _stream(stream),
                                       C.byref(dbg) if dbg is not None else None)
    if rc != MOE_OK:
        raise MoeError(rc, "moe_layer_forward_nvfp4")
    return s_out


def _latent_dims(T, D, d, E, F, eps) -> moe_latent_dims_t:
    return moe_latent_dims_t(int(T), int(D), int(d), int(E), int(F), float(eps))


def moe_latent_workspace_size(T, D, d, E, F, k, eps=1e-6) -> int:
    return int(lib().moe_latent_workspace_size(C.byref(_latent_dims(T, D, d, E, F, eps)), int(k)))


def _debug_struct(debug):
    """moe_debug_t from a dict of preallocated device tensors (ids, weights,
    offsets, perm, inv, xn) and "events": {stage: (begin, end)} pairs of
    torch.cuda.Event whose HIP events already exist."""
    if debug is None:
        return None
    dbg = moe_debug_t(*(_ptr(debug.get(n)) for n in ("ids", "weights", "offsets", "perm", "inv")))
    for i, name in enumerate(STAGES):
        ev = debug.get("events", {}).get(name)
        if ev is not None:
            dbg.stage_begin[i] = ev[0].cuda_event
            dbg.stage_end[i] = ev[1].cuda_event
    dbg.xn = _ptr(debug.get("xn"))
    return dbg


def moe_latent_forward(x, router_w, w_narrow, expert_w_packed, scales, w_widen, alpha, beta, k, *,
                       F, eps=1e-6, s_out=None, workspace=None, stream=None, debug=None):
    """Latent-width variant; returns s_out (bf16 [T][D]).

    x bf16 [T][D]; router_w fp32 [E][D]; w_narrow bf16 [d][D]; experts packed
    for width d (uint8 [E][3dF/2], [E][3dF/32]); w_widen bf16 [D][d]; alpha,
    beta fp32 [D].
    """
    T, D = x.shape
    d = w_narrow.shape[0]
    E = router_w.shape[0]
    _check(x, "x", torch.bfloat16, (T, D))
    _check(router_w, "router_w", torch.float32, (E, D))
    _check(w_narrow, "w_narrow", torch.bfloat16, (d, D))
    _check(expert_w_packed, "expert_w_packed", torch.uint8, (E, 3 * d * F // 2))
    _check(scales, "scales", torch.uint8, (E, 3 * d * F // 32))
    _check(w_widen, "w_widen", torch.bfloat16, (D, d))
    _check(alpha, "alpha", torch.float32, (D,))
    _check(beta, "beta", torch.float32, (D,))
    if s_out is None:
        s_out = torch.empty_like(x)
    _check(s_out, "s_out", torch.bfloat16, (T, D))
    if workspace is None:
        n = moe_latent_workspace_size(T, D, d, E, F, k, eps)
        if n == 0 and T != 0:
            raise MoeError(MOE_ERR_SHAPE, "moe_latent_workspace_size")
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=x.device)
    dbg = _debug_struct(debug)
    rc = lib().moe_latent_forward(C.byref(_latent_dims(T, D, d, E, F, eps)), _ptr(x), _ptr(router_w),
                                  _ptr(w_narrow), _ptr(expert_w_packed), _ptr(scales), _ptr(w_widen),
                                  _ptr(alpha), _ptr(beta), int(k), _ptr(s_out), _ptr(workspace),
                                  workspace.numel(), _stream(stream),
                                  C.byref(dbg) if dbg is not None else None)
    if rc != MOE_OK:
        raise MoeError(rc, "moe_latent_forward")
    return s_out


def moe_block_workspace_size(T, d, E, F, k, eps=1e-6) -> int:
    return int(lib().moe_block_workspace_size(C.byref(_dims(T, d, E, F, eps)), int(k)))


def moe_block_forward(x, gamma_pre, router_w, expert_w_packed, scales, gamma_post, alpha, beta, k, *,
                      F=None, eps=1e-6, s_out=None, workspace=None, stream=None, debug=None):
    """The block with its stream norms; returns s_out (bf16 [T][d]).

    x (the stream) bf16 [T][d]; gamma_pre, gamma_post, alpha, beta fp32 [d];
    router_w and the packed experts as moe_layer_forward.
    """
    T, d = x.shape
    E = router_w.shape[0]
    if F is None:
        F = expert_w_packed.shape[1] * 2 // (3 * d)
    _check(x, "x", torch.bfloat16, (T, d))
    _check(gamma_pre, "gamma_pre", torch.float32, (d,))
    _check(router_w, "router_w", torch.float32, (E, d))
    _check(expert_w_packed, "expert_w_packed", torch.uint8, (E, 3 * d * F // 2))
    _check(scales, "scales", torch.uint8, (E, 3 * d * F // 32))
    _check(gamma_post, "gamma_post", torch.float32, (d,))
    _check(alpha, "alpha", torch.float32, (d,))
    _check(beta, "beta", torch.float32, (d,))
    if s_out is None:
        s_out = torch.empty_like(x)
    _check(s_out, "s_out", torch.bfloat16, (T, d))
    if workspace is None:
        n = moe_block_workspace_size(T, d, E, F, k, eps)
        if n == 0 and T != 0:
            raise MoeError(MOE_ERR_SHAPE, "moe_block_workspace_size")
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=x.device)
    dbg = _debug_struct(debug)
    rc = lib().moe_block_forward(C.byref(_dims(T, d, E, F, eps)), _ptr(x), _ptr(gamma_pre),
                                 _ptr(router_w), _ptr(expert_w_packed), _ptr(scales), _ptr(gamma_post),
                                 _ptr(alpha), _ptr(beta), int(k), _ptr(s_out), _ptr(workspace),
                                 workspace.numel(), _stream(stream),
                                 C.byref(dbg) if dbg is not None else None)
    if rc != MOE_OK:
        raise MoeError(rc, "moe_block_forward")
    return s_out


def moe_dequant_mxfp4(codes, scales, K, out=None, stream=None):
    """codes uint8 [rows][K/2], scales uint8 [rows][K/32] -> bf16 [rows][K]."""
    rows = codes.shape[0]
    _check(codes, "codes", torch.uint8, (rows, K // 2))
    _check(scales, "scales", torch.uint8, (rows, K // 32))
    if out is None:
        out = torch.empty(rows, K, dtype=torch.bfloat16, device=codes.device)
    _check(out, "out", torch.bfloat16, (rows, K))
    rc = lib().moe_dequant_mxfp4(_ptr(codes), _ptr(scales), rows, int(K), _ptr(out), _stream(stream))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_dequant_mxfp4")
    return out
