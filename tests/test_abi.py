"""CPU checks of the C ABI: the library loads, exports every function the
header declares, sizes its workspace, names its status codes, and rejects bad
arguments before queuing any GPU work."""
import ctypes as C

import pytest

from mixture_experts_gemm_amd import binding as B


@pytest.fixture(scope="module")
def L():
    return B.lib()


def test_exports_every_declared_function(L):
    names = B.declared_functions()
    assert set(names) == {"moe_layer_workspace_size", "moe_layer_forward", "moe_pack_weights",
                          "moe_dequant_mxfp4", "moe_status_string", "moe_latent_workspace_size",
                          "moe_latent_forward", "moe_block_workspace_size", "moe_block_forward",
                          "moe_pack_weights_nvfp4", "moe_layer_forward_nvfp4",
                          "moe_layer_forward_noalloc"}
    for n in names:
        assert hasattr(L, n), n


def test_library_imports_no_allocator(L):
    """No entry point allocates: the library imports no HIP allocation or
    free routine at all (its workspace comes from the caller, or from the
    static scratch array of the no-allocation entry point)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", B.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    imported = {line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()}
    hip = sorted(n for n in imported if n.startswith("hip"))
    assert hip, "no HIP imports found: not the HIP library?"
    banned = [n for n in hip if "Malloc" in n or "Free" in n or "MemPool" in n or "HostRegister" in n]
    assert not banned, banned


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert B.moe_status_string(code) and B.moe_status_string(code) != "unknown status"
    assert B.moe_status_string(7) == "unknown status"
    assert B.moe_status_string(-8) == "unknown status"


def test_workspace_size():
    ws = B.moe_layer_workspace_size
    assert ws(0, 256, 8, 512, 2) > 0
    a, b = ws(64, 256, 8, 512, 2), ws(128, 256, 8, 512, 2)
    assert 0 < a < b
    big = ws(4096, 8192, 256, 2048, 8)
    S = 4096 * 8
    assert big >= S * 2048 * 2 + S * 8192 * 2
    assert ws(64, 250, 8, 512, 2) == 0       # d not a multiple of 256
    assert ws(64, 384, 8, 512, 2) == 0
    assert ws(64, 256, 8, 500, 2) == 0       # F not a multiple of 128
    assert ws(64, 256, 8, 512, 9) == 0       # k > E
    assert ws(64, 256, 8, 512, 0) == 0
    assert ws(64, 256, 1025, 512, 2) == 0    # E > 1024
    assert ws(-1, 256, 8, 512, 2) == 0
    assert ws(64, 256, 8, 512, 2, eps=float("nan")) == 0


def _call(dims, k=2, ws_bytes=1 << 30, null=None, ws_ptr=1 << 20, ptr=None):
    p = C.c_void_p(1 << 20)  # never dereferenced: every case below fails the checks first
    args = dict(x=p, router_w=p, w=p, s=p, alpha=p, beta=p, s_out=p, ws=C.c_void_p(ws_ptr))
    if null:
        args[null] = None
    args.update(ptr or {})
    return B.lib().moe_layer_forward(C.byref(dims) if dims is not None else None, args["x"],
                                     args["router_w"], args["w"], args["s"], args["alpha"],
                                     args["beta"], k, args["s_out"], args["ws"], ws_bytes, None, None)


def test_argument_errors():
    good = B.moe_dims_t(64, 256, 8, 512, 1e-6)
    assert _call(None) == B.MOE_ERR_NULL
    for name in ("x", "router_w", "w", "s", "alpha", "beta", "s_out", "ws"):
        assert _call(good, null=name) == B.MOE_ERR_NULL, name
    assert _call(B.moe_dims_t(64, 200, 8, 512, 1e-6)) == B.MOE_ERR_SHAPE
    assert _call(good, k=9) == B.MOE_ERR_SHAPE
    assert _call(B.moe_dims_t(64, 256, 8, 512, -1.0)) == B.MOE_ERR_SHAPE
    assert _call(good, ws_bytes=1024) == B.MOE_ERR_WORKSPACE
    assert _call(good, ws_ptr=(1 << 20) + 64) == B.MOE_ERR_WORKSPACE
    odd = C.c_void_p((1 << 20) + 8)
    for name in ("x", "router_w", "w", "s", "alpha", "beta", "s_out"):
        assert _call(good, ptr={name: odd}) == B.MOE_ERR_ALIGN, name
    # T = 0 is a successful no-op even with NULL buffers
    zero = B.moe_dims_t(0, 256, 8, 512, 1e-6)
    assert _call(zero, null="x") == B.MOE_OK


def test_dequant_argument_errors():
    f = B.lib().moe_dequant_mxfp4
    p = C.c_void_p(1 << 20)
    assert f(None, p, 4, 64, p, None) == B.MOE_ERR_NULL
    assert f(p, p, 4, 48, p, None) == B.MOE_ERR_SHAPE
    assert f(p, p, -1, 64, p, None) == B.MOE_ERR_SHAPE
    assert f(p, p, 0, 64, p, None) == B.MOE_OK


def test_pack_argument_errors():
    f = B.lib().moe_pack_weights
    p = C.c_void_p(1 << 20)
    odd = C.c_void_p((1 << 20) + 4)
    good = B.moe_dims_t(0, 256, 8, 512, 1e-6)
    assert f(None, p, p, p, p, None) == B.MOE_ERR_NULL
    assert f(C.byref(good), None, p, p, p, None) == B.MOE_ERR_NULL
    assert f(C.byref(good), p, p, None, p, None) == B.MOE_ERR_NULL
    assert f(C.byref(B.moe_dims_t(0, 128, 8, 512, 1e-6)), p, p, p, p, None) == B.MOE_ERR_SHAPE
    assert f(C.byref(B.moe_dims_t(0, 256, 8, 64, 1e-6)), p, p, p, p, None) == B.MOE_ERR_SHAPE
    assert f(C.byref(B.moe_dims_t(0, 256, 0, 512, 1e-6)), p, p, p, p, None) == B.MOE_ERR_SHAPE
    assert f(C.byref(good), odd, p, p, p, None) == B.MOE_ERR_ALIGN
    assert f(C.byref(good), p, p, p, odd, None) == B.MOE_ERR_ALIGN


# ------------------------------------------------------------- latent variant

def test_latent_workspace_size():
    ws = B.moe_latent_workspace_size
    assert ws(0, 512, 256, 8, 256, 2) > 0
    a, b = ws(64, 512, 256, 8, 256, 2), ws(128, 512, 256, 8, 256, 2)
    assert 0 < a < b
    # at least the full-width layer's workspace at the experts' width, plus z and y
    # (the widened sum goes straight into the gate: no buffer for it)
    T = 4096
    big = ws(T, 8192, 4096, 256, 4096, 8)
    assert big >= B.moe_layer_workspace_size(T, 4096, 256, 4096, 8) + T * 4096 * 4
    assert ws(64, 500, 256, 8, 256, 2) == 0    # D not a multiple of 256
    assert ws(64, 512, 200, 8, 256, 2) == 0    # d not a multiple of 256
    assert ws(64, 512, 256, 8, 100, 2) == 0    # F not a multiple of 128
    assert ws(64, 512, 256, 8, 256, 9) == 0    # k > E


def _latent_call(dims, k=2, ws_bytes=1 << 30, null=None, ws_ptr=1 << 20, ptr=None):
    p = C.c_void_p(1 << 20)  # never dereferenced: every case below fails the checks first
    names = ("x", "router_w", "w_narrow", "w", "s", "w_widen", "alpha", "beta", "s_out")
    args = {n: p for n in names}
    args["ws"] = C.c_void_p(ws_ptr)
    if null:
        args[null] = None
    args.update(ptr or {})
    return B.lib().moe_latent_forward(C.byref(dims) if dims is not None else None,
                                      *(args[n] for n in names[:8]), k, args["s_out"], args["ws"],
                                      ws_bytes, None, None)


def test_latent_argument_errors():
    good = B.moe_latent_dims_t(64, 512, 256, 8, 256, 1e-6)
    assert _latent_call(None) == B.MOE_ERR_NULL
    for name in ("x", "router_w", "w_narrow", "w", "s", "w_widen", "alpha", "beta", "s_out", "ws"):
        assert _latent_call(good, null=name) == B.MOE_ERR_NULL, name
    assert _latent_call(B.moe_latent_dims_t(64, 500, 256, 8, 256, 1e-6)) == B.MOE_ERR_SHAPE
    assert _latent_call(B.moe_latent_dims_t(64, 512, 300, 8, 256, 1e-6)) == B.MOE_ERR_SHAPE
    assert _latent_call(good, k=9) == B.MOE_ERR_SHAPE
    assert _latent_call(good, ws_bytes=1024) == B.MOE_ERR_WORKSPACE
    assert _latent_call(good, ws_ptr=(1 << 20) + 64) == B.MOE_ERR_WORKSPACE
    odd = C.c_void_p((1 << 20) + 8)
    for name in ("x", "router_w", "w_narrow", "w", "s", "w_widen", "alpha", "beta", "s_out"):
        assert _latent_call(good, ptr={name: odd}) == B.MOE_ERR_ALIGN, name
    zero = B.moe_latent_dims_t(0, 512, 256, 8, 256, 1e-6)
    assert _latent_call(zero, null="x") == B.MOE_OK


# -------------------------------------------------------- block with stream norms

def test_block_workspace_size():
    ws = B.moe_block_workspace_size
    T = 4096
    assert ws(T, 8192, 256, 2048, 8) >= B.moe_layer_workspace_size(T, 8192, 256, 2048, 8) + \
        T * 8192 * 2 + T * 8192 * 4
    assert ws(64, 250, 8, 512, 2) == 0
    assert ws(64, 256, 8, 512, 9) == 0


def _block_call(dims, k=2, ws_bytes=1 << 30, null=None, ws_ptr=1 << 20, ptr=None):
    p = C.c_void_p(1 << 20)  # never dereferenced: every case below fails the checks first
    names = ("x", "gamma_pre", "router_w", "w", "s", "gamma_post", "alpha", "beta", "s_out")
    args = {n: p for n in names}
    args["ws"] = C.c_void_p(ws_ptr)
    if null:
        args[null] = None
    args.update(ptr or {})
    return B.lib().moe_block_forward(C.byref(dims) if dims is not None else None,
                                     *(args[n] for n in names[:8]), k, args["s_out"], args["ws"],
                                     ws_bytes, None, None)


def test_block_argument_errors():
    good = B.moe_dims_t(64, 256, 8, 512, 1e-6)
    assert _block_call(None) == B.MOE_ERR_NULL
    names = ("x", "gamma_pre", "router_w", "w", "s", "gamma_post", "alpha", "beta", "s_out")
    for name in names + ("ws",):
        assert _block_call(good, null=name) == B.MOE_ERR_NULL, name
    assert _block_call(B.moe_dims_t(64, 200, 8, 512, 1e-6)) == B.MOE_ERR_SHAPE
    assert _block_call(good, k=9) == B.MOE_ERR_SHAPE
    assert _block_call(good, ws_bytes=1024) == B.MOE_ERR_WORKSPACE
    odd = C.c_void_p((1 << 20) + 8)
    for name in names:
        assert _block_call(good, ptr={name: odd}) == B.MOE_ERR_ALIGN, name
    assert _block_call(B.moe_dims_t(0, 256, 8, 512, 1e-6), null="x") == B.MOE_OK


# ------------------------------------------------------------ 16-block format

def _nv_call(dims, k=2, ws_bytes=1 << 30, null=None, ws_ptr=1 << 20, ptr=None):
    p = C.c_void_p(1 << 20)  # never dereferenced: every case below fails the checks first
    names = ("x", "router_w", "w", "s16", "gscale", "alpha", "beta", "s_out")
    args = {n: p for n in names}
    args["ws"] = C.c_void_p(ws_ptr)
    if null:
        args[null] = None
    args.update(ptr or {})
    return B.lib().moe_layer_forward_nvfp4(C.byref(dims) if dims is not None else None,
                                           *(args[n] for n in names[:7]), k, args["s_out"], args["ws"],
                                           ws_bytes, None, None)


def test_nv_forward_argument_errors():
    good = B.moe_dims_t(64, 256, 8, 512, 1e-6)
    assert _nv_call(None) == B.MOE_ERR_NULL
    for name in ("x", "router_w", "w", "s16", "gscale", "alpha", "beta", "s_out", "ws"):
        assert _nv_call(good, null=name) == B.MOE_ERR_NULL, name
    assert _nv_call(B.moe_dims_t(64, 250, 8, 512, 1e-6)) == B.MOE_ERR_SHAPE
    assert _nv_call(B.moe_dims_t(64, 256, 8, 500, 1e-6)) == B.MOE_ERR_SHAPE
    assert _nv_call(good, k=9) == B.MOE_ERR_SHAPE
    assert _nv_call(good, ws_bytes=1024) == B.MOE_ERR_WORKSPACE
    assert _nv_call(good, ws_ptr=(1 << 20) + 64) == B.MOE_ERR_WORKSPACE
    odd = C.c_void_p((1 << 20) + 8)
    for name in ("x", "router_w", "w", "s16", "gscale", "alpha", "beta", "s_out"):
        assert _nv_call(good, ptr={name: odd}) == B.MOE_ERR_ALIGN, name
    assert _nv_call(B.moe_dims_t(0, 256, 8, 512, 1e-6), null="x") == B.MOE_OK


def test_nv_pack_argument_errors():
    p = C.c_void_p(1 << 20)
    pack = B.lib().moe_pack_weights_nvfp4
    assert pack(None, p, p, p, p, None) == B.MOE_ERR_NULL
    assert pack(C.byref(B.moe_dims_t(0, 250, 8, 512, 1e-6)), p, p, p, p, None) == B.MOE_ERR_SHAPE
    assert pack(C.byref(B.moe_dims_t(0, 256, 8, 500, 1e-6)), p, p, p, p, None) == B.MOE_ERR_SHAPE
    assert pack(C.byref(B.moe_dims_t(0, 256, 0, 512, 1e-6)), p, p, p, p, None) == B.MOE_ERR_SHAPE
    dims = C.byref(B.moe_dims_t(0, 256, 8, 512, 1e-6))
    assert pack(dims, None, p, p, p, None) == B.MOE_ERR_NULL
    assert pack(dims, p, None, p, p, None) == B.MOE_ERR_NULL
    assert pack(dims, p, p, p, C.c_void_p((1 << 20) + 4), None) == B.MOE_ERR_ALIGN


# ------------------------------------------------- the variant without a workspace

def test_noalloc_argument_errors():
    """Argument errors of moe_layer_forward_noalloc, all returned before any
    HIP call: NULL pointers, bad sizes, misaligned pointers, and sizes whose
    workspace would exceed the static scratch (MOE_ERR_SCRATCH)."""
    f = B.lib().moe_layer_forward_noalloc
    p = C.c_void_p(1 << 20)
    odd = C.c_void_p((1 << 20) + 8)
    good = B.moe_dims_t(64, 256, 8, 512, 1e-6)

    def call(dims, k=2, **repl):
        a = dict(x=p, router_w=p, w=p, s=p, alpha=p, beta=p, s_out=p)
        a.update(repl)
        return f(C.byref(dims) if dims is not None else None, a["x"], a["router_w"], a["w"], a["s"],
                 a["alpha"], a["beta"], k, a["s_out"], None, None)

    assert call(None) == B.MOE_ERR_NULL
    for name in ("x", "router_w", "w", "s", "alpha", "beta", "s_out"):
        assert call(good, **{name: None}) == B.MOE_ERR_NULL, name
        assert call(good, **{name: odd}) == B.MOE_ERR_ALIGN, name
    assert call(B.moe_dims_t(64, 200, 8, 512, 1e-6)) == B.MOE_ERR_SHAPE
    assert call(good, k=9) == B.MOE_ERR_SHAPE
    assert call(B.moe_dims_t(0, 256, 8, 512, 1e-6), x=None) == B.MOE_OK
    # the Muse shape fits up to T = 128; T = 130 needs more than 32 MiB
    assert B.moe_layer_workspace_size(128, 8192, 256, 2048, 8) <= B.MOE_STATIC_SCRATCH_BYTES
    assert B.moe_layer_workspace_size(130, 8192, 256, 2048, 8) > B.MOE_STATIC_SCRATCH_BYTES
    assert call(B.moe_dims_t(130, 8192, 256, 2048, 1e-6), k=8) == B.MOE_ERR_SCRATCH
    assert call(B.moe_dims_t(4096, 8192, 256, 2048, 1e-6), k=8) == B.MOE_ERR_SCRATCH
