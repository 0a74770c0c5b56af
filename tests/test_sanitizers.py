"""The oracle and the C ABI's argument checking under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU (host code only; no call reaches a
GPU).  The oracle's sanitized build must give bit-for-bit the regular
build's results; the library's sanitized host build must return every
argument error without a report."""
import concurrent.futures as cf
import os
import subprocess

import numpy as np
import pytest

import oracle
from mixture_experts_gemm_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# leaks of the HIP and OpenMP runtimes at exit are not this code's
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="-1",
           ROCR_VISIBLE_DEVICES="-1", OMP_NUM_THREADS="4")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (cmd, r.stdout[-3000:], r.stderr[-3000:])
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
    return r


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_run")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off",
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_run.c"), "-lm", "-o", exe])
    L = synth.make_layer("tiny")
    N = synth.make_layer_nv("tiny")
    g_pre, g_post = synth.make_norm_gains(synth.WORKLOADS["tiny"])
    s = L.shape
    files = dict(x=L.x, wr=L.router_w, w=L.w_packed, sc=L.scales, sc16=N.scales16, gs=N.gscale,
                 alpha=L.alpha, beta=L.beta, gpre=g_pre, gpost=g_post)
    for name, arr in files.items():
        np.ascontiguousarray(arr).tofile(str(tmp_path / name))
    _run([exe, str(tmp_path), str(s.T), str(s.d), str(s.E), str(s.F), str(s.k)], env=ENV)
    got = lambda n, dt: np.fromfile(str(tmp_path / n), dtype=dt)
    ref, ids, _ = oracle.moe_forward(L.x, L.router_w, L.w_packed, L.scales, L.alpha, L.beta, s.k)
    np.testing.assert_array_equal(got("out_layer", np.float64).reshape(ref.shape), ref)
    r = oracle.route(L.x, L.router_w, s.k)
    np.testing.assert_array_equal(got("out_perm", np.int32), r["perm"])
    blk, _, _ = oracle.block_forward(L.x, g_pre, L.router_w, L.w_packed, L.scales, g_post, L.alpha,
                                     L.beta, s.k)
    np.testing.assert_array_equal(got("out_block", np.float64).reshape(blk.shape), blk)
    nv, _, _ = oracle.moe_forward_nv(L.x, L.router_w, L.w_packed, N.scales16, N.gscale, L.alpha,
                                     L.beta, s.k)
    np.testing.assert_array_equal(got("out_nv", np.float64).reshape(nv.shape), nv)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_argument_checks_under_sanitizers(tmp_path):
    # the device code is built as usual; each -fsanitize applies to the host pass only
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include")] + san
    srcs = ["api", "route", "expert", "combine", "weights", "latent"]
    csrc = os.path.join(ROOT, "mixture_experts_gemm_amd", "csrc")

    def compile_one(name):
        _run([HIPCC, *flags, "-c", os.path.join(csrc, name + ".hip"), "-o", str(tmp_path / (name + ".o"))])

    with cf.ThreadPoolExecutor(len(srcs)) as ex:
        list(ex.map(compile_one, srcs))
    lib = str(tmp_path / "libmoe_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", *[str(tmp_path / (n + ".o")) for n in srcs], "-o", lib])
    exe = str(tmp_path / "abi_args")
    _run([HIPCC, "-O1", "-g", "-std=c++17", "-x", "c++",
          "-I", os.path.join(ROOT, "include"), *san, os.path.join(HERE, "abi_args.cpp"),
          "-L" + str(tmp_path), "-lmoe_san", "-Wl,-rpath," + str(tmp_path), "-o", exe])
    r = _run([exe], env=ENV)
    assert "0 failure(s)" in r.stdout, r.stdout
