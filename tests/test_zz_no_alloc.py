"""moe_layer_forward_noalloc (the library's static device scratch, no
workspace argument, no allocation in the call) against moe_layer_forward on
the same inputs: bit-for-bit equal outputs and routing, on two calls in a
row, the second with a smaller input (the scratch keeps the first call's
contents)."""
import numpy as np
import pytest
import torch

from mixture_experts_gemm_amd import binding as B
from mixture_experts_gemm_amd import synth

from helpers import bf16_bits, debug_buffers, upload

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-case]", *a, flush=True)


def _both(L, dev, T):
    """(workspace entry point, no-allocation entry point) outputs and routing on the first T tokens."""
    s = L.shape
    x = dev["x"][:T]
    args = (dev["router_w"], dev["w"], dev["s"], dev["alpha"], dev["beta"], s.k)
    d1, d2 = debug_buffers(T, s.E, s.k), debug_buffers(T, s.E, s.k)
    ref = B.moe_layer_forward(x, *args, F=s.F, eps=L.eps, debug=d1)
    out = torch.empty_like(x)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    alloc0 = torch.cuda.memory_allocated()
    got = B.moe_layer_forward_noalloc(x, *args, F=s.F, eps=L.eps, s_out=out, debug=d2)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    alloc1 = torch.cuda.memory_allocated()
    routing_same = all(torch.equal(d1[n], d2[n]) for n in d1)
    return bf16_bits(ref), bf16_bits(got), routing_same, (free0 - free1, alloc1 - alloc0)


# (workload, first T, second T): tiled MX kernels then the 16-row ones;
# the streaming decode kernel at the Muse shape; the largest Muse-shaped T
# the scratch holds, then decode
CASES = [("tiny", 64, 37), ("decode4", 8, 4), ("decode4", 128, 1)]


@pytest.mark.parametrize("name,T1,T2", CASES)
def test_noalloc_matches_workspace_entry_point(name, T1, T2):
    L = synth.make_layer(name, T=T1, threads=16)
    dev = upload(L)
    # the first call on this GPU may load the library's device code (and with
    # it the static scratch); the calls below are measured after it
    B.moe_layer_forward_noalloc(dev["x"][:1], dev["router_w"], dev["w"], dev["s"], dev["alpha"],
                                dev["beta"], L.k, F=L.shape.F, eps=L.eps)
    torch.cuda.synchronize()
    for T in (T1, T2):
        _say("noalloc", name, "T", T)
        ref, got, routing_same, (dfree, dalloc) = _both(L, dev, T)
        assert routing_same, (name, T)
        assert np.array_equal(ref, got), (name, T, int((ref != got).sum()))
        assert dfree == 0 and dalloc == 0, (name, T, dfree, dalloc)
