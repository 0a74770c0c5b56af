"""MI355X-native MoE expert layer: router top-k, grouping by expert, grouped
MXFP4 SwiGLU experts on MFMA, per-expert RMSNorm and the gated residual.

The compute path is the HIP library libmoe.so (C ABI declared in
include/moe.h); `mixture_experts_gemm_amd.binding` marshals arguments to it.
"""
__all__ = ["binding", "synth", "roofline"]
