"""Routed mixture-of-experts layer on checkpoint-format quantized weights for
AMD MI355X (gfx950).

The compute lives in ``libmoe.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/moe.h``); this package only loads it, marshals arguments
and keeps weights resident through torch.  The C entry points are re-exported
here on first use; without the built library that first use raises
ImportError: there is no fallback path.  ``python -m
quantized_moe_expert_02_amd.build`` builds the library in-tree.
"""
import importlib

_EXPORTS = ("MOE_ACT_EXACT", "MOE_ACT_FP8_T128", "MOE_ACT_MXFP4", "MOE_ACT_MXFP8",
            "moe_expert_gemm_q", "moe_layer_forward_ex", "moe_quantize_act", "moe_route_table",
            "moe_layer_forward_routed", "moe_layer_forward_noalloc", "moe_noalloc_workspace_limit",
            "moe_decode_gate_up",
            "MOE_ERR_HIP", "MOE_ERR_INVALID_ARG", "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE",
            "MOE_FMT_FP8_B128", "MOE_FMT_MXFP4", "MOE_FMT_MXFP8", "MOE_FMT_NVFP4", "MOE_OK", "MOE_OP_DOWN",
            "MOE_OP_GATE_UP_SWIGLU", "LIB_PATH", "MoeError", "moe_abi_version", "moe_combine",
            "moe_expert_gemm", "moe_layer_desc", "moe_layer_forward", "moe_permute",
            "moe_permute_workspace_size", "moe_qweight", "moe_route_topk", "moe_validate_layer",
            "moe_workspace_size", "status_string")


def __getattr__(name):
    if name in _EXPORTS:
        return getattr(importlib.import_module("._lib", __name__), name)
    raise AttributeError(name)
