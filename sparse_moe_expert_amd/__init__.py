"""MI355X (gfx950) MoE layer forward: sigmoid/noaux_tc router (optionally
group-limited), stable dispatch, grouped SwiGLU expert GEMMs (bf16 / fp8 e4m3
MFMA), shared expert and deterministic combine, plus the decoder block around
it (RMSNorm before, residual after), as hand-written HIP kernels behind the C
ABI of include/moe.h (libmoe.so).

This package is the ctypes binding (``_lib``) plus device-buffer plumbing
(``device``).  The binding loads on first use of any of its names and raises
ImportError if libmoe.so has not been built; there is no other code path.
``python -m sparse_moe_expert_amd.build`` builds the library.
"""
import importlib

_BINDING = (
    "DTYPES", "EXPORTS", "LIB", "LIB_PATH", "MOE_BF16", "MOE_ERR_HIP", "MOE_ERR_INVALID_ARG",
    "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE", "MOE_F32", "MOE_FP8_E4M3", "MOE_OK", "MoEError",
    "make_config", "make_weights", "moe_combine", "moe_config_t", "moe_dispatch",
    "moe_expert_down", "moe_expert_gate_up", "moe_grouped_ffn", "moe_layer_forward",
    "moe_layer_forward_timed", "moe_rmsnorm", "moe_block_forward", "moe_layer_forward_fused",
    "moe_quantize_fp8", "moe_route", "moe_weights_t", "moe_workspace_size", "status_string",
    "version", "last_error_detail", "moe_pack_expert_weights", "MOE_LAYOUT_ROWS",
    "MOE_LAYOUT_TILED", "moe_workspace_offset", "MOE_WS_TOPK_IDX", "MOE_WS_TOPK_W",
    "MOE_WS_COUNTS", "MOE_WS_OFFSETS", "MOE_WS_PERM", "MOE_WS_INV", "MOE_WS_H",
    "MOE_WS_H_SCALES", "MOE_WS_H_LO", "MOE_WS_Y", "MOE_WS_Y_SHARED", "MOE_WS_H_EXP", "MOE_WS_BARRIER", "MOE_WS_Y_EXP",
    "moe_layer_forward_noalloc", "NOALLOC_SCRATCH_BYTES", "moe_stream_read", "moe_fused_set_spin_limit",
    "moe_convert_bf16_to_f16",
)

__all__ = list(_BINDING)


def __getattr__(name):
    if name in _BINDING:
        return getattr(importlib.import_module("._lib", __name__), name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
