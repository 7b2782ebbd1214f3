"""ctypes binding of libmoe.so: the C ABI of include/moe.h, same names.

Argument marshalling only.  Tensors are torch device tensors (their
``data_ptr()`` is passed through); every step of the layer runs in the HIP
kernels of libmoe.  There is no fallback: if the library is missing this
module raises on import.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_LIB", os.path.join(_PKG, "libmoe.so"))

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3}
MOE_LAYOUT_ROWS, MOE_LAYOUT_TILED = 0, 1
# moe_ws_part_t
(MOE_WS_TOPK_IDX, MOE_WS_TOPK_W, MOE_WS_COUNTS, MOE_WS_OFFSETS, MOE_WS_PERM, MOE_WS_INV,
 MOE_WS_H, MOE_WS_H_SCALES, MOE_WS_H_LO, MOE_WS_Y, MOE_WS_Y_SHARED, MOE_WS_H_EXP,
 MOE_WS_BARRIER, MOE_WS_Y_EXP) = range(14)
WS_NONE = (1 << 64) - 1

# every entry point of include/moe.h
EXPORTS = ("moe_status_string", "moe_last_error_detail", "moe_version", "moe_workspace_size",
           "moe_workspace_offset", "moe_route",
           "moe_dispatch", "moe_grouped_ffn", "moe_expert_gate_up", "moe_expert_down",
           "moe_combine", "moe_quantize_fp8", "moe_layer_forward", "moe_layer_forward_timed",
           "moe_rmsnorm", "moe_block_forward", "moe_layer_forward_fused",
           "moe_pack_expert_weights", "moe_layer_forward_noalloc", "moe_stream_read",
           "moe_fused_set_spin_limit", "moe_convert_bf16_to_f16")


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = LIB.moe_last_error_detail().decode() if status == MOE_ERR_HIP else ""
        super().__init__(f"{where}: {status_string(status)} (status {status})"
                         + (f" [{detail}]" if detail else ""))


class moe_config_t(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("S", ctypes.c_int32), ("k", ctypes.c_int32), ("I", ctypes.c_int32),
                ("I_shared", ctypes.c_int32), ("norm_topk_prob", ctypes.c_int32),
                ("routed_scaling_factor", ctypes.c_float), ("act_dtype", ctypes.c_int32),
                ("expert_dtype", ctypes.c_int32), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("expert_layout", ctypes.c_int32)]


class moe_weights_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_router", "router_bias", "w_gate_up", "w_down", "s_gate_up", "s_down",
        "w_sh_gate_up", "w_sh_down", "s_sh_gate_up", "s_sh_down", "w_down_f16", "w_sh_down_f16")]


def _load():
    # torch ships its own HIP runtime.  Load it first, so that libmoe's
    # dependency on libamdhip64.so.7 binds to that same runtime instead of
    # bringing a second one into the process (two runtimes cannot share
    # device pointers, streams or the device itself).
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libmoe.so not found at {LIB_PATH}; build it with "
                          "`python -m sparse_moe_expert_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32P, SZ = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t
    CP = ctypes.POINTER(moe_config_t)
    WP = ctypes.POINTER(moe_weights_t)
    sig = {
        "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_version": (ctypes.c_char_p, []),
        "moe_last_error_detail": (ctypes.c_char_p, []),
        "moe_workspace_size": (SZ, [CP]),
        "moe_workspace_offset": (SZ, [CP, ctypes.c_int32]),
        "moe_route": (ctypes.c_int, [CP, P, WP, I32P, P, I32P, P, SZ, P]),
        "moe_dispatch": (ctypes.c_int, [CP, I32P, I32P, I32P, I32P, I32P, P, SZ, P]),
        "moe_grouped_ffn": (ctypes.c_int, [CP, P, WP, I32P, I32P, P, P, P, SZ, P]),
        "moe_expert_gate_up": (ctypes.c_int, [CP, P, WP, I32P, I32P, P, SZ, P]),
        "moe_expert_down": (ctypes.c_int, [CP, WP, P, P, P, SZ, P]),
        "moe_combine": (ctypes.c_int, [CP, P, P, P, I32P, P, P]),
        "moe_quantize_fp8": (ctypes.c_int, [P, ctypes.c_int32, ctypes.c_int32, P, P, P]),
        "moe_pack_expert_weights": (ctypes.c_int, [P, P, ctypes.c_int64, ctypes.c_int32,
                                                   ctypes.c_int32, ctypes.c_int32, P]),
        "moe_convert_bf16_to_f16": (ctypes.c_int, [P, P, ctypes.c_int64, P]),
        "moe_layer_forward": (ctypes.c_int, [CP, WP, P, P, I32P, I32P, P, SZ, P]),
        "moe_layer_forward_timed": (ctypes.c_int, [CP, WP, P, P, I32P, I32P, P, SZ, P,
                                                   ctypes.POINTER(ctypes.c_void_p)]),
        "moe_layer_forward_fused": (ctypes.c_int, [CP, WP, P, P, I32P, I32P, P, SZ, P]),
        "moe_layer_forward_noalloc": (ctypes.c_int, [CP, WP, P, P, I32P, I32P, P]),
        "moe_stream_read": (ctypes.c_int, [P, SZ, P, ctypes.c_int32, P]),
        "moe_fused_set_spin_limit": (ctypes.c_int64, [ctypes.c_int64]),
        "moe_rmsnorm": (ctypes.c_int, [CP, P, P, ctypes.c_float, P, P]),
        "moe_block_forward": (ctypes.c_int, [CP, WP, P, P, ctypes.c_float, P, I32P, I32P, P, SZ,
                                             P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


LIB = _load()


def status_string(status: int) -> str:
    return LIB.moe_status_string(status).decode()


def last_error_detail() -> str:
    return LIB.moe_last_error_detail().decode()


def version() -> str:
    return LIB.moe_version().decode()


def make_config(T, H, E, S, k, I, I_shared=None, act="bf16", expert="bf16",
                norm_topk_prob=True, routed_scaling_factor=1.0, n_group=1,
                topk_group=1, tiled=False) -> moe_config_t:
    return moe_config_t(T, H, E, S, k, I, I if I_shared is None else I_shared,
                        1 if norm_topk_prob else 0, float(routed_scaling_factor),
                        DTYPES[act], DTYPES[expert], int(n_group), int(topk_group),
                        MOE_LAYOUT_TILED if tiled else MOE_LAYOUT_ROWS)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_weights(w_router=None, router_bias=None, w_gate_up=None, w_down=None, s_gate_up=None,
                 s_down=None, w_sh_gate_up=None, w_sh_down=None, s_sh_gate_up=None,
                 s_sh_down=None, w_down_f16=None, w_sh_down_f16=None) -> moe_weights_t:
    return moe_weights_t(*(_ptr(t) for t in (w_router, router_bias, w_gate_up, w_down, s_gate_up,
                                             s_down, w_sh_gate_up, w_sh_down, s_sh_gate_up,
                                             s_sh_down, w_down_f16, w_sh_down_f16)))


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoEError(status, where)


def moe_workspace_size(cfg: moe_config_t) -> int:
    return int(LIB.moe_workspace_size(ctypes.byref(cfg)))


def moe_workspace_offset(cfg: moe_config_t, part: int) -> int | None:
    """Byte offset of an intermediate in the layer workspace, or None."""
    off = int(LIB.moe_workspace_offset(ctypes.byref(cfg), int(part)))
    return None if off == WS_NONE else off


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def moe_route(cfg, x, weights, topk_idx, topk_w, tie_counts=None, workspace=None, stream=None):
    wp, wb = _ws(workspace)
    _check(LIB.moe_route(ctypes.byref(cfg), _ptr(x), ctypes.byref(weights), _ptr(topk_idx),
                         _ptr(topk_w), _ptr(tie_counts), wp, wb, _stream(stream)), "moe_route")


def moe_dispatch(cfg, topk_idx, counts, offsets, perm, inv, workspace=None, stream=None):
    wp, wb = _ws(workspace)
    _check(LIB.moe_dispatch(ctypes.byref(cfg), _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                            _ptr(perm), _ptr(inv), wp, wb, _stream(stream)), "moe_dispatch")


def moe_grouped_ffn(cfg, x, weights, perm, offsets, y_sorted, y_shared, workspace=None,
                    stream=None):
    wp, wb = _ws(workspace)
    _check(LIB.moe_grouped_ffn(ctypes.byref(cfg), _ptr(x), ctypes.byref(weights), _ptr(perm),
                               _ptr(offsets), _ptr(y_sorted), _ptr(y_shared), wp, wb,
                               _stream(stream)), "moe_grouped_ffn")


def moe_expert_gate_up(cfg, x, weights, perm, offsets, workspace=None, stream=None):
    wp, wb = _ws(workspace)
    _check(LIB.moe_expert_gate_up(ctypes.byref(cfg), _ptr(x), ctypes.byref(weights), _ptr(perm),
                                  _ptr(offsets), wp, wb, _stream(stream)), "moe_expert_gate_up")


def moe_expert_down(cfg, weights, y_sorted, y_shared, workspace=None, stream=None):
    wp, wb = _ws(workspace)
    _check(LIB.moe_expert_down(ctypes.byref(cfg), ctypes.byref(weights), _ptr(y_sorted),
                               _ptr(y_shared), wp, wb, _stream(stream)), "moe_expert_down")


def moe_combine(cfg, y_sorted, y_shared, topk_w, inv, out, stream=None):
    _check(LIB.moe_combine(ctypes.byref(cfg), _ptr(y_sorted), _ptr(y_shared), _ptr(topk_w),
                           _ptr(inv), _ptr(out), _stream(stream)), "moe_combine")


def moe_quantize_fp8(x, rows, cols, q, scales, stream=None):
    _check(LIB.moe_quantize_fp8(_ptr(x), rows, cols, _ptr(q), _ptr(scales), _stream(stream)),
           "moe_quantize_fp8")


def moe_pack_expert_weights(src, dst, count, rows, cols, dtype, stream=None):
    """dtype: "f32" | "bf16" | "fp8" (or a moe_dtype_t value)."""
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    _check(LIB.moe_pack_expert_weights(_ptr(src), _ptr(dst), int(count), int(rows), int(cols), dt,
                                       _stream(stream)), "moe_pack_expert_weights")


def moe_convert_bf16_to_f16(src, dst, n, stream=None):
    """n bf16 values of src -> fp16 in dst, rounded toward zero (the fp16
    copy of bf16 down weights, moe_weights_t w_down_f16 / w_sh_down_f16)."""
    _check(LIB.moe_convert_bf16_to_f16(_ptr(src), _ptr(dst), int(n), _stream(stream)),
           "moe_convert_bf16_to_f16")


def moe_layer_forward(cfg, weights, x, out, opt_counts=None, opt_tie_counts=None, workspace=None,
                      stream=None):
    wp, wb = _ws(workspace)
    _check(LIB.moe_layer_forward(ctypes.byref(cfg), ctypes.byref(weights), _ptr(x), _ptr(out),
                                 _ptr(opt_counts), _ptr(opt_tie_counts), wp, wb, _stream(stream)),
           "moe_layer_forward")


def moe_layer_forward_timed(cfg, weights, x, out, events, opt_counts=None, opt_tie_counts=None,
                            workspace=None, stream=None):
    """events: 7 torch.cuda.Event(enable_timing=True) objects (or raw hipEvent_t ints)."""
    if len(events) != 7:
        raise ValueError("moe_layer_forward_timed needs 7 events")
    arr = (ctypes.c_void_p * 7)(*[e if isinstance(e, int) else e.cuda_event for e in events])
    wp, wb = _ws(workspace)
    _check(LIB.moe_layer_forward_timed(ctypes.byref(cfg), ctypes.byref(weights), _ptr(x),
                                       _ptr(out), _ptr(opt_counts), _ptr(opt_tie_counts), wp, wb,
                                       _stream(stream), arr), "moe_layer_forward_timed")


def moe_layer_forward_fused(cfg, weights, x, out, opt_counts=None, opt_tie_counts=None,
                            workspace=None, stream=None):
    wp, wb = _ws(workspace)
    _check(LIB.moe_layer_forward_fused(ctypes.byref(cfg), ctypes.byref(weights), _ptr(x),
                                       _ptr(out), _ptr(opt_counts), _ptr(opt_tie_counts), wp, wb,
                                       _stream(stream)), "moe_layer_forward_fused")


def moe_layer_forward_noalloc(cfg, weights, x, out, opt_counts=None, opt_tie_counts=None,
                              stream=None):
    _check(LIB.moe_layer_forward_noalloc(ctypes.byref(cfg), ctypes.byref(weights), _ptr(x),
                                         _ptr(out), _ptr(opt_counts), _ptr(opt_tie_counts),
                                         _stream(stream)), "moe_layer_forward_noalloc")


NOALLOC_SCRATCH_BYTES = 96 << 20


def moe_fused_set_spin_limit(polls):
    """Bound of each grid-barrier wait of moe_layer_forward_fused (0: give up
    at once; polls < 0: the default); returns the previous bound."""
    return int(LIB.moe_fused_set_spin_limit(int(polls)))


def moe_stream_read(src, nbytes, sink, blocks, stream=None):
    """Measurement utility: one streaming read pass over nbytes of src."""
    _check(LIB.moe_stream_read(_ptr(src), int(nbytes), _ptr(sink), int(blocks), _stream(stream)),
           "moe_stream_read")


def moe_rmsnorm(cfg, h, gamma, eps, out, stream=None):
    _check(LIB.moe_rmsnorm(ctypes.byref(cfg), _ptr(h), _ptr(gamma), float(eps), _ptr(out),
                           _stream(stream)), "moe_rmsnorm")


def moe_block_forward(cfg, weights, h, gamma, eps, out, opt_counts=None, opt_tie_counts=None,
                      workspace=None, stream=None):
    wp, wb = _ws(workspace)
    _check(LIB.moe_block_forward(ctypes.byref(cfg), ctypes.byref(weights), _ptr(h), _ptr(gamma),
                                 float(eps), _ptr(out), _ptr(opt_counts), _ptr(opt_tie_counts),
                                 wp, wb, _stream(stream)), "moe_block_forward")
