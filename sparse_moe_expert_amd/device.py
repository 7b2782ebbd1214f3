"""Device buffers for one MoE layer: upload storage-format host arrays into
torch device tensors, build the C structs, and call the C ABI.

Plumbing only: torch provides device memory and the stream; every step of
the layer runs in libmoe's HIP kernels.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib
from ._lib import make_config, make_weights

_TORCH_STORAGE = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_device(a: np.ndarray, kind: str, device="cuda") -> torch.Tensor:
    """Storage array (fp32, bf16 bit patterns as uint16, e4m3 codes as uint8,
    int32) -> device tensor of the matching torch dtype (bits unchanged)."""
    a = np.ascontiguousarray(a)
    if kind == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    elif kind == "fp8":
        t = torch.from_numpy(a.view(np.uint8))
    elif kind in ("f32", "i32"):
        t = torch.from_numpy(a)
    else:
        raise ValueError(kind)
    return t.to(device, non_blocking=False)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host numpy array of its raw storage (bf16 -> uint16)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def pack_expert_weights(w: torch.Tensor, kind: str, stream=None) -> torch.Tensor:
    """[n, rows, cols] row-major device tensor -> a new tensor of the same
    shape and dtype holding the MOE_LAYOUT_TILED byte order (the library's
    moe_pack_expert_weights; the shape no longer indexes the elements)."""
    w = w.contiguous()
    out = torch.empty_like(w)
    n, rows, cols = w.shape
    _lib.moe_pack_expert_weights(w, out, n, rows, cols, kind, stream)
    return out


class DeviceLayer:
    """All inputs of one layer resident in device memory, plus a workspace.

    tiled=True stores the expert weights in MOE_LAYOUT_TILED order: they are
    uploaded row-major, packed on the device once, and the row-major copies
    are dropped.  down_f16=True (bf16 experts) also keeps the fp16 copies of
    the down weights (moe_convert_bf16_to_f16) that the large-tile down GEMM
    reads instead of converting bf16 fragments itself."""

    def __init__(self, cfg, inp: dict, device: str = "cuda", tiled: bool = False,
                 down_f16: bool = False):
        self.cfg = cfg
        self.device = device
        self.tiled = tiled
        self.ccfg = make_config(cfg.T, cfg.H, cfg.E, cfg.S, cfg.k, cfg.I, cfg.Is, act=cfg.act,
                                expert=cfg.expert, norm_topk_prob=cfg.norm_topk_prob,
                                routed_scaling_factor=cfg.routed_scaling_factor,
                                n_group=cfg.n_group, topk_group=cfg.topk_group, tiled=tiled)
        ek = cfg.expert
        t = {
            "x": to_device(inp["x"], cfg.act, device),
            "w_router": to_device(inp["w_router"], cfg.act, device),
            "bias": to_device(inp["bias"], "f32", device),
            "w_gate_up": to_device(inp["w_gate_up"], ek, device),
            "w_down": to_device(inp["w_down"], ek, device),
            "w_sh_gate_up": to_device(inp["w_sh_gate_up"], ek, device),
            "w_sh_down": to_device(inp["w_sh_down"], ek, device),
        }
        if ek == "fp8":
            for key in ("s_gate_up", "s_down", "s_sh_gate_up", "s_sh_down"):
                t[key] = to_device(inp[key], "f32", device)
        if tiled:
            for key in ("w_gate_up", "w_down", "w_sh_gate_up", "w_sh_down"):
                t[key] = pack_expert_weights(t[key], ek)
        if down_f16:
            for key in ("w_down", "w_sh_down"):
                if t[key].numel():
                    t[key + "_f16"] = torch.empty(t[key].shape, dtype=torch.float16, device=device)
                    _lib.moe_convert_bf16_to_f16(t[key], t[key + "_f16"], t[key].numel())
        self.t = t
        self.weights = make_weights(
            w_router=t["w_router"], router_bias=t["bias"], w_gate_up=t["w_gate_up"],
            w_down=t["w_down"], s_gate_up=t.get("s_gate_up"), s_down=t.get("s_down"),
            w_sh_gate_up=t["w_sh_gate_up"], w_sh_down=t["w_sh_down"],
            s_sh_gate_up=t.get("s_sh_gate_up"), s_sh_down=t.get("s_sh_down"),
            w_down_f16=t.get("w_down_f16"), w_sh_down_f16=t.get("w_sh_down_f16"))
        self.ws_bytes = _lib.moe_workspace_size(self.ccfg)
        self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        self.act_dtype = _TORCH_STORAGE[cfg.act]

    def empty_out(self) -> torch.Tensor:
        return torch.empty((self.cfg.T, self.cfg.H), dtype=self.act_dtype, device=self.device)

    def forward(self, out=None, counts=None, ties=None, stream=None) -> torch.Tensor:
        out = self.empty_out() if out is None else out
        _lib.moe_layer_forward(self.ccfg, self.weights, self.t["x"], out, counts, ties,
                               self.workspace, stream)
        return out
