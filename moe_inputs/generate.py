"""Seeded synthetic inputs for one MoE layer forward.

Every tensor has its own random stream,
``np.random.default_rng(SeedSequence([seed, cfg_id, tensor_id]))``, so any
single expert can be regenerated alone and the result does not depend on the
number of threads.  Stream ids: 0 = x, 1 = router weight, 2 = selection bias,
3 + 3*g + {0, 1, 2} = gate, up and down projection of expert g, where
g < E are the routed experts and g = E + s the shared ones.

Distributions (the workload descriptions of the five configs):

* x ~ N(0, 1); router and expert weights ~ N(0, 0.02) (0.02 is the
  ``initializer_range`` the Transformers Dots1 article lists among its config
  fields); drawn in fp32, then stored as fp32 or rounded to bf16.
* selection bias ~ U(-0.01, 0.01) in fp32, or, for the skewed workload, a
  Zipf(1.2) popularity profile: ``b_e = lambda * (ln p_e - mean ln p)`` with
  ``p_e ∝ (pi_e + 1) ** -1.2`` for a seeded permutation ``pi``.
* fp8 expert weights are stored as OCP e4m3 codes plus one fp32 scale per
  128x128 block.  The codes are drawn directly (a normal of std 64, clipped to
  +-448 and cast to e4m3 by torch); each block scale is 0.02 / 64 times a
  U(0.75, 1.25) factor, so the dequantised weights again have std about 0.02.
  Drawing codes directly keeps any quantisation rule out of this module.

The format conversions (fp32 -> bf16, fp32 -> e4m3) are torch's own casts.
This module holds no step of the layer's arithmetic: no routing, no matmul, no
quantisation of activations.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from .configs import MoEConfig

FP8_CODE_STD = 64.0
FP8_BLOCK = 128


def rng(seed: int, cfg_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cfg_id, tensor_id]))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), using torch's rounding cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    """fp32 array already inside [-448, 448] -> OCP e4m3 codes via torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _store(a32: np.ndarray, kind: str) -> np.ndarray:
    if kind == "f32":
        return a32.astype(np.float32, copy=False)
    if kind == "bf16":
        return to_bf16_bits(a32)
    raise ValueError(kind)


def _normal(g: np.random.Generator, shape, std: float) -> np.ndarray:
    a = g.standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(std)
    return a


def _fp8_weight(g: np.random.Generator, rows: int, cols: int, std: float):
    codes32 = g.standard_normal(size=(rows, cols), dtype=np.float32)
    codes32 *= np.float32(FP8_CODE_STD)
    np.clip(codes32, -448.0, 448.0, out=codes32)
    codes = to_e4m3_codes(codes32)
    fac = g.uniform(0.75, 1.25, size=(rows // FP8_BLOCK, cols // FP8_BLOCK))
    scales = (fac * (std / FP8_CODE_STD)).astype(np.float32)
    return codes, scales


def zipf_bias(cfg: MoEConfig, g: np.random.Generator) -> np.ndarray:
    pi = g.permutation(cfg.E)
    logp = -cfg.zipf_s * np.log(pi.astype(np.float64) + 1.0)
    logp -= np.log(np.exp(logp).sum())
    return (cfg.zipf_lambda * (logp - logp.mean())).astype(np.float32)


def weight_dtype(kind: str):
    return {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[kind]


def generate(cfg: MoEConfig, seed: int = 0, threads: int | None = None,
             weights: bool = True) -> dict:
    """Return every input of the layer as host numpy arrays in storage format.

    Keys: x [T,H], w_router [E,H] (act storage), bias [E] fp32,
    w_gate_up [E,2I,H], w_down [E,H,I], w_sh_gate_up [S,2Is,H], w_sh_down [S,H,Is]
    (expert storage); for fp8 also s_gate_up [E,2I/128,H/128], s_down [E,H/128,I/128],
    s_sh_gate_up, s_sh_down (fp32 block scales).  Gate rows come first in the
    packed gate_up tensor, up rows second.  bf16 arrays hold uint16 bit patterns;
    fp8 arrays hold uint8 e4m3 codes.  With weights=False only x, w_router and
    bias are drawn (the expert streams are independent, so this changes none
    of them).
    """
    T, H, E, S, I, Is = cfg.T, cfg.H, cfg.E, cfg.S, cfg.I, cfg.Is
    std = cfg.weight_std
    out: dict = {}

    out["x"] = _store(_normal(rng(seed, cfg.cfg_id, 0), (T, H), 1.0), cfg.act)
    out["w_router"] = _store(_normal(rng(seed, cfg.cfg_id, 1), (E, H), std), cfg.act)
    gb = rng(seed, cfg.cfg_id, 2)
    if cfg.bias_kind == "uniform":
        w = cfg.bias_half_width
        out["bias"] = gb.uniform(-w, w, size=E).astype(np.float32)
    elif cfg.bias_kind == "zipf":
        out["bias"] = zipf_bias(cfg, gb)
    else:
        raise ValueError(cfg.bias_kind)
    if not weights:
        return out

    wdt = weight_dtype(cfg.expert)
    gu = np.empty((E, 2 * I, H), dtype=wdt)
    dn = np.empty((E, H, I), dtype=wdt)
    sgu = np.empty((S, 2 * Is, H), dtype=wdt)
    sdn = np.empty((S, H, Is), dtype=wdt)
    fp8 = cfg.expert == "fp8"
    if fp8:
        B = FP8_BLOCK
        s_gu = np.empty((E, 2 * I // B, H // B), dtype=np.float32)
        s_dn = np.empty((E, H // B, I // B), dtype=np.float32)
        s_sgu = np.empty((S, 2 * Is // B, H // B), dtype=np.float32)
        s_sdn = np.empty((S, H // B, Is // B), dtype=np.float32)

    def fill(job):
        g_idx, part = job            # expert index g in [0, E+S), part 0/1/2
        shared = g_idx >= E
        e = g_idx - E if shared else g_idx
        inter = Is if shared else I
        g = rng(seed, cfg.cfg_id, 3 + 3 * g_idx + part)
        rows, cols = (inter, H) if part < 2 else (H, inter)
        if fp8:
            codes, sc = _fp8_weight(g, rows, cols, std)
        else:
            codes, sc = _store(_normal(g, (rows, cols), std), cfg.expert), None
        if part < 2:
            w = sgu if shared else gu
            w[e, part * inter:(part + 1) * inter] = codes
            if fp8:
                s = s_sgu if shared else s_gu
                nb = inter // FP8_BLOCK
                s[e, part * nb:(part + 1) * nb] = sc
        else:
            (sdn if shared else dn)[e] = codes
            if fp8:
                (s_sdn if shared else s_dn)[e] = sc

    jobs = [(g, p) for g in range(E + S) for p in range(3)]
    with ThreadPoolExecutor(max_workers=threads or _threads()) as ex:
        list(ex.map(fill, jobs))

    out.update(w_gate_up=gu, w_down=dn, w_sh_gate_up=sgu, w_sh_down=sdn)
    if fp8:
        out.update(s_gate_up=s_gu, s_down=s_dn, s_sh_gate_up=s_sgu, s_sh_down=s_sdn)
    return out
