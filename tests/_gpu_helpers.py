"""Shared pieces of the GPU parity tests (imported by test files only)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}   # max|Δ| / rms(oracle out)
TIE = 1e-6


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def tol_for(cfg) -> float:
    return TOL["fp8"] if cfg.expert == "fp8" else TOL[cfg.act]


def bf16_round(a: np.ndarray) -> np.ndarray:
    """fp64/fp32 values -> bf16 bit patterns via torch's cast (test-side input prep)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def untied(r) -> np.ndarray:
    ok = (r.gap_sel > TIE) & (r.gap_ord > TIE)
    if r.gap_grp is not None:
        ok &= r.gap_grp > TIE
    return ok


def check_routing(cfg, r, idx_gpu: np.ndarray, w_gpu: np.ndarray, where: str):
    """Indices bit-exact on every token without a near-tie; weights within
    1e-6; tied tokens must still hold a valid top-k (every chosen key within
    1e-6 of the oracle's k-th key, all distinct)."""
    ok = untied(r)
    bad = np.nonzero(ok & np.any(idx_gpu != r.idx, axis=1))[0]
    assert bad.size == 0, f"{where}: idx differs on untied tokens {bad[:10]}"
    dw = np.abs(w_gpu[ok] - r.w[ok])
    assert dw.size == 0 or dw.max() <= 1e-6, f"{where}: max |dw| {dw.max():.3e}"
    kth = np.sort(r.keys, axis=1)[:, ::-1][:, cfg.k - 1]
    grouped = getattr(cfg, "n_group", 1) > 1
    for t in np.nonzero(~ok)[0]:
        row = idx_gpu[t]
        assert len(set(row.tolist())) == cfg.k and row.min() >= 0 and row.max() < cfg.E
        if not grouped:     # with groups, a group near-tie changes the allowed set
            assert np.all(r.keys[t, row] >= kth[t] - TIE), f"{where}: token {t} invalid top-k"
    return int((~ok).sum())


def assert_close(cfg, got: np.ndarray, ref: np.ndarray, where: str, mask=None):
    if mask is not None:
        got, ref = got[mask], ref[mask]
    scale = oracle.rms(ref)
    err = np.abs(got - ref).max() if got.size else 0.0
    tol = tol_for(cfg)
    log(f"{where}: max|Δ|/rms = {err / scale:.3e} (tol {tol:.0e})")
    assert np.all(np.isfinite(got)), f"{where}: non-finite output"
    assert err <= tol * scale, f"{where}: max|Δ| {err:.4e} > {tol} * rms {scale:.4e}"
