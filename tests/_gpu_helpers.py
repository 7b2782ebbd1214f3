"""Shared pieces of the GPU parity tests (imported by test files only)."""
from __future__ import annotations

import itertools
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


def _valid_topk(keys: np.ndarray, row: np.ndarray, allowed: np.ndarray) -> bool:
    """row is a top-k of `keys` restricted to `allowed` (bool [E]) up to
    1e-6 near-ties: every chosen expert allowed, no unchosen allowed key above
    the smallest chosen key by more than 1e-6, and slot order non-increasing
    within 1e-6."""
    if not np.all(allowed[row]):
        return False
    rest = allowed.copy()
    rest[row] = False
    if rest.any() and keys[rest].max() > keys[row].min() + TIE:
        return False
    return bool(np.all(keys[row][:-1] >= keys[row][1:] - TIE))


def _valid_grouped(cfg, keys: np.ndarray, row: np.ndarray) -> bool:
    """Group-limited routing: some choice of topk_group groups that is valid
    up to 1e-6 near-ties of the group scores admits `row` as its top-k."""
    ng, tg = cfg.n_group, cfg.topk_group
    G = cfg.E // ng
    gs = oracle.group_scores(keys[None, :], ng)[0]
    b = np.sort(gs)[::-1][tg - 1]
    sure = [g for g in range(ng) if gs[g] > b + TIE]
    near = [g for g in range(ng) if abs(gs[g] - b) <= TIE]
    for extra in itertools.combinations(near, tg - len(sure)):
        chosen = set(sure) | set(extra)
        allowed = np.repeat(np.isin(np.arange(ng), list(chosen)), G)
        if _valid_topk(keys, row, allowed):
            return True
    return False


def check_routing(cfg, r, idx_gpu: np.ndarray, w_gpu: np.ndarray, where: str):
    """Indices bit-exact on every token without a near-tie.  On every token,
    the weights equal (within 1e-6) the oracle's renormalised unbiased scores
    of the set the GPU chose.  A near-tied token must hold a valid top-k: k
    distinct experts in range, no unchosen key more than 1e-6 above a chosen
    one, slots in non-increasing key order within 1e-6 (with groups: inside
    some valid choice of groups).  Returns the number of near-tied tokens."""
    ok = untied(r)
    bad = np.nonzero(ok & np.any(idx_gpu != r.idx, axis=1))[0]
    assert bad.size == 0, f"{where}: idx differs on untied tokens {bad[:10]}"
    w_sel = oracle.selection_weights(r.scores, idx_gpu, cfg.norm_topk_prob,
                                     cfg.routed_scaling_factor)
    dw = np.abs(w_gpu - w_sel)
    assert dw.max() <= 1e-6, f"{where}: max |dw| {dw.max():.3e} (token {dw.max(1).argmax()})"
    grouped = getattr(cfg, "n_group", 1) > 1
    every = np.ones(cfg.E, bool)
    n_other = 0
    for t in np.nonzero(~ok)[0]:
        row = idx_gpu[t]
        assert len(set(row.tolist())) == cfg.k and row.min() >= 0 and row.max() < cfg.E, where
        valid = _valid_grouped(cfg, r.keys[t], row) if grouped else _valid_topk(r.keys[t], row, every)
        assert valid, f"{where}: token {t} holds no valid top-k {row} (oracle {r.idx[t]})"
        n_other += int(np.any(row != r.idx[t]))
    if (~ok).any():
        log(f"{where}: {(~ok).sum()} near-tied tokens, {n_other} with another valid choice")
    return int((~ok).sum())


def assert_close(cfg, got: np.ndarray, ref: np.ndarray, where: str, mask=None, tol=None):
    if mask is not None:
        got, ref = got[mask], ref[mask]
    scale = oracle.rms(ref)
    err = np.abs(got - ref).max() if got.size else 0.0
    tol = tol_for(cfg) if tol is None else tol
    log(f"{where}: max|Δ|/rms = {err / scale:.3e} (tol {tol:.0e})")
    assert np.all(np.isfinite(got)), f"{where}: non-finite output"
    assert err <= tol * scale, f"{where}: max|Δ| {err:.4e} > {tol} * rms {scale:.4e}"
    return err / scale


# ------------------------------------------------------------------ workspace views

def ws_part(moe, ccfg, workspace: torch.Tensor, part: int, dtype, shape) -> torch.Tensor:
    """A view of one intermediate inside the layer workspace (moe_workspace_offset)."""
    off = moe.moe_workspace_offset(ccfg, part)
    assert off is not None, f"workspace part {part} absent"
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    assert off + n <= workspace.numel()
    return workspace[off:off + n].view(dtype).view(*shape)


def layer_routing(moe, lay):
    """(idx, w) the last layer forward on `lay` chose, read from its workspace."""
    cfg = lay.cfg
    idx = ws_part(moe, lay.ccfg, lay.workspace, moe.MOE_WS_TOPK_IDX, torch.int32, (cfg.T, cfg.k))
    w = ws_part(moe, lay.ccfg, lay.workspace, moe.MOE_WS_TOPK_W, torch.float32, (cfg.T, cfg.k))
    return idx.cpu().numpy(), w.cpu().numpy()


def check_layer_output(cfg, inp, out: np.ndarray, idx_gpu: np.ndarray, where: str, tokens=None,
                       r_all=None, w_gpu=None):
    """The layer output on `tokens` (all by default) against the oracle
    evaluated with the GPU's own choice of experts.  Routing is checked first
    (bit-exact away from near-ties, valid top-k on them); then every token,
    near-tied ones included, is compared.  Returns (max|Δ|/rms, LayerResult)."""
    tokens = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    if r_all is None:
        r_all = oracle.route_inputs(cfg, inp)
    if w_gpu is not None:
        check_routing(cfg, r_all, idx_gpu, w_gpu, where + " routing")
    res = oracle.layer_forward(cfg, inp, tokens=tokens, idx=idx_gpu[tokens])
    e = assert_close(cfg, out[tokens] if out.shape[0] == cfg.T else out, res.out, where)
    return e, res


def tied_tokens(r) -> np.ndarray:
    return np.nonzero(~untied(r))[0]


# ------------------------------------------------------------------ intermediates

def oracle_h_rows(cfg, inp, perm: np.ndarray, offsets: np.ndarray, rows: np.ndarray):
    """The oracle's h (before any rounding or quantisation, fp64) of the given
    sorted rows: routed row p < T*k is token perm[p] // k through expert e with
    offsets[e] <= p < offsets[e+1]; row T*k + s*T + t is token t through
    shared expert s."""
    _, x_e = oracle.layer_inputs(cfg, inp)
    W = oracle.Weights(cfg, inp)
    R = cfg.T * cfg.k
    rows = np.asarray(rows)
    grp = np.where(rows < R, np.searchsorted(offsets, rows, side="right") - 1,
                   cfg.E + (rows - R) // max(cfg.T, 1))
    tok = np.where(rows < R, perm[np.minimum(rows, R - 1)] // cfg.k, (rows - R) % max(cfg.T, 1))
    h = np.zeros((rows.size, cfg.I))
    for g in np.unique(grp):
        sel = np.nonzero(grp == g)[0]
        wg, wu, _ = W.expert(int(g))
        h[sel] = oracle.swiglu_hidden(x_e[tok[sel]], wg, wu)
    return h, grp, tok


def check_fp8_h_codes(cfg, h_ref: np.ndarray, codes: np.ndarray, scales: np.ndarray, where: str):
    """FP8 h codes of the GPU against the oracle's quantisation of its exact h.
    The fp8 MFMA sums each group of 8 products to ~17 bits of the largest one,
    so the GPU's h differs from the exact value by a small amount that scales
    with the products, not with h itself.  A GPU code is valid if it is the
    rounding of some value within delta of the exact h / scale, delta = 0.02
    code units (~100x the error expected at a block amax of 448 units) plus
    2e-4 of the value: its value lies between the oracle's encodings of
    q - delta and q + delta (rounding is monotone).  Near zero that admits the
    smallest code of either sign.  Scales (amax / 448) within 2e-4 relative.
    Returns the number of differing codes."""
    q_ref, s_ref = oracle.quantize_fp8_rows(h_ref.astype(np.float32))
    ds = np.abs(scales.astype(np.float64) / s_ref.astype(np.float64) - 1.0)
    assert ds.max() <= 2e-4, f"{where}: h scale off by {ds.max():.3e}"
    diff = np.nonzero(codes != q_ref)
    n = diff[0].size
    if n:
        q_exact = h_ref[diff] / np.repeat(s_ref.astype(np.float64), 128, 1)[diff]
        delta = 0.02 + 2e-4 * np.abs(q_exact)
        v_g = oracle.decode_e4m3(codes[diff])
        lo = oracle.decode_e4m3(oracle.encode_e4m3((q_exact - delta).astype(np.float32)))
        hi = oracle.decode_e4m3(oracle.encode_e4m3((q_exact + delta).astype(np.float32)))
        v_o = oracle.decode_e4m3(q_ref[diff])
        margin = np.abs(q_exact - 0.5 * (v_g + v_o))
        log(f"{where}: {n} of {codes.size} h codes differ ({n / codes.size:.2e}); "
            f"max |q - midpoint of the two codes| {margin.max():.3e} code units")
        ok = (v_g >= lo) & (v_g <= hi)
        assert ok.all(), (f"{where}: {(~ok).sum()} h codes are no rounding of a value within "
                          f"delta of the exact one (e.g. q={q_exact[~ok][:3]}, gpu={v_g[~ok][:3]})")
    else:
        log(f"{where}: all {codes.size} h codes equal the oracle's")
    return n
