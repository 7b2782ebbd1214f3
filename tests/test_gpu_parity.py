"""GPU parity: every step of the HIP path, called through the C ABI, against
the fp64 oracle on the same seeded inputs.

Bars: routing indices bit-exact on every token whose top-k is not within 1e-6
of a tie (tied tokens counted and checked for validity), weights within 1e-6;
dispatch and FP8 activation codes bit-exact; outputs within max|Δ| <=
1e-4 / 2e-2 / 6e-2 x rms(oracle) for fp32 / bf16 / fp8.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from moe_inputs import config, generate
from _gpu_helpers import (assert_close, bf16_round, check_fp8_h_codes, check_layer_output,
                          check_routing, layer_routing, log, oracle_h_rows, out_to_f64,
                          tied_tokens, tol_for, untied, ws_part)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import sparse_moe_expert_amd as moe
    from sparse_moe_expert_amd.device import DeviceLayer, to_device


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def small(**kw):
    base = dict(name="small", cfg_id=90, T=100, H=256, E=8, S=1, k=2, I=256, Is=256,
                act="bf16", expert="bf16")
    base.update(kw)
    if base["expert"] == "f32":
        base["act"] = "f32"
    if "Is" not in kw:
        base["Is"] = base["I"]
    return config(0).with_(**base)


def ccfg(cfg):
    return moe.make_config(cfg.T, cfg.H, cfg.E, cfg.S, cfg.k, cfg.I, cfg.Is, act=cfg.act,
                           expert=cfg.expert, norm_topk_prob=cfg.norm_topk_prob,
                           routed_scaling_factor=cfg.routed_scaling_factor,
                           n_group=cfg.n_group, topk_group=cfg.topk_group)


def workspace(c):
    return torch.empty(max(moe.moe_workspace_size(c), 256), dtype=torch.uint8, device="cuda")


# ------------------------------------------------------------------ FP8 codes

def test_quantize_fp8_bitexact():
    import json, os
    rng = np.random.default_rng(21)
    rows, cols = 333, 640
    x32 = (rng.normal(size=(rows, cols)) * rng.uniform(1e-3, 30, size=(rows, 1))).astype(np.float32)
    x32[3, 128:256] = 0.0
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fp8_block_by_hand.json")))
    x32[7, :128] = 0.0
    x32[7, :len(g["values"])] = g["values"]
    bits = bf16_round(x32)
    xd = to_device(bits, "bf16")
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, cols // 128), dtype=torch.float32, device="cuda")
    log("quantize_fp8 rows=333 cols=640")
    moe.moe_quantize_fp8(xd, rows, cols, q, s)
    torch.cuda.synchronize()
    ref_q, ref_s = oracle.quantize_fp8_rows(oracle.decode_bf16(bits).astype(np.float32))
    gq, gs = q.cpu().numpy(), s.cpu().numpy()
    bad = np.argwhere(gq != ref_q)
    log(f"quantize_fp8: scale mismatches {(gs != ref_s).sum()}, code mismatches {len(bad)}")
    for r, c in bad[:8]:
        v = oracle.decode_bf16(bits[r, c])
        log(f"  [{r},{c}] x={v!r} scale={ref_s[r, c // 128]!r} gpu={gq[r, c]:#04x} oracle={ref_q[r, c]:#04x}")
    np.testing.assert_array_equal(s.cpu().numpy(), ref_s)
    np.testing.assert_array_equal(q.cpu().numpy(), ref_q)
    np.testing.assert_array_equal(q.cpu().numpy()[7, :len(g["expected_codes"])], g["expected_codes"])


# ------------------------------------------------------------------ routing

@pytest.mark.timeout(600)
@pytest.mark.parametrize("cid", [0, 1, 2, 3, 4])
def test_route_matches_oracle(cid):
    cfg = config(cid)
    log(f"route C{cid}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k}")
    inp = generate(cfg, weights=False)
    c = ccfg(cfg)
    x = to_device(inp["x"], cfg.act)
    wr = to_device(inp["w_router"], cfg.act)
    b = to_device(inp["bias"], "f32")
    w = moe.make_weights(w_router=wr, router_bias=b)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    tw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    ties = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    moe.moe_route(c, x, w, idx, tw, ties, workspace(c))
    torch.cuda.synchronize()
    r = oracle.route_inputs(cfg, inp)
    n = check_routing(cfg, r, idx.cpu().numpy(), tw.cpu().numpy(), f"route C{cid}")
    t = ties.cpu().numpy()
    log(f"route C{cid}: oracle near-tie tokens {n} (sel {(r.gap_sel <= 1e-6).sum()}, "
        f"ord {(r.gap_ord <= 1e-6).sum()}); GPU tie counts {t.tolist()}")
    assert t.min() >= 0 and t.max() <= cfg.T


@pytest.mark.parametrize("E,k,T", [(512, 16, 300), (320, 8, 300), (96, 6, 300), (33, 4, 300),
                                   (1, 1, 4096), (8, 2, 4096), (100, 4, 4096)])
def test_route_expert_counts(E, k, T):
    """Routing on expert counts that give 8, 5 of 8, 2 and 1 keys per lane
    (expert e = slot * 64 + lane), including a partly filled last slot.  At
    T = 4096 (bf16) the logits come from the large-tile GEMM with N = E
    columns: fewer than one 16-row weight tile (E = 1, 8) and a partial last
    tile (E = 100)."""
    cfg = small(T=T, H=256, E=E, S=1, k=k, I=128)
    log(f"route E={E} k={k}: T={cfg.T}")
    inp = generate(cfg, weights=False)
    c = ccfg(cfg)
    x = to_device(inp["x"], cfg.act)
    w = moe.make_weights(w_router=to_device(inp["w_router"], cfg.act),
                         router_bias=to_device(inp["bias"], "f32"))
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    tw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    moe.moe_route(c, x, w, idx, tw, None, workspace(c))
    torch.cuda.synchronize()
    r = oracle.route_inputs(cfg, inp)
    n = check_routing(cfg, r, idx.cpu().numpy(), tw.cpu().numpy(), f"route E={E}")
    log(f"route E={E}: near-tie tokens {n}")


# ------------------------------------------------------------------ dispatch

def _dispatch_cases():
    return ["C0", "C1", "C2", "C3", "ragged_T1000_E100_k6", "one_token_E256_k8",
            "E1_k1_T777", "E512_k16_T3000"]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", _dispatch_cases())
def test_dispatch_bitexact(case):
    if case.startswith("C"):
        cfg = config(int(case[1]))
        idx = oracle.route_inputs(cfg, generate(cfg, weights=False)).idx
        T, k, E = cfg.T, cfg.k, cfg.E
    else:
        T, E, k = {"ragged_T1000_E100_k6": (1000, 100, 6), "one_token_E256_k8": (1, 256, 8),
                   "E1_k1_T777": (777, 1, 1), "E512_k16_T3000": (3000, 512, 16)}[case]
        rng = np.random.default_rng(zlib.crc32(case.encode()))
        p = rng.random(E) ** 3          # uneven popularity, some experts rare or empty
        p /= p.sum()
        idx = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    log(f"dispatch {case}: T={T} E={E} k={k}")
    c = moe.make_config(T, 128, E, 1, k, 128, act="bf16", expert="bf16")
    d_idx = torch.from_numpy(idx).cuda()
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    moe.moe_dispatch(c, d_idx, counts, offsets, perm, inv, workspace(c))
    torch.cuda.synchronize()
    ref = oracle.dispatch(idx, E)
    np.testing.assert_array_equal(counts.cpu().numpy(), ref.counts)
    np.testing.assert_array_equal(offsets.cpu().numpy(), ref.offsets)
    np.testing.assert_array_equal(perm.cpu().numpy(), ref.perm)
    np.testing.assert_array_equal(inv.cpu().numpy(), ref.inv)
    log(f"dispatch {case}: empty experts {(ref.counts == 0).sum()}, max rows {ref.counts.max()}")


# ------------------------------------------------------------------ combine

@pytest.mark.parametrize("act,T,H,k,S", [("f32", 50, 256, 4, 1), ("bf16", 300, 512, 8, 2),
                                         ("bf16", 33, 128, 3, 0), ("bf16", 256, 5120, 8, 1)])
def test_combine_matches_oracle(act, T, H, k, S):
    """fp32 expert outputs in, one rounding to the output type: the bf16
    result must be within half a bf16 step of the exact sum (plus fp32
    accumulation noise), the fp32 result within fp32 accumulation noise."""
    rng = np.random.default_rng(31)
    R = T * k
    y = rng.normal(size=(R, H)).astype(np.float32)
    ysh = rng.normal(size=(S, T, H)).astype(np.float32)
    w = rng.uniform(0.05, 1, size=(T, k))
    w = (w / w.sum(1, keepdims=True)).astype(np.float32)
    inv = rng.permutation(R).astype(np.int32)
    dy, dysh = to_device(y, "f32"), to_device(ysh, "f32")
    if S == 0:
        dysh = None
    out = torch.empty((T, H), dtype=torch.bfloat16 if act == "bf16" else torch.float32,
                      device="cuda")
    c = moe.make_config(T, H, 8, S, k, 128, act=act, expert=act)
    log(f"combine {act} T={T} H={H} k={k} S={S}")
    moe.moe_combine(c, dy, dysh, torch.from_numpy(w).cuda(), torch.from_numpy(inv).cuda(), out)
    torch.cuda.synchronize()
    ref = oracle.combine(y.astype(np.float64), ysh.astype(np.float64), w.astype(np.float64),
                         inv, k)
    got = out_to_f64(out)
    rel_out = 2.0 ** -8 if act == "bf16" else 0.0
    err = np.abs(got - ref) - rel_out * np.abs(ref)
    assert err.max() <= 1e-5 * oracle.rms(ref), err.max()


# ------------------------------------------------------------------ grouped FFN

FFN_CASES = {
    "C0": lambda: config(0),
    "bf16_small": lambda: small(),
    "bf16_ragged_S2": lambda: small(T=77, H=384, E=40, S=2, k=3, I=256),
    # FP8 cases use the method's intermediate size (moe_intermediate 1536): the
    # fp8 MFMA's inner sums keep ~17 bits per 8-product group, so h codes on a
    # rounding boundary may differ from the exact oracle's, and with a small I
    # one such code is an outsized share of y.
    "fp8_small": lambda: small(T=100, H=512, E=8, S=1, k=2, I=1536, expert="fp8"),
    "f32_S0": lambda: small(T=60, H=256, E=5, S=0, k=2, I=128, expert="f32"),
}


@pytest.mark.parametrize("case", list(FFN_CASES))
def test_grouped_ffn_matches_oracle(case):
    cfg = FFN_CASES[case]()
    log(f"grouped_ffn {case}: {cfg}")
    inp = generate(cfg)
    lay = DeviceLayer(cfg, inp)
    r = oracle.route_inputs(cfg, inp)
    d = oracle.dispatch(r.idx, cfg.E)
    perm = torch.from_numpy(d.perm).cuda()
    offsets = torch.from_numpy(d.offsets).cuda()
    R = cfg.T * cfg.k
    y = torch.empty((R, cfg.H), dtype=torch.float32, device="cuda")
    ysh = torch.empty((max(cfg.S, 1), cfg.T, cfg.H), dtype=torch.float32, device="cuda")
    moe.moe_grouped_ffn(lay.ccfg, lay.t["x"], lay.weights, perm, offsets, y,
                        ysh if cfg.S else None, lay.workspace)
    torch.cuda.synchronize()
    _, y_ref, _, ysh_ref = oracle.sorted_expert_rows(cfg, inp, r, d)
    assert_close(cfg, out_to_f64(y), y_ref, f"grouped_ffn {case} routed")
    if cfg.S:
        assert_close(cfg, out_to_f64(ysh)[:cfg.S], ysh_ref, f"grouped_ffn {case} shared")


# ------------------------------------------------------------------ whole layer, small

LAYER_CASES = {
    "C0": lambda: config(0),
    "bf16_ragged_S2": lambda: small(T=77, H=384, E=40, S=2, k=3, I=256),
    "bf16_S0": lambda: small(T=64, H=256, E=16, S=0, k=4, I=128),
    "bf16_E1_k1": lambda: small(T=50, H=256, E=1, S=1, k=1, I=128),
    "bf16_E33": lambda: small(T=70, H=256, E=33, S=1, k=5, I=128),
    "bf16_T1": lambda: small(T=1, H=512, E=64, S=1, k=8, I=256),
    "bf16_k16_E64": lambda: small(T=40, H=256, E=64, S=1, k=16, I=128),
    "bf16_midT": lambda: small(T=600, H=512, E=32, S=1, k=8, I=256),
    # an input whose largest |out| is ~5.6 rms: rounding the exact output to
    # bf16 alone costs 1.67e-2 rms there, so h must reach the down GEMM with
    # more than bf16 precision to stay under 2e-2 (64 rows per expert: the
    # mid-size kernel, h as two bf16 terms)
    "bf16_rounding_tail": lambda: small(T=256, H=768, E=32, S=1, k=8, I=256),
    "bf16_rounding_tail_decode": lambda: small(T=256, H=768, E=256, S=1, k=8, I=256),
    "fp8_small": lambda: small(T=200, H=512, E=16, S=1, k=4, I=1536, expert="fp8"),
    "fp8_midT": lambda: small(T=700, H=512, E=16, S=2, k=4, I=1536, expert="fp8"),
    # I not a multiple of the 256-column gate/up tile: the last tile's upper
    # waves skip their work (bf16 covered by the T=8192 workload, I = 1408)
    "fp8_partial_tile": lambda: small(T=700, H=512, E=16, S=1, k=4, I=1408, expert="fp8"),
    # FP8 at decode sizes (<= 24 rows per expert: the 16-row generic tiles)
    "fp8_decode16": lambda: small(T=64, H=512, E=16, S=1, k=4, I=1536, expert="fp8"),
    "fp8_decode2_empty": lambda: small(T=16, H=512, E=64, S=1, k=8, I=1536, expert="fp8"),
    "fp8_decode_S2": lambda: small(T=48, H=768, E=32, S=2, k=6, I=1536, expert="fp8"),
    "f32_ragged": lambda: small(T=45, H=384, E=12, S=1, k=3, I=256, expert="f32"),
    # T >= 4096 in bf16: the router logits go through the large-tile kernel
    # with N = E output columns.  E below one 16-row weight tile (the one
    # dense expert), and E not a multiple of 16 (a partial last tile).
    "bf16_T4096_E1_dense": lambda: small(T=4096, H=512, E=1, S=0, k=1, I=256),
    "bf16_T4096_E8": lambda: small(T=4096, H=256, E=8, S=1, k=2, I=128),
    "bf16_T4096_E100": lambda: small(T=4096, H=512, E=100, S=1, k=4, I=128),
    # large-tile path (scaled fp16 h and y) with the combine splitting each
    # token's columns over 2 and 4 blocks (T < 1024, H >= 2048)
    "bf16_large_tile_combine_split2": lambda: small(T=512, H=2048, E=8, S=1, k=2, I=256),
    "bf16_large_tile_combine_split4": lambda: small(T=256, H=4096, E=4, S=1, k=2, I=256),
}


# Cases that miss the bar, with the measured reason (kept, expected to fail).
LAYER_XFAIL = {}


@pytest.mark.parametrize("case", [
    pytest.param(c, marks=pytest.mark.xfail(strict=True, reason=LAYER_XFAIL[c]))
    if c in LAYER_XFAIL else c for c in LAYER_CASES])
def test_layer_forward_small(case):
    """Every token, near-tied ones included: the oracle is evaluated with the
    choice of experts the layer made (read from its workspace), after that
    choice is checked (bit-exact away from near-ties, a valid top-k on them)."""
    cfg = LAYER_CASES[case]()
    log(f"layer {case}: {cfg}")
    inp = generate(cfg)
    lay = DeviceLayer(cfg, inp)
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    ties = torch.empty(2, dtype=torch.int32, device="cuda")
    out = lay.forward(counts=counts, ties=ties)
    torch.cuda.synchronize()
    idx, w = layer_routing(moe, lay)
    check_layer_output(cfg, inp, out_to_f64(out), idx, f"layer {case}", w_gpu=w)
    np.testing.assert_array_equal(counts.cpu().numpy(), np.bincount(idx.ravel(), minlength=cfg.E))
    assert int(counts.sum()) == cfg.T * cfg.k


# ------------------------------------------------------------------ intermediates of the layer

INTERMEDIATE_CASES = {
    "bf16_decode_split": lambda: small(T=64, H=512, E=64, S=1, k=4, I=256),
    "bf16_mid_split": lambda: small(T=256, H=768, E=32, S=1, k=8, I=256),
    "bf16_big_scaled_f16": lambda: small(T=600, H=512, E=32, S=2, k=8, I=384),
    "fp8_small": lambda: small(T=200, H=512, E=16, S=1, k=4, I=1536, expert="fp8"),
    "fp8_decode": lambda: small(T=64, H=512, E=16, S=2, k=4, I=1536, expert="fp8"),
    "fp8_midT": lambda: small(T=700, H=512, E=16, S=2, k=4, I=1536, expert="fp8"),
}


@pytest.mark.parametrize("case", list(INTERMEDIATE_CASES))
def test_layer_intermediates(case):
    """h and y as the layer leaves them in its workspace.
    bf16: h within its rounding of the exact h plus 1e-5 rms(h) of fp32
    accumulation: 2^-16 relative for two bf16 terms (h and its residue); for
    scaled fp16 codes c with block exponents e (h = c * 2^e), 2^-11 relative
    plus 2^-25 * 2^e (fp16 subnormals), and each block's largest |c| in
    [2^14, 2^15] (or a block of zeros with e = 0).
    fp8: h codes equal the oracle's except at rounding boundaries (see
    check_fp8_h_codes); then y, recomputed by the oracle from the GPU's own h
    codes, within 1e-3 rms (the fp8 MFMA's ~17-bit group sums); and the layer
    output against the oracle fed those codes within the bf16 bar."""
    cfg = INTERMEDIATE_CASES[case]()
    log(f"intermediates {case}: {cfg}")
    inp = generate(cfg)
    lay = DeviceLayer(cfg, inp)
    out = lay.forward()
    torch.cuda.synchronize()
    idx, w = layer_routing(moe, lay)
    R, rows_all = cfg.T * cfg.k, cfg.T * cfg.k + cfg.S * cfg.T
    c, ws = lay.ccfg, lay.workspace
    perm = ws_part(moe, c, ws, moe.MOE_WS_PERM, torch.int32, (R,)).cpu().numpy()
    offs = ws_part(moe, c, ws, moe.MOE_WS_OFFSETS, torch.int32, (cfg.E + 1,)).cpu().numpy()
    d = oracle.dispatch(idx, cfg.E)
    np.testing.assert_array_equal(perm, d.perm)
    np.testing.assert_array_equal(offs, d.offsets)
    rows = np.arange(rows_all)
    h_ref, grp, tok = oracle_h_rows(cfg, inp, perm, offs, rows)
    W = oracle.Weights(cfg, inp)
    if cfg.expert == "bf16":
        split = moe.moe_workspace_offset(c, moe.MOE_WS_H_LO) is not None
        scaled = moe.moe_workspace_offset(c, moe.MOE_WS_H_EXP) is not None
        assert split != scaled, "bf16 h is either two bf16 terms or scaled fp16"
        if split:
            h_gpu = (oracle.decode_bf16(ws_part(moe, c, ws, moe.MOE_WS_H, torch.int16,
                                                (rows_all, cfg.I)).cpu().numpy().view(np.uint16))
                     + oracle.decode_bf16(ws_part(moe, c, ws, moe.MOE_WS_H_LO, torch.int16,
                                                  (rows_all, cfg.I)).cpu().numpy().view(np.uint16)))
            bound = 2.0 ** -16 * np.abs(h_ref)
        else:
            nb = -(-cfg.I // 256)
            codes = (ws_part(moe, c, ws, moe.MOE_WS_H, torch.float16, (rows_all, cfg.I))
                     .cpu().numpy().astype(np.float64))
            ex = ws_part(moe, c, ws, moe.MOE_WS_H_EXP, torch.int32, (rows_all, nb)).cpu().numpy()
            ex_col = np.repeat(ex, 256, axis=1)[:, :cfg.I].astype(np.float64)
            h_gpu = codes * np.exp2(ex_col)
            bound = 2.0 ** -11 * np.abs(h_ref) + 2.0 ** -25 * np.exp2(ex_col)
            for b in range(nb):
                amax = np.abs(codes[:, 256 * b:256 * (b + 1)]).max(axis=1)
                ok = ((amax >= 2.0 ** 14) & (amax <= 2.0 ** 15)) | ((amax == 0) & (ex[:, b] == 0))
                assert ok.all(), f"{case}: block {b} codes out of [2^14, 2^15]: {amax[~ok][:4]}"
        excess = np.abs(h_gpu - h_ref) - bound
        log(f"intermediates {case}: h {'two bf16 terms' if split else 'scaled fp16'}; max (|Δh| - "
            f"rounding)/rms(h) = {max(excess.max(), 0) / oracle.rms(h_ref):.3e}")
        assert excess.max() <= 1e-5 * oracle.rms(h_ref)
        if split:
            return
        # y in the same scaled fp16 form (exponents per row and 256 output
        # columns), against y recomputed in fp64 from the GPU's own h: one
        # fp16 rounding of y plus 1e-4 rms(y) for the fp32 sums and for h
        # brought to one exponent per row before the MFMAs.
        nby = -(-cfg.H // 256)
        yc = np.concatenate([
            ws_part(moe, c, ws, moe.MOE_WS_Y, torch.float16, (R, cfg.H)).cpu().numpy(),
            (ws_part(moe, c, ws, moe.MOE_WS_Y_SHARED, torch.float16, (cfg.S * cfg.T, cfg.H))
             .cpu().numpy() if cfg.S else np.zeros((0, cfg.H), np.float16))]).astype(np.float64)
        yex = ws_part(moe, c, ws, moe.MOE_WS_Y_EXP, torch.int32, (rows_all, nby)).cpu().numpy()
        yex_col = np.repeat(yex, 256, axis=1)[:, :cfg.H].astype(np.float64)
        y_gpu = yc * np.exp2(yex_col)
        for b in range(nby):
            amax = np.abs(yc[:, 256 * b:256 * (b + 1)]).max(axis=1)
            ok = ((amax >= 2.0 ** 14) & (amax <= 2.0 ** 15)) | ((amax == 0) & (yex[:, b] == 0))
            assert ok.all(), f"{case}: y block {b} codes out of [2^14, 2^15]: {amax[~ok][:4]}"
        y_ref = np.zeros((rows_all, cfg.H))
        for g in np.unique(grp):
            sel = np.nonzero(grp == g)[0]
            y_ref[sel] = h_gpu[sel] @ W.expert(int(g))[2].T
        y_excess = np.abs(y_gpu - y_ref) - 2.0 ** -11 * np.abs(y_ref) - 2.0 ** -25 * np.exp2(yex_col)
        log(f"intermediates {case}: y scaled fp16; max (|Δy| - rounding)/rms(y) = "
            f"{max(y_excess.max(), 0) / oracle.rms(y_ref):.3e}")
        assert y_excess.max() <= 1e-4 * oracle.rms(y_ref)
        return
    y_gpu = ws_part(moe, c, ws, moe.MOE_WS_Y, torch.float32, (R, cfg.H)).cpu().numpy()
    ysh_gpu = (ws_part(moe, c, ws, moe.MOE_WS_Y_SHARED, torch.float32, (cfg.S, cfg.T, cfg.H))
               .cpu().numpy() if cfg.S else np.zeros((0, cfg.T, cfg.H)))
    # fp8
    codes = ws_part(moe, c, ws, moe.MOE_WS_H, torch.uint8, (rows_all, cfg.I)).cpu().numpy()
    scales = ws_part(moe, c, ws, moe.MOE_WS_H_SCALES, torch.float32,
                     (rows_all, cfg.I // 128)).cpu().numpy()
    check_fp8_h_codes(cfg, h_ref, codes, scales, f"intermediates {case}")
    hd = oracle.dequantize_fp8_rows(codes, scales)
    y_ref = np.zeros((rows_all, cfg.H))
    for g in np.unique(grp):
        sel = np.nonzero(grp == g)[0]
        y_ref[sel] = hd[sel] @ W.expert(int(g))[2].T
    y_all = np.concatenate([y_gpu, ysh_gpu.reshape(-1, cfg.H)])
    assert_close(cfg, y_all, y_ref, f"intermediates {case} y from the GPU's h codes", tol=1e-3)
    r = oracle.route_inputs(cfg, inp)
    wsel = oracle.selection_weights(r.scores, idx, cfg.norm_topk_prob, cfg.routed_scaling_factor)
    out_ref = oracle.combine(y_ref[:R], y_ref[R:].reshape(cfg.S, cfg.T, cfg.H), wsel, d.inv, cfg.k)
    assert_close(cfg, out_to_f64(out), out_ref, f"intermediates {case} out from the GPU's h codes",
                 tol=2e-2)


# ------------------------------------------------------------------ whole layer, full size

FULL_CASES = [(1, 0), (2, 0), (3, 0), (4, 0), (1, 1), (1, 2), (2, 1), (2, 2)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid,seed", FULL_CASES, ids=[f"C{c}_seed{s}" for c, s in FULL_CASES])
def test_layer_forward_full_size(cid, seed):
    """The full workload shapes, in the launch configuration the benchmark times.
    Routing is checked on all tokens; the output on all tokens (T=256) or on
    a seeded sample of 128 tokens plus every near-tied token (the layer is
    per-token independent, so a token's output does not depend on which
    others are evaluated), against the oracle evaluated with the GPU's own
    choice of experts."""
    cfg = config(cid)
    log(f"layer full C{cid} seed {seed}: generating inputs")
    inp = generate(cfg, seed=seed)
    lay = DeviceLayer(cfg, inp)
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    ties = torch.empty(2, dtype=torch.int32, device="cuda")
    log(f"layer full C{cid} seed {seed}: forward")
    out = lay.forward(counts=counts, ties=ties)
    torch.cuda.synchronize()
    idx_h, w_h = layer_routing(moe, lay)
    r_all = oracle.route_inputs(cfg, inp)
    n_tied = check_routing(cfg, r_all, idx_h, w_h, f"layer full C{cid} routing")
    np.testing.assert_array_equal(counts.cpu().numpy(), np.bincount(idx_h.ravel(), minlength=cfg.E))
    cnt = counts.cpu().numpy()
    log(f"layer full C{cid} seed {seed}: near-tie tokens {n_tied}; GPU ties {ties.cpu().tolist()}; "
        f"rows/expert max {cnt.max()} mean {cnt.mean():.1f}; empty {(cnt == 0).sum()}")
    if cfg.T <= 256:
        tokens = np.arange(cfg.T)
    else:
        tokens = np.random.default_rng(100 + cid + 10 * seed).choice(cfg.T, 128, replace=False)
        tokens = np.union1d(np.union1d(tokens, [0, cfg.T - 1]), tied_tokens(r_all))
    check_layer_output(cfg, inp, out_to_f64(out), idx_h, f"layer full C{cid} seed {seed}",
                       tokens=tokens)


# ------------------------------------------------------------------ determinism, streams, errors

def test_deterministic_and_stream_independent():
    cfg = small(T=512, H=1024, E=64, S=1, k=8, I=512)
    inp = generate(cfg)
    lay = DeviceLayer(cfg, inp)
    a = lay.forward().clone()
    b = lay.forward().clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # two streams, separate workspaces and outputs, enqueued back to back
    ws2 = torch.empty_like(lay.workspace)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    o1, o2 = lay.empty_out(), lay.empty_out()
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        moe.moe_layer_forward(lay.ccfg, lay.weights, lay.t["x"], o1, workspace=lay.workspace,
                              stream=s1)
    with torch.cuda.stream(s2):
        moe.moe_layer_forward(lay.ccfg, lay.weights, lay.t["x"], o2, workspace=ws2, stream=s2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), a.view(torch.int16))
    assert torch.equal(o2.view(torch.int16), a.view(torch.int16))


def test_errors_leave_output_untouched():
    cfg = small()
    lay = DeviceLayer(cfg, generate(cfg))
    out = torch.full((cfg.T, cfg.H), 3.0, dtype=lay.act_dtype, device="cuda")
    small_ws = lay.workspace[: lay.ws_bytes // 2]
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_layer_forward(lay.ccfg, lay.weights, lay.t["x"], out, workspace=small_ws)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
    c0 = moe.make_config(0, cfg.H, cfg.E, cfg.S, cfg.k, cfg.I)
    moe.moe_layer_forward(c0, lay.weights, lay.t["x"], out, workspace=lay.workspace)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


def test_stream_read_folds_every_word():
    """The read-ceiling utility touches every 16-byte chunk: its per-block
    XOR fold equals the host fold of the same chunk assignment (chunk q to
    block (q // 256) % blocks over the grid-stride loop)."""
    rng = np.random.default_rng(41)
    blocks, n_chunks = 64, 64 * 256 * 5 + 77
    words = rng.integers(0, 2 ** 32, size=n_chunks * 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    moe.moe_stream_read(src, n_chunks * 16, sink, blocks)
    torch.cuda.synchronize()
    fold = np.bitwise_xor.reduce(words.reshape(n_chunks, 4), axis=1)
    blk = (np.arange(n_chunks) // 256) % blocks
    want = np.zeros(blocks, np.uint32)
    np.bitwise_xor.at(want, blk, fold)
    np.testing.assert_array_equal(sink.cpu().numpy().view(np.uint32), want)
