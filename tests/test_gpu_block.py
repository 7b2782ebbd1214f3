"""GPU parity of the widened path, through the C ABI, against the fp64
oracle: group-limited routing (n_group / topk_group of the Transformers
dots.llm1 field table) and the decoder block around the layer (RMSNorm
before, residual after; single-layer figure of the Deep Dive, §3.3).

Bars as for the layer: routing indices bit-exact on every token away from a
1e-6 near-tie (selection, slot order or group boundary), weights within 1e-6;
RMSNorm outputs within one rounding of the activation type; block outputs
within max|Δ| <= 1e-4 / 2e-2 / 6e-2 x rms(oracle) for fp32 / bf16 / fp8.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import config, generate
from _gpu_helpers import (assert_close, bf16_round, check_layer_output, check_routing,
                          layer_routing, log, out_to_f64, tied_tokens, untied)

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
    base = dict(name="small", cfg_id=91, T=100, H=256, E=8, S=1, k=2, I=256, Is=256,
                act="bf16", expert="bf16")
    base.update(kw)
    if base["expert"] == "f32":
        base["act"] = "f32"
    base["Is"] = base["I"]
    return config(0).with_(**base)


def gamma_for(cfg, seed=5):
    """A seeded RMSNorm weight near 1, in storage format, and its fp64 value."""
    g = 1.0 + 0.1 * np.random.default_rng(seed).standard_normal(cfg.H)
    if cfg.act == "bf16":
        st = bf16_round(g)
        return st, oracle.decode_bf16(st)
    st = g.astype(np.float32)
    return st, st.astype(np.float64)


# ------------------------------------------------------------------ RMSNorm

@pytest.mark.parametrize("act,T,H", [("bf16", 300, 5120), ("bf16", 1, 4096), ("f32", 77, 512),
                                     ("bf16", 65, 128)])
def test_rmsnorm_matches_oracle(act, T, H):
    cfg = small(T=T, H=H, act=act, expert=act)
    log(f"rmsnorm {act} T={T} H={H}")
    inp = generate(cfg, weights=False)
    g_st, g = gamma_for(cfg)
    c = moe.make_config(T, H, cfg.E, cfg.S, cfg.k, cfg.I, act=act, expert=act)
    h = to_device(inp["x"], act)
    gamma = to_device(g_st, act)
    out = torch.empty_like(h)
    moe.moe_rmsnorm(c, h, gamma, cfg.rms_norm_eps, out)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(oracle.widen(inp["x"], act), g, cfg.rms_norm_eps)
    got = out_to_f64(out)
    if act == "bf16":
        # one rounding of an fp32 result: equal to the oracle's rounding of
        # the exact value, or one bf16 step away where the two straddle a
        # rounding boundary
        want = oracle.decode_bf16(oracle.encode_bf16(ref))
        step = np.abs(oracle.decode_bf16(oracle.encode_bf16(ref) + 1) - want)
        diff = np.abs(got - want)
        n_off = int((diff > 0).sum())
        log(f"rmsnorm bf16: {n_off} of {diff.size} values one step off")
        assert np.all(diff <= step * 1.0001)
        assert n_off <= max(2, diff.size // 1000)
    else:
        err = np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30))
        log(f"rmsnorm f32: max rel err {err:.3e}")
        assert err <= 2e-6


# ------------------------------------------------------------------ grouped routing

GROUP_CASES = {
    # DeepSeek-V3-style grouping on the dots3 router shape
    "E256_g8_t4_k8": lambda: config(2, T=2048, n_group=8, topk_group=4),
    # dots.llm1 shape with the skewed bias
    "E128_g4_t2_k6": lambda: config(3, T=2048, n_group=4, topk_group=2),
    # one expert per group
    "E64_g64_t8_k4": lambda: small(T=500, H=512, E=64, k=4, n_group=64, topk_group=8),
    # every group kept: the plain top-k
    "E32_g4_t4_k4": lambda: small(T=300, H=256, E=32, k=4, n_group=4, topk_group=4),
    # exactly k allowed experts
    "E16_g4_t2_k8": lambda: small(T=300, H=256, E=16, k=8, n_group=4, topk_group=2),
}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", list(GROUP_CASES))
def test_grouped_route_matches_oracle(case):
    cfg = GROUP_CASES[case]()
    log(f"grouped route {case}: T={cfg.T} E={cfg.E} k={cfg.k} groups {cfg.n_group}/{cfg.topk_group}")
    inp = generate(cfg, weights=False)
    c = moe.make_config(cfg.T, cfg.H, cfg.E, cfg.S, cfg.k, cfg.I, act=cfg.act, expert=cfg.expert,
                        n_group=cfg.n_group, topk_group=cfg.topk_group)
    # the device tensors must outlive the call: the struct holds raw pointers
    wr = to_device(inp["w_router"], cfg.act)
    b = to_device(inp["bias"], "f32")
    x = to_device(inp["x"], cfg.act)
    w = moe.make_weights(w_router=wr, router_bias=b)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    tw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    ties = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(moe.moe_workspace_size(c), 256), dtype=torch.uint8, device="cuda")
    moe.moe_route(c, x, w, idx, tw, ties, ws)
    torch.cuda.synchronize()
    r = oracle.route_inputs(cfg, inp)
    idx_h = idx.cpu().numpy()
    n = check_routing(cfg, r, idx_h, tw.cpu().numpy(), f"grouped route {case}")
    # every chosen expert lies in one of the chosen groups: at most
    # topk_group distinct groups per token
    G = cfg.E // cfg.n_group
    ngroups = np.array([len(set((row // G).tolist())) for row in idx_h])
    assert ngroups.max() <= cfg.topk_group
    log(f"grouped route {case}: oracle near-ties {n} (group {(r.gap_grp <= 1e-6).sum()}); "
        f"GPU tie counts {ties.cpu().tolist()}")


def test_grouped_layer_forward_small():
    cfg = small(T=300, H=512, E=32, S=1, k=4, I=256, n_group=8, topk_group=3)
    inp = generate(cfg)
    lay = DeviceLayer(cfg, inp)
    out = lay.forward()
    torch.cuda.synchronize()
    idx, w = layer_routing(moe, lay)
    check_layer_output(cfg, inp, out_to_f64(out), idx, "grouped layer", w_gpu=w)


def test_grouping_arguments_are_checked():
    base = dict(T=8, H=256, E=32, S=1, k=4, I=128)
    for ng, tg, k in ((3, 1, 4), (8, 0, 4), (8, 9, 4), (8, 1, 5), (-1, 1, 4)):
        c = moe.make_config(**{**base, "k": k}, n_group=ng, topk_group=tg)
        assert moe.moe_workspace_size(c) == 0, (ng, tg, k)
    c = moe.make_config(**base, n_group=128, topk_group=1, )
    assert moe.moe_workspace_size(c) == 0


# ------------------------------------------------------------------ block forward

BLOCK_CASES = {
    "C0": lambda: config(0),
    "bf16_small": lambda: small(T=150, H=512, E=16, S=1, k=4, I=256),
    "bf16_grouped": lambda: small(T=150, H=512, E=32, S=2, k=4, I=256, n_group=4, topk_group=2),
    "fp8_small": lambda: small(T=200, H=512, E=16, S=1, k=4, I=1536, expert="fp8"),
    # large-tile path: the residual joins the scaled fp16 y in a combine split
    # over 2 blocks per token
    "bf16_large_tile_split2": lambda: small(T=512, H=2048, E=8, S=1, k=2, I=256),
}


def _block(cfg, inp, lay, g_st):
    out = torch.empty_like(lay.t["x"])
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    ties = torch.empty(2, dtype=torch.int32, device="cuda")
    gamma = to_device(g_st, cfg.act)
    moe.moe_block_forward(lay.ccfg, lay.weights, lay.t["x"], gamma, cfg.rms_norm_eps, out,
                          counts, ties, lay.workspace)
    torch.cuda.synchronize()
    return out, counts, ties


def _normed_rows(cfg, inp, lay, g_st, g, where):
    """The block's normalised rows (moe_rmsnorm: the kernel the block runs),
    checked against the oracle's RMSNorm: bf16 rows equal the oracle's
    rounding of the exact value or lie one bf16 step from it where the two
    straddle a rounding boundary (as in test_rmsnorm_matches_oracle); fp32
    rows within 2e-6 relative.  Returns them in storage format."""
    xn = torch.empty_like(lay.t["x"])
    moe.moe_rmsnorm(lay.ccfg, lay.t["x"], to_device(g_st, cfg.act), cfg.rms_norm_eps, xn)
    torch.cuda.synchronize()
    _, xn_ref = oracle.block_inputs(cfg, inp, g)
    ref = oracle.widen(xn_ref, cfg.act)
    got = out_to_f64(xn)
    if cfg.act == "bf16":
        step = np.abs(oracle.decode_bf16(xn_ref + 1) - ref)
        assert np.all(np.abs(got - ref) <= step * 1.0001), f"{where}: RMSNorm rows"
        return xn.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.all(np.abs(got - ref) <= 2e-6 * np.maximum(np.abs(ref), 1e-30)), f"{where}: RMSNorm rows"
    return xn.cpu().numpy().astype(np.float32)


@pytest.mark.parametrize("case", list(BLOCK_CASES))
def test_block_forward_small(case):
    """The normalised rows are checked against the oracle's RMSNorm; routing
    and every output token against the oracle's layer on the block's own
    normalised rows (a row one bf16 step off at a rounding boundary moves its
    router scores by ~1e-5), with the block's choice of experts."""
    cfg = BLOCK_CASES[case]()
    log(f"block {case}: {cfg}")
    inp = generate(cfg)
    lay = DeviceLayer(cfg, inp)
    g_st, g = gamma_for(cfg)
    out, counts, _ = _block(cfg, inp, lay, g_st)
    idx, w = layer_routing(moe, lay)
    inp_n = dict(inp)
    inp_n["x"] = _normed_rows(cfg, inp, lay, g_st, g, f"block {case}")
    tokens = np.arange(cfg.T)
    res0 = oracle.layer_forward(cfg, inp_n, tokens)
    check_routing(cfg, res0.routing, idx, w, f"block {case} routing")
    # every token, against the oracle evaluated with the block's own choice
    res = oracle.layer_forward(cfg, inp_n, tokens, idx=idx)
    h = oracle.widen(inp["x"], cfg.act)
    ref = h + res.out
    assert_close(cfg, out_to_f64(out), ref, f"block {case}")
    # the MoE part alone, against the layer output of the oracle
    moe_part = out_to_f64(out) - h
    rnd = np.abs(ref) * (2.0 ** -8 if cfg.act == "bf16" else 2.0 ** -23)
    err = np.abs(moe_part - res.out) - rnd
    log(f"block {case}: MoE part max (|Δ| - output rounding)/rms = "
        f"{max(err.max(), 0) / oracle.rms(res.out):.3e}")
    np.testing.assert_array_equal(counts.cpu().numpy(), np.bincount(idx.ravel(), minlength=cfg.E))
    assert int(counts.sum()) == cfg.T * cfg.k


def test_block_forward_zero_gamma_is_identity():
    cfg = small(T=64, H=256, E=16, S=1, k=4, I=128)
    inp = generate(cfg)
    lay = DeviceLayer(cfg, inp)
    out, _, _ = _block(cfg, inp, lay, bf16_round(np.zeros(cfg.H)))
    np.testing.assert_array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), inp["x"])


@pytest.mark.timeout(900)
def test_block_forward_full_size_c2():
    cfg = config(2)
    log("block full C2: generating inputs")
    inp = generate(cfg)
    lay = DeviceLayer(cfg, inp)
    g_st, g = gamma_for(cfg)
    log("block full C2: forward")
    out, counts, ties = _block(cfg, inp, lay, g_st)
    idx, w = layer_routing(moe, lay)
    tokens = np.random.default_rng(202).choice(cfg.T, 128, replace=False)
    tokens = np.union1d(tokens, [0, cfg.T - 1])
    _, res0 = oracle.block_forward(cfg, inp, g, tokens=tokens)
    check_routing(cfg, res0.routing, idx[tokens], w[tokens], "block full C2 routing")
    ref, res = oracle.block_forward(cfg, inp, g, tokens=tokens, idx=idx[tokens])
    log(f"block full C2: GPU ties {ties.cpu().tolist()}")
    assert_close(cfg, out_to_f64(out)[tokens], ref, "block full C2")
    assert int(counts.sum()) == cfg.T * cfg.k


def test_block_arguments_are_checked():
    cfg = small(T=16, H=256, E=8, S=1, k=2, I=128)
    inp = generate(cfg)
    lay = DeviceLayer(cfg, inp)
    g = to_device(bf16_round(np.ones(cfg.H)), cfg.act)
    out = torch.full_like(lay.t["x"], 7)
    for args, code in (((lay.t["x"], g, -1.0, out), moe.MOE_ERR_INVALID_ARG),
                       ((lay.t["x"], g, float("nan"), out), moe.MOE_ERR_INVALID_ARG),
                       ((lay.t["x"], None, 1e-6, out), moe.MOE_ERR_INVALID_ARG),
                       ((lay.t["x"], g, 1e-6, lay.t["x"]), moe.MOE_ERR_INVALID_ARG)):
        with pytest.raises(moe.MoEError) as e:
            moe.moe_block_forward(lay.ccfg, lay.weights, args[0], args[1], args[2], args[3],
                                  None, None, lay.workspace)
        assert e.value.status == code
        with pytest.raises(moe.MoEError):
            moe.moe_rmsnorm(lay.ccfg, args[0], args[1], args[2], args[3])
    torch.cuda.synchronize()
    assert torch.all(out == 7)
