"""Pins for the oracle's expert and layer arithmetic: the hand-derived layer,
a textbook dense SwiGLU when E = k = 1, brute-force dense evaluation of every
expert, and symmetries the layer must have."""
import json
import math
import os
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import oracle
from moe_inputs import config, generate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
L3 = math.log(3.0)


def _golden_layer():
    g = json.load(open(os.path.join(GOLDEN, "tiny_layer_by_hand.json")))
    d = g["dims"]
    cfg = SimpleNamespace(T=d["T"], H=d["H"], E=d["E"], S=d["S"], k=d["k"], I=d["I"],
                          Is=d["Is"], act="f64", expert="f64", norm_topk_prob=True,
                          routed_scaling_factor=1.0, n_group=1, topk_group=1)
    wg = np.array(g["w_gate_in_units_of_ln3"]) * L3
    wu = np.array(g["w_up"], float)
    inp = {
        "x": np.array(g["x"], float),
        "w_router": np.array(g["w_router_in_units_of_ln3"]) * L3,
        "bias": np.array(g["bias"]),
        "w_gate_up": np.concatenate([wg, wu], axis=1),
        "w_down": np.array(g["w_down"], float),
        "w_sh_gate_up": np.concatenate([np.array(g["w_sh_gate_in_units_of_ln3"]) * L3,
                                        np.array(g["w_sh_up"], float)], axis=1),
        "w_sh_down": np.array(g["w_sh_down"], float),
    }
    return g, cfg, inp


def test_layer_golden_by_hand():
    g, cfg, inp = _golden_layer()
    res = oracle.layer_forward(cfg, inp)
    np.testing.assert_allclose(res.out, np.array(g["expected"]["out_in_units_of_ln3"]) * L3,
                               rtol=0, atol=1e-14)
    np.testing.assert_array_equal(res.routing.idx, g["expected"]["idx"])
    np.testing.assert_allclose(oracle.dense_layer_forward(cfg, inp), res.out, atol=1e-14)


def test_swiglu_matches_torch_silu():
    rng = np.random.default_rng(9)
    a, wg, wu = rng.normal(size=(6, 20)), rng.normal(size=(7, 20)), rng.normal(size=(7, 20))
    ref = (torch.nn.functional.silu(torch.from_numpy(a @ wg.T)) * torch.from_numpy(a @ wu.T)).numpy()
    np.testing.assert_allclose(oracle.swiglu_hidden(a, wg, wu), ref, rtol=1e-13, atol=1e-15)


def _small_cfg(**kw):
    base = dict(T=24, H=128, E=6, S=1, k=2, I=128, Is=128, act="f32", expert="f32")
    base.update(kw)
    return config(0).with_(**base)


def test_single_expert_is_dense_swiglu():
    """E = k = 1: the only expert gets weight 1 on every token, so the layer is
    two textbook SwiGLU MLPs (torch.nn.functional.silu, fp64) added."""
    cfg = _small_cfg(E=1, k=1)
    inp = generate(cfg)
    out = oracle.layer_forward(cfg, inp).out
    x = torch.from_numpy(inp["x"].astype(np.float64))

    def mlp(gu, dn):
        gu = torch.from_numpy(gu.astype(np.float64))
        dn = torch.from_numpy(dn.astype(np.float64))
        I = gu.shape[0] // 2
        h = torch.nn.functional.silu(x @ gu[:I].T) * (x @ gu[I:].T)
        return h @ dn.T

    ref = mlp(inp["w_gate_up"][0], inp["w_down"][0]) + mlp(inp["w_sh_gate_up"][0], inp["w_sh_down"][0])
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("cfg_kw", [dict(), dict(S=2, k=3, E=7, I=256), dict(expert="fp8", act="bf16")])
def test_sparse_equals_dense_bruteforce(cfg_kw):
    cfg = _small_cfg(**cfg_kw)
    inp = generate(cfg)
    sparse = oracle.layer_forward(cfg, inp).out
    dense = oracle.dense_layer_forward(cfg, inp)
    np.testing.assert_allclose(sparse, dense, rtol=0, atol=1e-12 * oracle.rms(dense))


def test_sparse_equals_dense_bruteforce_c0():
    cfg = config(0)
    inp = generate(cfg)
    sparse = oracle.layer_forward(cfg, inp).out
    dense = oracle.dense_layer_forward(cfg, inp)
    np.testing.assert_allclose(sparse, dense, rtol=0, atol=1e-12 * oracle.rms(dense))


def test_sorted_rows_and_combine_agree_with_layer():
    cfg = _small_cfg(S=2, k=3)
    inp = generate(cfg)
    res = oracle.layer_forward(cfg, inp)
    d = oracle.dispatch(res.routing.idx, cfg.E)
    h_s, y_s, h_sh, y_sh = oracle.sorted_expert_rows(cfg, inp, res.routing, d)
    out = oracle.combine(y_s, y_sh, res.routing.w, d.inv, cfg.k)
    np.testing.assert_allclose(out, res.out, rtol=0, atol=1e-13 * oracle.rms(out))
    np.testing.assert_allclose(y_s[d.inv].reshape(cfg.T, cfg.k, cfg.H), res.y, atol=1e-14)


def test_zero_input_gives_zero_output():
    cfg = _small_cfg()
    inp = generate(cfg)
    inp["x"] = np.zeros_like(inp["x"])
    assert not np.any(oracle.layer_forward(cfg, inp).out)


def test_identical_experts_ignore_routing():
    """All routed experts equal: the routed sum is that expert's output, since
    the renormalised weights sum to 1, whatever the routing chose."""
    cfg = _small_cfg(E=5, k=3)
    inp = generate(cfg)
    inp["w_gate_up"][:] = inp["w_gate_up"][0]
    inp["w_down"][:] = inp["w_down"][0]
    out = oracle.layer_forward(cfg, inp).out
    W = oracle.Weights(cfg, inp)
    x = oracle.widen(inp["x"], cfg.act)
    ref = oracle.expert_forward(cfg, x, *W.expert(0)) + oracle.expert_forward(cfg, x, *W.expert(cfg.E))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13 * oracle.rms(ref))


def test_token_permutation_equivariance():
    cfg = _small_cfg()
    inp = generate(cfg)
    out = oracle.layer_forward(cfg, inp).out
    p = np.random.default_rng(10).permutation(cfg.T)
    inp2 = dict(inp, x=inp["x"][p])
    np.testing.assert_allclose(oracle.layer_forward(cfg, inp2).out, out[p], atol=1e-14)
    sub = oracle.layer_forward(cfg, inp, tokens=p[:5]).out
    np.testing.assert_allclose(sub, out[p[:5]], atol=1e-14)


def test_expert_relabelling_invariance():
    cfg = _small_cfg(E=8, k=3)
    inp = generate(cfg)
    res = oracle.layer_forward(cfg, inp)
    q = np.random.default_rng(11).permutation(cfg.E)
    inp2 = dict(inp, w_router=inp["w_router"][q], bias=inp["bias"][q],
                w_gate_up=inp["w_gate_up"][q], w_down=inp["w_down"][q])
    res2 = oracle.layer_forward(cfg, inp2)
    ok = (res.routing.gap_sel > 1e-9) & (res.routing.gap_ord > 1e-9)
    assert ok.sum() >= cfg.T - 1
    np.testing.assert_allclose(res2.out[ok], res.out[ok], atol=1e-14)
    np.testing.assert_array_equal(q[res2.routing.idx[ok]], res.routing.idx[ok])


def test_fp8_layer_close_to_unquantised():
    """FP8 emulation only perturbs the layer by quantisation noise: compared
    with the same dequantised weights and unquantised activations, the relative
    error is a few percent (3 mantissa bits: relative rounding error up to
    2^-4 per element, about 3.6% rms, applied to x and to h)."""
    cfg = _small_cfg(expert="fp8", act="bf16", E=4, k=2, H=256, I=256, Is=128)
    inp = generate(cfg)
    out = oracle.layer_forward(cfg, inp).out
    # reference: same weights, activations and h not quantised
    W = oracle.Weights(cfg, inp)
    x = oracle.widen(inp["x"], "bf16")
    r = oracle.route_inputs(cfg, inp)
    ref = np.zeros_like(out)
    for s in range(cfg.S):
        wg, wu, wd = W.expert(cfg.E + s)
        ref += oracle.swiglu_hidden(x, wg, wu) @ wd.T
    for t in range(cfg.T):
        for j in range(cfg.k):
            wg, wu, wd = W.expert(int(r.idx[t, j]))
            ref[t] += r.w[t, j] * (oracle.swiglu_hidden(x[t:t + 1], wg, wu) @ wd.T)[0]
    rel = oracle.rms(out - ref) / oracle.rms(ref)
    assert 1e-3 < rel < 0.08


def _fp8_expert_fixture():
    """The hand-derived FP8 expert of tests/golden/fp8_expert_by_hand.json as
    layer inputs in storage format (E = 1 routed expert, k = 1, and the same
    weights as the one shared expert)."""
    g = json.load(open(os.path.join(GOLDEN, "fp8_expert_by_hand.json")))
    T, H, I = g["dims"]["T"], g["dims"]["H"], g["dims"]["I"]
    x = np.zeros((T, H), np.uint16)
    x[0, 0] = x[1, 1] = 0x43E0                        # bf16 448.0
    gu = np.zeros((2 * I, H), np.uint8)
    gu[:I, 0] = gu[:I, 1] = 0x28                      # 0.25
    for i, code, _ in g["w_up_codes_token0_column0"]:
        gu[I + i, 0] = int(code, 16)
    for i, code, _ in g["w_up_codes_token1_column1"]:
        gu[I + i, 1] = int(code, 16)
    s_gu = np.array([[1.0], [1.0], [2.0 ** -10], [2.0 ** -10]], np.float32)
    dn = np.zeros((H, I), np.uint8)
    dn[np.arange(H), np.arange(H)] = 0x38             # 1.0
    dn[np.arange(H), 128 + np.arange(H)] = 0x30       # 0.5
    s_dn = np.ones((1, 2), np.float32)
    cfg = SimpleNamespace(T=T, H=H, E=1, S=1, k=1, I=I, Is=I, act="bf16", expert="fp8",
                          norm_topk_prob=True, routed_scaling_factor=1.0, n_group=1,
                          topk_group=1)
    inp = {"x": x, "w_router": np.zeros((1, H), np.uint16), "bias": np.zeros(1, np.float32),
           "w_gate_up": gu[None], "w_down": dn[None], "s_gate_up": s_gu[None],
           "s_down": s_dn[None], "w_sh_gate_up": gu[None], "w_sh_down": dn[None],
           "s_sh_gate_up": s_gu[None], "s_sh_down": s_dn[None]}
    exp = np.zeros((T, H))
    unq = np.zeros((T, H))
    for t in range(T):
        for o, v in g["expected_y"][f"token{t}"]:
            exp[t, o] = v
        for o, v in g["unquantised_y_for_contrast"][f"token{t}"]:
            unq[t, o] = v
    return cfg, inp, exp, unq


def test_fp8_expert_golden_by_hand():
    """expert_forward quantises h per token and per 128 channels before the
    down projection: the hand-derived codes of the fixture, exactly.  Skipping
    that step gives the unquantised column; quantising along the token axis
    (one scale per channel) would reproduce h exactly; a single 256-wide block
    would give token 0's second block the first block's scale 7."""
    cfg, inp, exp, unq = _fp8_expert_fixture()
    _, x_e = oracle.layer_inputs(cfg, inp)
    a = np.zeros((cfg.T, cfg.H))
    a[0, 0] = a[1, 1] = 448.0
    np.testing.assert_array_equal(x_e, a)
    W = oracle.Weights(cfg, inp)
    y = oracle.expert_forward(cfg, a, *W.expert(0))
    np.testing.assert_array_equal(y, exp)
    assert np.any(y != unq)
    np.testing.assert_array_equal(oracle.expert_forward(cfg, a, *W.expert(cfg.E)), exp)


def test_fp8_sorted_rows_and_layer_golden_by_hand():
    """sorted_expert_rows' FP8 branch and the whole layer on the same fixture:
    E = k = 1, so every routing weight is 1 and out = y_shared + y_routed."""
    cfg, inp, exp, _ = _fp8_expert_fixture()
    res = oracle.layer_forward(cfg, inp)
    np.testing.assert_array_equal(res.routing.idx, np.zeros((cfg.T, 1), np.int32))
    np.testing.assert_array_equal(res.routing.w, np.ones((cfg.T, 1)))
    np.testing.assert_array_equal(res.out, 2.0 * exp)
    d = oracle.dispatch(res.routing.idx, cfg.E)
    _, y_s, _, y_sh = oracle.sorted_expert_rows(cfg, inp, res.routing, d)
    np.testing.assert_array_equal(y_s[d.inv], exp)
    np.testing.assert_array_equal(y_sh[0], exp)
