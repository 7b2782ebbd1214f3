"""Pins for the oracle's decoder block around the MoE layer (single-layer
figure of 'Xiaohongshu dots3 note Open Source Deep Dive', §3.3: "Residual +
RMSNorm", MoE FFN, "Residual + Output"; RMSNorm as the Transformers dots.llm1
article describes it: fp32 variance, rsqrt, times the weight, eps 1e-6):
torch's own rms_norm and bf16 cast, closed forms, and special cases of the
whole block."""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import config, generate


def test_rmsnorm_matches_torch_rms_norm():
    rng = np.random.default_rng(3)
    h = rng.standard_normal((37, 256)) * rng.uniform(0.1, 10, (37, 1))
    gamma = rng.uniform(0.5, 1.5, 256)
    for eps in (1e-6, 1e-2):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(h), (256,), torch.from_numpy(gamma),
                                           eps=eps).numpy()
        np.testing.assert_allclose(oracle.rmsnorm(h, gamma, eps), ref, rtol=1e-13, atol=0)


def test_rmsnorm_closed_forms():
    # constant row c: gamma * c / sqrt(c^2 + eps)
    c, eps = -3.0, 1e-6
    out = oracle.rmsnorm(np.full((1, 4), c), np.array([1.0, 2.0, 0.5, 0.0]), eps)
    np.testing.assert_allclose(out[0], np.array([1.0, 2.0, 0.5, 0.0]) * c / np.sqrt(c * c + eps),
                               rtol=1e-15)
    # (3, 4): mean square 12.5
    out = oracle.rmsnorm(np.array([[3.0, 4.0]]), np.ones(2), 0.0)
    np.testing.assert_allclose(out[0], [3 / np.sqrt(12.5), 4 / np.sqrt(12.5)], rtol=1e-15)
    # eps = 0, unit gamma: scale invariant and unit mean square
    rng = np.random.default_rng(1)
    h = rng.standard_normal((5, 64))
    a = oracle.rmsnorm(h, np.ones(64), 0.0)
    np.testing.assert_allclose(a, oracle.rmsnorm(7.5 * h, np.ones(64), 0.0), rtol=1e-14)
    np.testing.assert_allclose(np.mean(a * a, axis=1), 1.0, rtol=1e-14)


def test_encode_bf16_is_round_to_nearest_even():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000),
                        [0.0, -0.0, 1.0, -1.0, 3.0e38]])
    ours = oracle.encode_bf16(v)
    np.testing.assert_array_equal(oracle.decode_bf16(ours), oracle.decode_bf16(ours))
    # torch casts fp64 -> fp32 -> bf16; the two agree except where the fp32
    # rounding lands exactly on a bf16 midpoint, where ours rounds the exact
    # value instead of the tie
    t = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    diff = np.nonzero(t != ours)[0]
    f32_bits = v.astype(np.float32).view(np.uint32)
    assert np.all((f32_bits[diff] & 0xFFFF) == 0x8000)
    for i in diff:          # ours is the nearer neighbour of the exact value
        a = abs(oracle.decode_bf16(np.array([ours[i]]))[0] - v[i])
        b = abs(oracle.decode_bf16(np.array([t[i]]))[0] - v[i])
        assert a < b
    # exact halfway cases go to the even neighbour
    one_plus_half_ulp = 1.0 + 2.0 ** -8
    assert oracle.encode_bf16(np.array([one_plus_half_ulp]))[0] == 0x3F80
    assert oracle.encode_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82


def _tiny(**kw):
    cfg = config(0, T=12, **kw)
    return cfg, generate(cfg)


def test_block_with_zero_experts_is_identity():
    cfg, inp = _tiny()
    inp = dict(inp)
    for key in list(inp):
        if key.startswith(("w_gate_up", "w_down", "w_sh")):
            inp[key] = np.zeros_like(inp[key])
    gamma = np.linspace(0.5, 1.5, cfg.H)
    out, _ = oracle.block_forward(cfg, inp, gamma)
    np.testing.assert_array_equal(out, oracle.widen(inp["x"], cfg.act))


def test_block_with_zero_gamma_routes_by_bias_and_adds_nothing():
    cfg, inp = _tiny()
    out, res = oracle.block_forward(cfg, inp, np.zeros(cfg.H))
    np.testing.assert_array_equal(out, oracle.widen(inp["x"], cfg.act))
    # logits 0 -> every score is 1/2 and the bias alone orders the experts
    order = np.argsort(-np.asarray(inp["bias"], float), kind="stable")[:cfg.k]
    assert np.all(res.routing.idx == order[None, :])
    np.testing.assert_allclose(res.routing.w, 1.0 / cfg.k, rtol=1e-15)


def test_block_residual_and_layer_input():
    cfg, inp = _tiny()
    gamma = np.linspace(0.5, 1.5, cfg.H)
    out, res = oracle.block_forward(cfg, inp, gamma, tokens=np.arange(3, 9))
    h = oracle.widen(inp["x"], cfg.act)[3:9]
    # layer input: the normalised rows in the activation type (fp32 here)
    xn = torch.nn.functional.rms_norm(torch.from_numpy(h), (cfg.H,), torch.from_numpy(gamma),
                                      eps=cfg.rms_norm_eps).numpy().astype(np.float32)
    sub = dict(inp)
    sub["x"] = np.zeros_like(inp["x"])
    sub["x"][3:9] = xn
    ref = oracle.layer_forward(cfg, sub, np.arange(3, 9))
    np.testing.assert_allclose(out - h, ref.out, rtol=0, atol=1e-12)
