"""GPU parity of the single-launch layer (moe_layer_forward_fused: one
cooperative grid for route -> dispatch -> gate/up + SwiGLU -> down ->
combine, the chain of the FUSED_MC2 figure, Deep Dive §8.2) against the fp64
oracle, and against the multi-launch path, in the decode regime it serves.

Bars as for the layer: routing indices bit-exact on every token away from a
1e-6 near-tie, dispatch counts bit-exact, outputs within max|Δ| <= 2e-2 x
rms(oracle) (bf16)."""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import config, generate
from _gpu_helpers import (assert_close, check_layer_output, layer_routing, log, out_to_f64,
                          untied)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import sparse_moe_expert_amd as moe
    from sparse_moe_expert_amd.device import DeviceLayer


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def small(**kw):
    base = dict(name="small", cfg_id=92, T=64, H=512, E=32, S=1, k=4, I=256, Is=256,
                act="bf16", expert="bf16")
    base.update(kw)
    base["Is"] = base["I"]
    return config(0).with_(**base)


def fused(lay):
    out = lay.empty_out()
    counts = torch.empty(lay.cfg.E, dtype=torch.int32, device="cuda")
    ties = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    moe.moe_layer_forward_fused(lay.ccfg, lay.weights, lay.t["x"], out, counts, ties, lay.workspace)
    torch.cuda.synchronize()
    return out, counts, ties


FUSED_CASES = {
    "small": lambda: small(),
    "S2_k6": lambda: small(T=80, E=48, S=2, k=6, H=384, I=128),
    "T1": lambda: small(T=1, E=64, k=8),
    "ragged_T37": lambda: small(T=37, E=32, k=8),
    "grouped": lambda: small(T=96, E=64, k=6, n_group=8, topk_group=3),
    "S0": lambda: small(T=50, S=0),
}


@pytest.mark.parametrize("case", list(FUSED_CASES))
def test_fused_matches_oracle(case):
    cfg = FUSED_CASES[case]()
    log(f"fused {case}: {cfg}")
    inp = generate(cfg)
    lay = DeviceLayer(cfg, inp)
    out, counts, ties = fused(lay)
    idx, w = layer_routing(moe, lay)
    check_layer_output(cfg, inp, out_to_f64(out), idx, f"fused {case}", w_gpu=w)
    np.testing.assert_array_equal(counts.cpu().numpy(), np.bincount(idx.ravel(), minlength=cfg.E))
    assert int(counts.sum()) == cfg.T * cfg.k
    t = ties.cpu().numpy()
    assert t.min() >= 0 and t.max() <= cfg.T


@pytest.mark.timeout(900)
def test_fused_full_size_c1_matches_oracle_and_layer():
    cfg = config(1)
    log("fused full C1: generating inputs")
    inp = generate(cfg)
    lay = DeviceLayer(cfg, inp)
    out, counts, _ = fused(lay)
    idx_f, w_f = layer_routing(moe, lay)
    check_layer_output(cfg, inp, out_to_f64(out), idx_f, "fused full C1", w_gpu=w_f)
    np.testing.assert_array_equal(counts.cpu().numpy(), np.bincount(idx_f.ravel(), minlength=cfg.E))
    # against the multi-launch path: where both made the same choice of
    # experts (they sum the router logits in different orders, so a near-tie
    # may go either way), outputs within the same bar
    ref = lay.forward()
    torch.cuda.synchronize()
    idx_l, _ = layer_routing(moe, lay)
    same = np.all(idx_f == idx_l, axis=1)
    log(f"fused full C1: {(~same).sum()} tokens chose differently from the multi-launch layer")
    assert (~same).sum() <= 4
    assert_close(cfg, out_to_f64(out), out_to_f64(ref), "fused vs layer C1", mask=same)


def test_fused_rejects_other_regimes():
    for cfg in (small(T=2048, E=32, k=8),             # 512 rows per expert: large tiles
                small(act="f32", expert="f32"),       # fp32
                small(E=24, k=2)):                   # E not a multiple of 16
        lay = DeviceLayer(cfg, generate(cfg))
        out = torch.full((cfg.T, cfg.H), 7, dtype=lay.act_dtype, device="cuda")
        with pytest.raises(moe.MoEError) as e:
            moe.moe_layer_forward_fused(lay.ccfg, lay.weights, lay.t["x"], out, None, None,
                                        lay.workspace)
        assert e.value.status == moe.MOE_ERR_UNSUPPORTED
        torch.cuda.synchronize()
        assert torch.all(out == 7)


def test_fused_is_deterministic():
    cfg = small(T=128, E=128, k=8, H=1024, I=512)
    lay = DeviceLayer(cfg, generate(cfg))
    a, _, _ = fused(lay)
    b, _, _ = fused(lay)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def barrier_words(lay):
    off = moe.moe_workspace_offset(lay.ccfg, moe.MOE_WS_BARRIER)
    return lay.workspace[off:off + 8].view(torch.int32).cpu().numpy()


def test_fused_barrier_status_and_timeout():
    """The grid barrier's bounded wait: after a completed launch the status
    word is 0 and the arrival counter holds one arrival per block and barrier
    (5 barriers); with a spin limit of 0 every block that finds blocks missing
    gives up at its first poll and sets the status, and every other block
    stops at its next barrier, so the launch still ends.  The next launch with
    the default limit completes and gives the same output as before."""
    cfg = small(T=64, E=64, k=8)
    lay = DeviceLayer(cfg, generate(cfg))
    ref, _, _ = fused(lay)
    words = barrier_words(lay)
    log(f"fused barrier words after a completed launch: {words.tolist()}")
    assert words[1] == 0 and words[0] > 0 and words[0] % 5 == 0
    prev = moe.moe_fused_set_spin_limit(0)
    try:
        log("fused launch with spin limit 0")
        fused(lay)
    finally:
        moe.moe_fused_set_spin_limit(prev)
    words = barrier_words(lay)
    log(f"fused barrier words after the launch with spin limit 0: {words.tolist()}")
    assert words[1] == 1
    assert moe.moe_fused_set_spin_limit(-1) == prev  # the default restored
    again, _, _ = fused(lay)
    assert barrier_words(lay)[1] == 0
    assert torch.equal(again.view(torch.int16), ref.view(torch.int16))
