"""moe_layer_forward_noalloc: the layer without a caller workspace (its scratch
is a device array inside the library), called through the C ABI.  Its output
must equal moe_layer_forward's bit for bit (same kernels, same arithmetic
order) and meet the oracle's bar; two calls in a row, the second smaller,
check that nothing carries over in the shared array; a configuration whose
workspace exceeds the array is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

from moe_inputs import config, generate
from _gpu_helpers import check_layer_output, layer_routing, log, out_to_f64

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
    base = dict(name="noalloc", cfg_id=94, T=200, H=1024, E=64, S=1, k=8, I=512, Is=512,
                act="bf16", expert="bf16")
    base.update(kw)
    base["Is"] = base["I"]
    return config(0).with_(**base)


def _compare(cfg, tiled=False):
    inp = generate(cfg)
    lay = DeviceLayer(cfg, inp, tiled=tiled)
    log(f"noalloc {cfg.T}x{cfg.H} E={cfg.E} k={cfg.k} I={cfg.I} {cfg.expert}: "
        f"workspace {lay.ws_bytes} bytes")
    assert lay.ws_bytes <= moe.NOALLOC_SCRATCH_BYTES
    ref_counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    ref = lay.forward(counts=ref_counts)
    idx, w = layer_routing(moe, lay)
    out = torch.full_like(ref, 7)
    counts = torch.full_like(ref_counts, -1)
    ties = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    moe.moe_layer_forward_noalloc(lay.ccfg, lay.weights, lay.t["x"], out, counts, ties)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), ref.view(torch.uint8))
    assert torch.equal(counts, ref_counts)
    assert int(ties.min()) >= 0
    check_layer_output(cfg, inp, out_to_f64(out), idx, f"noalloc T={cfg.T}", w_gpu=w)


def test_noalloc_two_calls_second_smaller():
    """Weight-streaming regime (8 rows per expert), then a smaller batch of
    the same layer shape through the same scratch array."""
    _compare(small(T=256))
    _compare(small(T=37, cfg_id=95))


def test_noalloc_other_paths():
    """The mid-size kernel (64 rows per expert), fp8 experts, fp32, tiled weights."""
    _compare(small(T=256, E=32))
    _compare(small(T=128, E=16, k=4, I=1536, expert="fp8"))
    _compare(config(0))
    _compare(small(T=64, E=64, k=4), tiled=True)


def test_noalloc_rejects_oversized_workspace():
    cfg = small(T=64)
    lay = DeviceLayer(cfg, generate(cfg))
    big = moe.make_config(4096, 5120, 256, 1, 8, 1536)    # ~1 GB of workspace
    assert moe.moe_workspace_size(big) > moe.NOALLOC_SCRATCH_BYTES
    out = torch.full((8, 8), 3.0, device="cuda")
    with pytest.raises(moe.MoEError) as e:
        moe.moe_layer_forward_noalloc(big, lay.weights, lay.t["x"], out)
    assert e.value.status == moe.MOE_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
    # T = 0 is a no-op
    moe.moe_layer_forward_noalloc(moe.make_config(0, 1024, 64, 1, 8, 512), lay.weights,
                                  lay.t["x"], out)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
