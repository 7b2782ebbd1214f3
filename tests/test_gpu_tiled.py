"""Tiled expert weight storage (MOE_LAYOUT_TILED, moe_pack_expert_weights).

The pack is a byte permutation: checked bit for bit against a numpy
statement of the layout the header defines.  The layer with packed weights
runs the same kernels in the same arithmetic order as with row-major ones,
only the weight addresses differ, so its output must equal the row-major
output bit for bit; it is also checked against the fp64 oracle with the
usual bars (max|Δ| <= 1e-4 / 2e-2 / 6e-2 x rms for fp32 / bf16 / fp8).
The cases cover every GEMM kernel that reads expert weights: the
weight-streaming decode kernel (16- and 32-row tiles), the generic kernel
(bf16, fp8, fp32), the large-tile kernel (bf16, fp8) and the single-launch
layer."""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import config, generate
from _gpu_helpers import check_layer_output, layer_routing, log, out_to_f64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import sparse_moe_expert_amd as moe
    from sparse_moe_expert_amd.device import DeviceLayer, pack_expert_weights


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def tiled_bytes(a: np.ndarray) -> np.ndarray:
    """[n, rows, cols] row-major -> the bytes of the tiled order: 16-row x
    64-byte tiles, row group major, then along the row; inside a tile the
    16-byte chunks chunk-major (chunk c of tile row r at 256 c + 16 r)."""
    n, rows = a.shape[:2]
    b = np.ascontiguousarray(a).view(np.uint8).reshape(n, rows, -1)
    rb = b.shape[2]
    # axes: matrix, row group, tile row, tile column, chunk, byte
    t = b.reshape(n, rows // 16, 16, rb // 64, 4, 16).transpose(0, 1, 3, 4, 2, 5)
    return np.ascontiguousarray(t).reshape(-1)


@pytest.mark.parametrize("kind,shape", [("bf16", (3, 48, 384)), ("fp8", (2, 32, 512)),
                                        ("f32", (1, 16, 64)), ("bf16", (257, 32, 256)),
                                        ("fp8", (3, 16, 64)), ("bf16", (2, 32, 96)),
                                        # > 2^24 chunks: the kernel's grid-stride loop wraps
                                        ("bf16", (40, 3072, 1280))])
def test_pack_is_the_stated_permutation(kind, shape):
    rng = np.random.default_rng(7)
    esz = {"bf16": 2, "fp8": 1, "f32": 4}[kind]
    raw = rng.integers(0, 256, size=int(np.prod(shape)) * esz, dtype=np.uint8)
    src = torch.from_numpy(raw).cuda()
    dst = torch.full_like(src, 0xAB)
    log(f"pack {kind} {shape}")
    moe.moe_pack_expert_weights(src, dst, shape[0], shape[1], shape[2], kind)
    torch.cuda.synchronize()
    a = raw.reshape(shape[0], shape[1], shape[2] * esz)
    np.testing.assert_array_equal(dst.cpu().numpy(), tiled_bytes(a))


def small(**kw):
    base = dict(name="tiled", cfg_id=93, T=64, H=512, E=64, S=1, k=4, I=256, Is=256,
                act="bf16", expert="bf16")
    base.update(kw)
    if base["expert"] == "f32":
        base["act"] = "f32"
    base["Is"] = base["I"]
    return config(0).with_(**base)


# (case, kernel it exercises): mean rows per expert T*k/E picks the kernel
TILED_CASES = {
    "decode16": lambda: small(T=64, E=64, k=4),                     # 4 rows/expert
    "decode32": lambda: small(T=128, E=64, k=8, S=2),               # 16
    "generic_bf16": lambda: small(T=256, E=32, k=8),                # 64
    "big_bf16": lambda: small(T=600, E=32, k=8, I=384),             # 150
    "generic_fp8": lambda: small(T=200, E=16, k=4, I=1536, expert="fp8"),
    "big_fp8": lambda: small(T=700, E=16, S=2, k=4, I=1536, expert="fp8"),
    "generic_f32": lambda: small(T=45, H=384, E=12, k=3, I=256, expert="f32"),
    "S0": lambda: small(T=50, S=0),
}


def both_layouts(cfg, inp):
    rows = DeviceLayer(cfg, inp)
    tiled = DeviceLayer(cfg, inp, tiled=True)
    return rows, tiled


@pytest.mark.parametrize("case", list(TILED_CASES))
def test_layer_tiled_equals_row_major(case):
    cfg = TILED_CASES[case]()
    log(f"tiled layer {case}: {cfg}")
    inp = generate(cfg)
    rows, tiled = both_layouts(cfg, inp)
    a = rows.forward()
    b = tiled.forward()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{case}: layouts differ"
    idx, w = layer_routing(moe, tiled)
    check_layer_output(cfg, inp, out_to_f64(b), idx, f"tiled layer {case}", w_gpu=w)


@pytest.mark.parametrize("case", ["decode16", "S0"])
def test_fused_tiled_equals_row_major(case):
    cfg = TILED_CASES[case]()
    log(f"tiled fused {case}: {cfg}")
    rows, tiled = both_layouts(cfg, generate(cfg))
    outs = []
    for lay in (rows, tiled):
        out = lay.empty_out()
        moe.moe_layer_forward_fused(lay.ccfg, lay.weights, lay.t["x"], out,
                                    workspace=lay.workspace)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.uint8), outs[1].view(torch.uint8))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_full_size_tiled_equals_row_major(cid):
    """The full-size workloads, in the launch configuration the benchmark
    times: the tiled layer equals the row-major one bit for bit (the
    row-major layer is checked against the oracle in test_gpu_parity)."""
    cfg = config(cid)
    log(f"tiled full C{cid}: generating inputs")
    lay = DeviceLayer(cfg, generate(cfg))
    a = lay.forward()
    ek = cfg.expert
    packed = {key: pack_expert_weights(lay.t[key], ek)
              for key in ("w_gate_up", "w_down", "w_sh_gate_up", "w_sh_down")}
    ct = moe.make_config(cfg.T, cfg.H, cfg.E, cfg.S, cfg.k, cfg.I, cfg.Is, act=cfg.act,
                         expert=ek, norm_topk_prob=cfg.norm_topk_prob,
                         routed_scaling_factor=cfg.routed_scaling_factor, n_group=cfg.n_group,
                         topk_group=cfg.topk_group, tiled=True)
    t = lay.t
    wt = moe.make_weights(w_router=t["w_router"], router_bias=t["bias"],
                          w_gate_up=packed["w_gate_up"], w_down=packed["w_down"],
                          s_gate_up=t.get("s_gate_up"), s_down=t.get("s_down"),
                          w_sh_gate_up=packed["w_sh_gate_up"], w_sh_down=packed["w_sh_down"],
                          s_sh_gate_up=t.get("s_sh_gate_up"), s_sh_down=t.get("s_sh_down"))
    b = lay.empty_out()
    log(f"tiled full C{cid}: forward")
    moe.moe_layer_forward(ct, wt, t["x"], b, workspace=lay.workspace)
    torch.cuda.synchronize()
    same = torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    if not same:
        d = (a.float() - b.float()).abs()
        log(f"tiled full C{cid}: max |diff| {d.max().item():.3e}")
    assert same
    if ek == "bf16":
        # the benchmark's weights: tiled plus the fp16 copies of the down weights
        f16 = {key: torch.empty(packed[key].shape, dtype=torch.float16, device="cuda")
               for key in ("w_down", "w_sh_down")}
        for key in f16:
            moe.moe_convert_bf16_to_f16(packed[key], f16[key], packed[key].numel())
        w16 = moe.make_weights(w_router=t["w_router"], router_bias=t["bias"],
                               w_gate_up=packed["w_gate_up"], w_down=packed["w_down"],
                               w_sh_gate_up=packed["w_sh_gate_up"], w_sh_down=packed["w_sh_down"],
                               w_down_f16=f16["w_down"], w_sh_down_f16=f16["w_sh_down"])
        c = lay.empty_out()
        log(f"tiled full C{cid}: forward with fp16 down copies")
        moe.moe_layer_forward(ct, w16, t["x"], c, workspace=lay.workspace)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.uint8), c.view(torch.uint8))


def bf16_to_f16_rtz(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp16 bit patterns of the value rounded toward
    zero, from the IEEE definition on the exact (fp64) value: exact on
    fp16's normal range, the subnormal grid 2^-24 truncated below 2^-14,
    +-65504 beyond the largest finite fp16, inf and NaN kept."""
    with np.errstate(invalid="ignore"):  # NaN patterns
        v = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    a = np.abs(v)
    q = np.where(a < 2.0 ** -14, np.trunc(v * 2.0 ** 24) * 2.0 ** -24, v)
    q = np.where(np.isfinite(v) & (a > 65504.0), np.sign(v) * 65504.0, q)
    return q.astype(np.float16).view(np.uint16)


def test_convert_bf16_to_f16_every_pattern():
    """All 65536 bf16 patterns (normal, subnormal, zero, beyond fp16's range,
    inf, NaN) against the rounding-toward-zero definition."""
    bits = np.tile(np.arange(65536, dtype=np.uint16), 2)
    src = torch.from_numpy(bits.view(np.int16)).cuda()
    dst = torch.full_like(src, 0x5555)
    moe.moe_convert_bf16_to_f16(src, dst, bits.size)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint16)
    ref = bf16_to_f16_rtz(bits)
    nan = np.isnan(ref.view(np.float16))
    assert np.isnan(got.view(np.float16)[nan]).all()
    np.testing.assert_array_equal(got[~nan], ref[~nan])


# the optional fp16 down copies: read only on the large-tile path, where
# they replace the in-register conversion of the same bf16 values, so the
# layer's output is the same bit for bit (and is ignored elsewhere)
F16_CASES = {
    "big_bf16": lambda: small(T=600, E=32, k=8, I=384),             # 150 rows/expert
    "big_bf16_S2": lambda: small(T=640, H=768, E=16, S=2, k=4, I=512),  # 160
    "big_bf16_S0": lambda: small(T=600, E=32, k=8, I=384, S=0),
    "decode16": lambda: small(T=64, E=64, k=4),                     # ignored here
}


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("case", list(F16_CASES))
def test_layer_down_f16_copy_equals_bf16(case, tiled):
    cfg = F16_CASES[case]()
    log(f"down f16 copy {case} tiled={tiled}: {cfg}")
    inp = generate(cfg)
    a = DeviceLayer(cfg, inp, tiled=tiled).forward()
    lay = DeviceLayer(cfg, inp, tiled=tiled, down_f16=True)
    b = lay.forward()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{case}: fp16 copy changed the output"
    idx, w = layer_routing(moe, lay)
    check_layer_output(cfg, inp, out_to_f64(b), idx, f"down f16 copy {case}", w_gpu=w)
