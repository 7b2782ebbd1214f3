"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, the ctypes structs match the C layout, and host-side
validation rejects bad calls before anything reaches the device."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

moe = pytest.importorskip("sparse_moe_expert_amd._lib",
                          reason="libmoe.so not built (python -m sparse_moe_expert_amd.build)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text))


def test_exports_match_header():
    declared = declared_functions()
    assert declared == set(moe.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (moe_[a-z0-9_]+)$", out, flags=re.M))
    assert declared <= exported, declared - exported
    for name in declared:
        assert getattr(moe.LIB, name) is not None


def test_package_reexports_every_wrapper():
    """Every C entry point with a Python wrapper in the binding is reachable
    from the package itself."""
    import sparse_moe_expert_amd as pkg
    for name in moe.EXPORTS:
        if hasattr(moe, name):
            assert name in pkg.__all__, name
            assert getattr(pkg, name) is getattr(moe, name)


def test_struct_layout_matches_c():
    src = r"""
#include <stdio.h>
#include <stddef.h>
#include "moe.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(moe_config_t), offsetof(moe_config_t, routed_scaling_factor),
         offsetof(moe_config_t, expert_dtype), offsetof(moe_config_t, expert_layout),
         sizeof(moe_weights_t), offsetof(moe_weights_t, s_gate_up), offsetof(moe_weights_t, s_sh_down),
         offsetof(moe_weights_t, w_sh_down_f16));
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "probe.c")
        exe = os.path.join(d, "probe")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        vals = list(map(int, subprocess.run([exe], capture_output=True, text=True,
                                            check=True).stdout.split()))
    C, W = moe.moe_config_t, moe.moe_weights_t
    assert vals == [ctypes.sizeof(C), C.routed_scaling_factor.offset, C.expert_dtype.offset,
                    C.expert_layout.offset, ctypes.sizeof(W), W.s_gate_up.offset,
                    W.s_sh_down.offset, W.w_sh_down_f16.offset]


def test_status_strings_and_version():
    for code in (0, -1, -2, -3, -4):
        assert moe.status_string(code).startswith("MOE_")
    assert "unknown" in moe.status_string(7)
    assert moe.version().startswith("moe-gfx950")


def cfg(**kw):
    base = dict(T=64, H=512, E=32, S=1, k=4, I=128, act="f32", expert="f32")
    base.update(kw)
    return moe.make_config(**base)


@pytest.mark.parametrize("kw,ok", [
    (dict(), True),
    (dict(act="bf16", expert="bf16"), True),
    (dict(act="bf16", expert="fp8", I=512), True),
    # FP8 needs I >= 512 (re-quantised h: one boundary code is too large a share of y below)
    (dict(act="bf16", expert="fp8"), False), (dict(act="bf16", expert="fp8", I=384), False),
    (dict(T=0), True),
    (dict(E=0), False), (dict(k=0), False), (dict(k=33), False), (dict(E=513, k=4), False),
    (dict(k=17, E=64), False), (dict(H=500), False), (dict(I=100), False), (dict(S=5), False),
    (dict(I_shared=256), False), (dict(act="f32", expert="bf16"), False),
    (dict(act="bf16", expert="f32"), False), (dict(T=-1), False),
    # tiled expert weights need whole 64-byte tile columns along H and I (always
    # so with multiples of 128 elements)
    (dict(tiled=True), True), (dict(act="bf16", expert="bf16", tiled=True), True),
    (dict(act="bf16", expert="fp8", I=640, tiled=True), True),
    (dict(act="bf16", expert="fp8", I=512, tiled=True), True),
    (dict(act="bf16", expert="fp8", H=640, I=512, tiled=True), True),
    # bf16 experts: at most 16384 intermediate channels (64 blocks of scaled h)
    (dict(act="bf16", expert="bf16", I=16384, T=4), True),
    (dict(act="bf16", expert="bf16", I=16512, T=4), False),
])
def test_workspace_size_validates(kw, ok):
    n = moe.moe_workspace_size(cfg(**kw))
    assert (n > 0) == ok


def test_workspace_size_covers_buffers():
    c = moe.make_config(T=16384, H=5120, E=256, S=1, k=8, I=1536)
    n = moe.moe_workspace_size(c)
    R = 16384 * 8
    # h (fp16 codes) and its block exponents (6 per row) + y_sorted and
    # y_shared (fp16 codes) and their exponents (20 per row) + router logits
    # (fp32, K split 2 ways at this T) + the normalised block input (bf16)
    need = ((R + 16384) * 1536 * 2 + (R + 16384) * 6 * 4 + R * 5120 * 2 + 16384 * 5120 * 2
            + (R + 16384) * 20 * 4 + 2 * 16384 * 256 * 4 + 16384 * 5120 * 2)
    assert need <= n < need * 1.05


FAKE = 1 << 20   # an aligned, never-dereferenced address: every call below fails validation


def weights(**kw):
    base = dict(w_router=FAKE, router_bias=FAKE, w_gate_up=FAKE, w_down=FAKE,
                w_sh_gate_up=FAKE, w_sh_down=FAKE)
    base.update(kw)
    return moe.make_weights(**base)


def call(name, *args):
    return getattr(moe.LIB, name)(*args)


def test_validation_rejects_before_launch():
    c = cfg()
    w = weights()
    by = ctypes.byref
    n = moe.moe_workspace_size(c)
    # null config / weights
    assert call("moe_route", None, FAKE, by(w), FAKE, FAKE, None, FAKE, n, None) == moe.MOE_ERR_INVALID_ARG
    assert call("moe_layer_forward", by(c), None, FAKE, FAKE, None, None, FAKE, n, None) == moe.MOE_ERR_INVALID_ARG
    # null / misaligned tensors
    assert call("moe_route", by(c), None, by(w), FAKE, FAKE, None, FAKE, n, None) == moe.MOE_ERR_INVALID_ARG
    assert call("moe_route", by(c), FAKE + 4, by(w), FAKE, FAKE, None, FAKE, n, None) == moe.MOE_ERR_INVALID_ARG
    assert call("moe_layer_forward", by(c), by(weights(w_down=None)), FAKE, FAKE, None, None,
                FAKE, n, None) == moe.MOE_ERR_INVALID_ARG
    # workspace missing, misaligned or too small
    assert call("moe_layer_forward", by(c), by(w), FAKE, FAKE, None, None, None, n, None) == moe.MOE_ERR_WORKSPACE
    assert call("moe_layer_forward", by(c), by(w), FAKE, FAKE, None, None, FAKE + 16, n, None) == moe.MOE_ERR_WORKSPACE
    assert call("moe_layer_forward", by(c), by(w), FAKE, FAKE, None, None, FAKE, n - 1, None) == moe.MOE_ERR_WORKSPACE
    assert call("moe_grouped_ffn", by(c), FAKE, by(w), FAKE, FAKE, FAKE, FAKE, FAKE, n - 256, None) == moe.MOE_ERR_WORKSPACE
    # unsupported shapes
    bad = cfg(H=640 + 64)
    assert call("moe_layer_forward", by(bad), by(w), FAKE, FAKE, None, None, FAKE, n, None) == moe.MOE_ERR_UNSUPPORTED
    # fp8 needs its block scales
    c8 = cfg(act="bf16", expert="fp8", I=512)
    n8 = moe.moe_workspace_size(c8)
    assert call("moe_layer_forward", by(c8), by(w), FAKE, FAKE, None, None, FAKE, n8, None) == moe.MOE_ERR_INVALID_ARG
    # fp8 below I = 512 is refused before anything is checked or enqueued
    c8s = cfg(act="bf16", expert="fp8", I=256)
    w8 = weights(s_gate_up=FAKE, s_down=FAKE, s_sh_gate_up=FAKE, s_sh_down=FAKE)
    for name in ("moe_layer_forward", "moe_layer_forward_fused"):
        assert call(name, by(c8s), by(w8), FAKE, FAKE, None, None, FAKE, n8, None) == moe.MOE_ERR_UNSUPPORTED
    # optional fp16 down copies: bf16 experts only, shared copy required with
    # S > 0, never the shared copy alone, 16-byte aligned
    cb = cfg(act="bf16", expert="bf16")
    both = dict(w_down_f16=FAKE, w_sh_down_f16=FAKE)
    scales = dict(s_gate_up=FAKE, s_down=FAKE, s_sh_gate_up=FAKE, s_sh_down=FAKE)
    for bad_w, bad_c in ((weights(**scales, **both), c8),
                         (weights(**both), c), (weights(w_sh_down_f16=FAKE), cb),
                         (weights(w_down_f16=FAKE), cb), (weights(w_down_f16=FAKE + 8, w_sh_down_f16=FAKE), cb),
                         (weights(w_down_f16=FAKE, w_sh_down_f16=FAKE + 8), cb)):
        nb = moe.moe_workspace_size(bad_c)
        assert call("moe_layer_forward", by(bad_c), by(bad_w), FAKE, FAKE, None, None, FAKE, nb,
                    None) == moe.MOE_ERR_INVALID_ARG
    # fp16 conversion of bf16 weights: n a multiple of 8, aligned, no overlap
    cv = "moe_convert_bf16_to_f16"
    assert call(cv, FAKE, FAKE + 4096, 0, None) == moe.MOE_OK
    for args in ((FAKE, FAKE + 4096, 12), (FAKE, FAKE + 4096, -8), (None, FAKE, 8), (FAKE, None, 8),
                 (FAKE + 2, FAKE + 4096, 8), (FAKE, FAKE + 4096 + 8, 8), (FAKE, FAKE + 8, 16)):
        assert call(cv, *args, None) == moe.MOE_ERR_INVALID_ARG, args
    # combine / dispatch / quantiser argument checks
    assert call("moe_combine", by(c), FAKE, None, FAKE, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert call("moe_dispatch", by(c), FAKE, None, FAKE, FAKE, FAKE, FAKE, n, None) == moe.MOE_ERR_INVALID_ARG
    assert call("moe_quantize_fp8", FAKE, 4, 100, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert call("moe_quantize_fp8", FAKE + 8, 4, 128, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    # decoder block: eps, gamma, aliasing
    f = ctypes.c_float
    assert call("moe_rmsnorm", by(c), FAKE, FAKE, f(-1.0), FAKE + 4096, None) == moe.MOE_ERR_INVALID_ARG
    assert call("moe_rmsnorm", by(c), FAKE, FAKE, f(float("inf")), FAKE + 4096, None) == moe.MOE_ERR_INVALID_ARG
    assert call("moe_rmsnorm", by(c), FAKE, None, f(1e-6), FAKE + 4096, None) == moe.MOE_ERR_INVALID_ARG
    assert call("moe_rmsnorm", by(c), FAKE, FAKE, f(1e-6), FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert call("moe_rmsnorm", by(c), FAKE + 8, FAKE, f(1e-6), FAKE + 4096, None) == moe.MOE_ERR_INVALID_ARG
    assert call("moe_block_forward", by(c), by(w), FAKE, FAKE, f(float("nan")), FAKE + 4096, None,
                None, FAKE, n, None) == moe.MOE_ERR_INVALID_ARG
    assert call("moe_block_forward", by(c), by(w), FAKE, None, f(1e-6), FAKE + 4096, None, None,
                FAKE, n, None) == moe.MOE_ERR_INVALID_ARG
    assert call("moe_block_forward", by(c), by(w), FAKE, FAKE, f(1e-6), FAKE, None, None,
                FAKE, n, None) == moe.MOE_ERR_INVALID_ARG
    assert call("moe_block_forward", by(c), by(w), FAKE, FAKE, f(1e-6), FAKE + 4096, None, None,
                FAKE, n - 1, None) == moe.MOE_ERR_WORKSPACE


@pytest.mark.parametrize("n_group,topk_group,k,ok", [
    (0, 0, 4, True), (1, 1, 4, True), (8, 4, 8, True), (32, 32, 4, True), (4, 1, 8, True),
    (3, 1, 4, False), (8, 0, 4, False), (8, 9, 4, False), (8, 1, 9, False), (-1, 1, 4, False),
    (64, 4, 4, None),
])
def test_group_fields_validate(n_group, topk_group, k, ok):
    """n_group must divide E with topk_group in 1..n_group and k within the
    chosen groups; more than 64 groups is unsupported."""
    c = cfg(E=64 if n_group == 64 else 32, k=k)
    c.n_group, c.topk_group = n_group, topk_group
    n = moe.moe_workspace_size(c)
    if ok is None:
        assert n > 0
        c.E, c.n_group = 128, 128
        assert moe.moe_workspace_size(c) == 0
        return
    assert (n > 0) == ok


def test_zero_tokens_is_a_noop():
    """T = 0 returns success without touching the device (no GPU here)."""
    c = cfg(T=0)
    w = weights()
    by = ctypes.byref
    assert call("moe_layer_forward", by(c), by(w), FAKE, FAKE, None, None, None, 0, None) == moe.MOE_OK
    assert call("moe_route", by(c), None, by(w), None, None, None, None, 0, None) == moe.MOE_OK
    assert call("moe_quantize_fp8", None, 0, 128, None, None, None) == moe.MOE_OK


def test_python_binding_raises_moe_error():
    c = cfg(E=0)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_combine(c, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG


def test_bad_layout_value_rejected():
    c = cfg()
    c.expert_layout = 2
    assert moe.moe_workspace_size(c) == 0


def test_pack_validation():
    P = "moe_pack_expert_weights"
    A, B = FAKE, FAKE + (1 << 24)   # far enough apart not to overlap below
    assert call(P, A, B, 0, 16, 128, moe.MOE_BF16, None) == moe.MOE_OK    # count 0: no-op
    assert call(P, A, B, -1, 16, 128, moe.MOE_BF16, None) == moe.MOE_ERR_INVALID_ARG
    assert call(P, A, B, 1, 0, 128, moe.MOE_BF16, None) == moe.MOE_ERR_INVALID_ARG
    assert call(P, A, B, 1, 16, 0, moe.MOE_BF16, None) == moe.MOE_ERR_INVALID_ARG
    assert call(P, A, B, 1, 16, 128, 7, None) == moe.MOE_ERR_INVALID_ARG
    assert call(P, A, B, 1, 24, 128, moe.MOE_BF16, None) == moe.MOE_ERR_UNSUPPORTED  # rows % 16
    assert call(P, A, B, 1, 16, 40, moe.MOE_BF16, None) == moe.MOE_ERR_UNSUPPORTED   # 80-byte rows
    assert call(P, A, B, 1, 16, 96, moe.MOE_FP8_E4M3, None) == moe.MOE_ERR_UNSUPPORTED
    assert call(P, A, B, 0, 16, 32, moe.MOE_BF16, None) == moe.MOE_OK               # 64-byte rows
    assert call(P, None, B, 1, 16, 128, moe.MOE_BF16, None) == moe.MOE_ERR_INVALID_ARG
    assert call(P, A, None, 1, 16, 128, moe.MOE_BF16, None) == moe.MOE_ERR_INVALID_ARG
    assert call(P, A + 8, B, 1, 16, 128, moe.MOE_BF16, None) == moe.MOE_ERR_INVALID_ARG
    # overlapping source and destination (4 KB matrix, 2 KB apart)
    assert call(P, A, A + 2048, 1, 16, 128, moe.MOE_BF16, None) == moe.MOE_ERR_INVALID_ARG
    # byte count overflowing int64
    assert call(P, A, B, 1 << 62, 16, 128, moe.MOE_BF16, None) == moe.MOE_ERR_INVALID_ARG


MAX_PART = 13


def test_workspace_offsets():
    """moe_workspace_offset: every part lies inside the workspace, in the order
    of the carve-out; h's bf16 residue exists only where the down GEMM streams
    its weights, h's block exponents only on the bf16 large-tile path (T=16384),
    neither for fp8."""
    parts = [moe.MOE_WS_TOPK_IDX, moe.MOE_WS_TOPK_W, moe.MOE_WS_COUNTS, moe.MOE_WS_OFFSETS,
             moe.MOE_WS_PERM, moe.MOE_WS_INV, moe.MOE_WS_H, moe.MOE_WS_H_LO, moe.MOE_WS_Y,
             moe.MOE_WS_Y_SHARED]
    dec = moe.make_config(T=256, H=5120, E=256, S=1, k=8, I=1536)
    n = moe.moe_workspace_size(dec)
    offs = [moe.moe_workspace_offset(dec, p) for p in parts]
    assert all(o is not None and o % 256 == 0 for o in offs)
    assert offs == sorted(offs) and offs[-1] < n
    R = 256 * 8
    assert offs[parts.index(moe.MOE_WS_H_LO)] - offs[parts.index(moe.MOE_WS_H)] >= (R + 256) * 1536 * 2
    assert moe.moe_workspace_offset(dec, moe.MOE_WS_H_SCALES) is None
    big = moe.make_config(T=16384, H=5120, E=256, S=1, k=8, I=1536)
    assert moe.moe_workspace_offset(big, moe.MOE_WS_H_LO) is None
    assert moe.moe_workspace_offset(big, moe.MOE_WS_H) is not None
    assert moe.moe_workspace_offset(dec, moe.MOE_WS_H_EXP) is None
    hb, ex = (moe.moe_workspace_offset(big, p) for p in (moe.MOE_WS_H, moe.MOE_WS_H_EXP))
    assert ex is not None and ex - hb >= (16384 * 9) * 1536 * 2
    assert ex + (16384 * 9) * 6 * 4 <= moe.moe_workspace_size(big)
    f8 = moe.make_config(T=256, H=5120, E=256, S=1, k=8, I=1536, expert="fp8")
    assert moe.moe_workspace_offset(f8, moe.MOE_WS_H_LO) is None
    assert moe.moe_workspace_offset(f8, moe.MOE_WS_H_EXP) is None
    assert moe.moe_workspace_offset(f8, moe.MOE_WS_H_SCALES) is not None
    s0 = moe.make_config(T=64, H=512, E=8, S=0, k=2, I=128)
    assert moe.moe_workspace_offset(s0, moe.MOE_WS_Y_SHARED) is None
    bar = moe.moe_workspace_offset(dec, moe.MOE_WS_BARRIER)
    assert bar is not None and bar % 256 == 0 and bar + 8 <= n
    assert moe.moe_workspace_offset(dec, MAX_PART + 1) is None and moe.moe_workspace_offset(dec, -1) is None
    assert moe.moe_workspace_offset(dec, moe.MOE_WS_Y_EXP) is None
    ye = moe.moe_workspace_offset(big, moe.MOE_WS_Y_EXP)
    assert ye is not None and ye + (16384 * 9) * 20 * 4 <= moe.moe_workspace_size(big)
    assert moe.moe_workspace_offset(moe.make_config(T=1, H=100, E=8, S=1, k=2, I=128),
                                    moe.MOE_WS_H) is None


def test_stream_read_validation():
    P = "moe_stream_read"
    assert call(P, FAKE, 0, None, 1, None) == moe.MOE_OK                 # nothing to read
    assert call(P, None, 1024, FAKE, 8, None) == moe.MOE_ERR_INVALID_ARG
    assert call(P, FAKE + 8, 1024, FAKE, 8, None) == moe.MOE_ERR_INVALID_ARG
    assert call(P, FAKE, 1000, FAKE, 8, None) == moe.MOE_ERR_INVALID_ARG
    assert call(P, FAKE, 1024, None, 8, None) == moe.MOE_ERR_INVALID_ARG
    assert call(P, FAKE, 1024, FAKE, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert call(P, FAKE, 1024, FAKE, 65537, None) == moe.MOE_ERR_INVALID_ARG
