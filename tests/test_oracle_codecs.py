"""Pins for the oracle's storage formats: bf16 and OCP e4m3 decode/encode and
the per-128-channel FP8 quantiser.  Checked against torch's own casts (a
library routine), values fixed by the e4m3 definition, and a hand-derived
block (tests/golden/fp8_block_by_hand.json)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32).astype(np.uint16)
    # drop NaN patterns (exponent all ones, mantissa non-zero)
    keep = ~(((bits >> 7) & 0xFF) == 0xFF)
    bits = bits[keep]
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = oracle.decode_bf16(bits)
    np.testing.assert_array_equal(got, ref)


def test_e4m3_table_matches_torch_and_definition():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = oracle.decode_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    # values fixed by the format: bias 7, 3 mantissa bits, no infinities
    assert got[0x7E] == 448.0
    assert got[0x01] == 2.0 ** -9          # smallest subnormal
    assert got[0x08] == 2.0 ** -6          # smallest normal
    assert got[0x38] == 1.0
    assert got[0x80] == 0.0 and np.signbit(got[0x80])


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(2)
    v = np.concatenate([
        rng.uniform(-448, 448, 50000),
        rng.normal(0, 1, 50000),
        rng.normal(0, 0.01, 20000),
        rng.uniform(-2 ** -6, 2 ** -6, 20000),      # subnormal range
    ]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.encode_e4m3(v), ref)


def test_e4m3_encode_ties_to_even_and_saturates():
    vals = oracle.E4M3_TABLE[:127]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)   # exact in fp32
    codes = oracle.encode_e4m3(mids)
    lo = np.arange(126)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    np.testing.assert_array_equal(codes, expect)
    big = np.array([448.0, 449.0, 463.9, 464.0, 1e6, -1e30], dtype=np.float32)
    np.testing.assert_array_equal(oracle.encode_e4m3(big), [0x7E] * 5 + [0xFE])


def test_fp8_block_golden():
    g = json.load(open(os.path.join(GOLDEN, "fp8_block_by_hand.json")))
    row = np.zeros((1, 128), dtype=np.float32)
    row[0, :len(g["values"])] = g["values"]
    codes, scales = oracle.quantize_fp8_rows(row)
    assert scales.shape == (1, 1) and scales[0, 0] == g["expected_scale"]
    np.testing.assert_array_equal(codes[0, :len(g["expected_codes"])], g["expected_codes"])
    assert not codes[0, len(g["expected_codes"]):].any()


def test_fp8_quantiser_properties():
    rng = np.random.default_rng(3)
    v = (rng.normal(size=(64, 512)) * rng.uniform(0.01, 100, size=(64, 1))).astype(np.float32)
    v[5, 128:256] = 0.0                                    # an all-zero block
    codes, scales = oracle.quantize_fp8_rows(v)
    assert scales.dtype == np.float32 and scales.shape == (64, 4)
    assert scales[5, 1] == 1.0 and not codes[5, 128:256].any()
    blocks = np.abs(v.reshape(64, 4, 128)).max(axis=2)
    nz = blocks > 0
    # scale is amax/448 rounded once to fp32
    exact = blocks.astype(np.float64) / 448.0
    ulp = np.spacing(scales.astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(scales[nz] - exact[nz]) <= 0.5 * ulp[nz])
    # the amax element of each block maps to +-448 (code 0x7E / 0xFE)
    am = np.abs(v.reshape(64, 4, 128)).argmax(axis=2)
    top = np.take_along_axis(codes.reshape(64, 4, 128), am[:, :, None], 2)[:, :, 0]
    assert np.all((top[nz] & 0x7F) == 0x7E)
    # dequantisation error: half a mantissa step (2^-4 relative) in the
    # normal range, half a subnormal step (2^-10 * scale) below it
    deq = oracle.dequantize_fp8_rows(codes, scales)
    s = np.repeat(scales.astype(np.float64), 128, axis=1)
    err = np.abs(deq - v.astype(np.float64))
    bound = np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** -10 * s) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_fp8_weight_dequant_blocks():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 0x7E, size=(256, 384), dtype=np.uint8)
    scales = rng.uniform(0.5, 2.0, size=(2, 3)).astype(np.float32)
    w = oracle.dequantize_fp8_weight(codes, scales)
    for bn in range(2):
        for bk in range(3):
            blk = w[bn * 128:(bn + 1) * 128, bk * 128:(bk + 1) * 128]
            ref = oracle.E4M3_TABLE[codes[bn * 128:(bn + 1) * 128, bk * 128:(bk + 1) * 128]]
            np.testing.assert_array_equal(blk, ref * np.float64(scales[bn, bk]))
