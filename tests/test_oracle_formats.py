"""Pins for oracle/formats.py: the OCP format tables, torch's own casts, RNE ties,
saturation, block-scale recipes and the pages' KV bytes-per-token figure."""

import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_points(name):
    pts = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            pts.append((int(code, 16), float(val)))
    return pts


def test_e4m3fn_table_matches_spec_points():
    for code, val in _read_points("ocp_e4m3fn_points.txt"):
        got = F.E4M3FN_TABLE[code]
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), (hex(code), got, val)


def test_e4m3fn_table_matches_torch_decode():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(ref), np.isnan(F.E4M3FN_TABLE))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ref[ok], F.E4M3FN_TABLE[ok])


def test_e4m3fn_encode_matches_torch_cast_in_range():
    g = np.random.default_rng(11)
    x = np.concatenate([g.standard_normal(20000) * s for s in (1e-3, 0.1, 1, 30, 120)])
    x = np.clip(x, -448, 448).astype(np.float32)       # torch casts fp32; no overflow here
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.encode_e4m3fn(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_e4m3fn_rne_ties_and_saturation():
    # 1.0625 lies halfway between 1.0 (mantissa 000) and 1.125 (001): even -> 1.0
    # 1.1875 lies halfway between 1.125 (001) and 1.25 (010): even -> 1.25
    # 464 lies halfway between 448 (110) and 480 (not finite in e4m3fn): -> 448
    x = np.array([1.0625, 1.1875, 464.0, 1000.0, -1e6, -1e-9, 2.0 ** -10, 3 * 2.0 ** -10])
    got = F.decode_e4m3fn(F.encode_e4m3fn(x))
    # 2^-10 is halfway between 0 and 2^-9 (code 1): even -> 0;
    # 3*2^-10 is halfway between 2^-9 (code 1) and 2^-8 (code 2): even -> 2^-8
    exp = np.array([1.0, 1.25, 448.0, 448.0, -448.0, -0.0, 0.0, 2.0 ** -8])
    np.testing.assert_array_equal(got, exp)
    assert np.signbit(got[5])


def test_e2m1_table_matches_spec():
    for code, val in _read_points("ocp_mx_e2m1.txt"):
        got = F.E2M1_TABLE[code]
        assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)


def test_e2m1_rne_ties_and_saturation():
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0, -0.1, -2.9])
    exp = np.array([0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, -0.0, -3.0])
    got = F.decode_e2m1(F.encode_e2m1(x))
    np.testing.assert_array_equal(got, exp)
    assert np.signbit(got[9])


def test_e8m0_decode():
    np.testing.assert_array_equal(F.decode_e8m0(np.array([127, 128, 0, 254])),
                                  np.array([1.0, 2.0, 2.0 ** -127, 2.0 ** 127]))
    assert np.isnan(F.decode_e8m0(np.array([255]))[0])


def test_bf16_encode_matches_torch():
    g = np.random.default_rng(3)
    x = np.concatenate([g.standard_normal(50000) * s for s in (1e-30, 1e-3, 1, 1e5, 1e30)]).astype(np.float32)
    # exact ties of bf16 precision, representable in fp32
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(2 + 2.0 ** -7)], dtype=np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = F.encode_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(F.decode_bf16(got), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16)
                                  .to(torch.float64).numpy())


def test_bf16_direct_rounding_from_float64():
    # 1 + 2^-8 + 2^-40 is above the tie: direct RNE gives 1 + 2^-7 (double rounding via
    # fp32 would give 1.0).
    assert F.decode_bf16(F.encode_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -40])))[0] == 1 + 2.0 ** -7


def test_mxfp4_scale_exponent_and_roundtrip():
    blk = np.zeros((3, 32))
    blk[0, :] = np.linspace(-6, 6, 32)      # amax 6 -> E = floor(log2 6) - 2 = 0
    blk[1, :] = np.linspace(-7.9, 7.9, 32)  # amax 7.9 -> E = 0, +-7.9 saturates to +-6
    blk[2, :] = np.linspace(-0.3, 0.3, 32)  # amax 0.3 -> floor(log2 0.3) = -2 -> E = -4
    packed, sc = F.quant_mxfp4(blk)
    np.testing.assert_array_equal(sc[:, 0], np.array([127, 127, 123], dtype=np.uint8))
    deq = F.dequant_mxfp4(packed, sc)
    assert deq[1, 0] == -6.0 and deq[1, -1] == 6.0
    # away from saturation the error is at most half an e2m1 spacing times the scale
    for r in (0, 2):
        E = int(sc[r, 0]) - 127
        v = blk[r] / 2.0 ** E
        spacing = np.where(np.abs(v) < 2, 0.5, np.where(np.abs(v) < 4, 1.0, 2.0))
        assert np.all(np.abs(deq[r] - blk[r]) <= 0.5 * spacing * 2.0 ** E + 1e-15)
    z_packed, z_sc = F.quant_mxfp4(np.zeros((1, 32)))
    assert z_sc[0, 0] == 0 and np.all(z_packed == 0)


def test_mxfp4_packing_low_nibble_first():
    x = np.zeros((1, 32))
    x[0, 0], x[0, 1] = 1.0, 6.0   # with amax 6 -> E = 0: codes 0x2 and 0x7
    packed, sc = F.quant_mxfp4(x)
    assert packed[0, 0] == 0x72 and sc[0, 0] == 127


def test_kv_split_recipe_and_roundtrip():
    g = np.random.default_rng(5)
    x = g.standard_normal((64, 512))
    x[3, 10] = 20.0
    codes, scales, rope = F.quant_kv_split(x, 64)
    assert codes.shape == (64, 448) and scales.shape == (64, 4) and rope.shape == (64, 64)
    # blocks are [0,128), [128,256), [256,384), [384,448)
    assert F.kv_split_blocks(448) == [(0, 128), (128, 256), (256, 384), (384, 448)]
    np.testing.assert_array_equal(scales[:, 0], (np.abs(x[:, :128]).max(1) / 448).astype(np.float32))
    np.testing.assert_array_equal(scales[:, 3], (np.abs(x[:, 384:448]).max(1) / 448).astype(np.float32))
    deq = F.dequant_kv_split(codes, scales, rope)
    # the block maximum maps to +-448 exactly
    assert abs(abs(deq[3, 10]) - 448 * float(scales[3, 0])) == 0
    rel = np.abs(deq[:, :448] - x[:, :448]) / np.repeat(scales.astype(np.float64), [128, 128, 128, 64], axis=1)
    assert rel.max() <= 16.0 + 1e-9          # half of the largest e4m3 spacing (32) in scale units
    np.testing.assert_array_equal(deq[:, 448:], F.decode_bf16(F.encode_bf16(x[:, 448:])))
    zc, zs, _ = F.quant_kv_split(np.zeros((1, 512)), 64)
    assert np.all(zc == 0) and np.all(zs == 0)


def test_fp8_b128_recipe_matches_torch_cast():
    """The FP8 1x128 rows of the indexer: scale = fp32(amax / 448) per 128 dims, codes the
    e4m3fn rounding of x / scale -- checked against torch's own float8_e4m3fn cast of the
    scaled values (saturation at the block maximum, a ragged last block of 64 dims, a zero
    block)."""
    g = np.random.default_rng(6)
    x = g.standard_normal((50, 192)) * np.exp(g.uniform(-6, 6, (50, 1)))
    x[7, 5] = -300.0
    x[9, 128:] = 0.0
    codes, scales = F.quant_fp8_b128(x)
    assert codes.shape == (50, 192) and scales.shape == (50, 2) and scales.dtype == np.float32
    for b, (lo, hi) in enumerate([(0, 128), (128, 192)]):
        sc = (np.abs(x[:, lo:hi]).max(1) / 448).astype(np.float32)
        np.testing.assert_array_equal(scales[:, b], sc)
        safe = np.where(sc > 0, sc, 1).astype(np.float64)[:, None]
        y = torch.from_numpy(np.clip(x[:, lo:hi] / safe, -448, 448)).to(torch.float8_e4m3fn)
        want = y.view(torch.uint8).numpy()
        want = np.where(sc[:, None] > 0, want, 0)
        np.testing.assert_array_equal(codes[:, lo:hi], want)
    deq = F.dequant_fp8_b128(codes, scales)
    assert np.all(deq[9, 128:] == 0)
    assert deq[7, 5] == -448 * float(scales[7, 0])


def _golden_kv():
    vals = {}
    with open(os.path.join(GOLD, "kv_bytes_per_token.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v)
    return vals


def test_layout_reproduces_pages_kv_bytes_per_token():
    """The 512-wide KV row as 448 fp8 + 64 bf16 RoPE dims (576 B) and a 128-dim FP4
    indexer key (64 B) per CSA entry reproduce the pages' 4924 B/token to 0.3%."""
    gv = _golden_kv()
    row = 448 * 1 + 64 * 2
    key = 128 // 2
    per_tok = gv["csa_layers"] * (row + key) / 4 + gv["hca_layers"] * row / 128
    assert abs(per_tok - gv["bytes_per_token"]) / gv["bytes_per_token"] < 0.003
    window = gv["swa_layers"] * 128 * row / 1e6
    assert abs(window - gv["window_megabytes"]) / gv["window_megabytes"] < 0.15
