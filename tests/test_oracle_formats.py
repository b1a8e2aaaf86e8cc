"""Pins of the oracle's format decoding (CPU only).

Pinned against: the OCP tables stored under tests/golden (with citations),
torch's CPU float8 / bfloat16 casts (library routines) and asymmetric byte
patterns that expose a swapped nibble or a wrong scale block.
"""
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        a, b = line.split()
        rows.append((int(a, 16), float(b)))
    return rows


def _same(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.array_equal(np.isnan(a), np.isnan(b)) and \
        np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)]) and \
        np.array_equal(np.signbit(a[~np.isnan(a)]), np.signbit(b[~np.isnan(b)]))


def test_e2m1_all_16_codes_exact():
    rows = _read_table("e2m1_codes.txt")
    assert len(rows) == 16
    codes = np.array([c for c, _ in rows])
    want = np.array([v for _, v in rows])
    assert _same(F.e2m1_value(codes), want)


def test_e4m3_all_256_codes_vs_torch_cast():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(F.e4m3_value(b), ref)


def test_e4m3_table_points():
    for byte, val in _read_table("e4m3_points.txt"):
        assert _same(F.e4m3_value(np.array([byte])), np.array([val])), hex(byte)


def test_e8m0_all_256_codes_vs_torch_cast():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = F.e8m0_value(b)
    assert _same(got, ref)
    assert got[127] == 1.0 and got[128] == 2.0 and got[0] == 2.0 ** -127


def test_bf16_vs_torch_cast():
    rng = np.random.default_rng(5)
    u = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(u.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(F.bf16_value(u), ref)


def test_nibble_order_low_first():
    # byte 0x21: element 0 = code 1 (0.5), element 1 = code 2 (1.0)
    codes = F.unpack_e2m1_codes(np.array([[0x21, 0xF7]], np.uint8))
    assert codes.tolist() == [[1, 2, 7, 15]]


def test_dequant_block_scale_and_exactness():
    rng = np.random.default_rng(1)
    packed = rng.integers(0, 256, size=(5, 256), dtype=np.uint8)
    scale = rng.integers(0, 253, size=(5, 16), dtype=np.uint8)
    got = F.dequant_latent(packed, scale)
    # element i uses scale block i // 32: check with torch's casts, element by element
    e8 = torch.from_numpy(scale.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    codes = F.unpack_e2m1_codes(packed)
    table = {c: v for c, v in _read_table("e2m1_codes.txt")}
    for r in range(5):
        for i in range(0, 512, 7):
            want = table[int(codes[r, i])] * e8[r, i // 32]
            assert got[r, i] == want
    # a scale change in block 3 touches elements 96..127 only
    s2 = scale.copy()
    s2[0, 3] = s2[0, 3] + 1 if s2[0, 3] < 252 else s2[0, 3] - 1
    diff = F.dequant_latent(packed[:1], s2[:1]) != F.dequant_latent(packed[:1], scale[:1])
    nz = np.nonzero(diff[0])[0]
    assert nz.size == 0 or (nz.min() >= 96 and nz.max() < 128)


def test_generator_mxfp4_roundtrip_is_nearest_grid_point():
    """The generator's encoder (not the oracle) follows the OCP MX rounding rule."""
    from fp4_kv_cache_score_amd.synth import encode_mxfp4
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 512)).astype(np.float32) * 3
    packed, scale = encode_mxfp4(x)
    deq = F.dequant_latent(packed, scale)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    s = F.e8m0_value(scale)
    for r in range(4):
        for blk in range(16):
            sc = s[r, blk]
            amax = np.abs(x[r, blk * 32:(blk + 1) * 32]).max()
            assert sc == 2.0 ** (np.floor(np.log2(amax)) - 2)
            for i in range(blk * 32, blk * 32 + 32):
                m = abs(float(x[r, i])) / sc
                d = np.abs(grid - m)
                best = grid[d == d.min()]
                assert abs(deq[r, i]) / sc in best or m > 6
