"""Pins of the oracle's write side (new pool entries, window ring) against definitions.

Checked without any GPU: exact round trips of every representable E2M1 and
E4M3 value, the ties-to-even cases written out, saturation and the scale
exponent rule at their edges, brute-force nearest-value optimality on random
blocks, torch's float8_e4m3fn cast (a library routine) for E4M3, the input
generator's separate MXFP4 encoder, and brute force for the pool and ring
appends.
"""
import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import write_side as WS
from fp4_kv_cache_score_amd import synth


E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_every_value_round_trips_at_every_scale():
    codes = np.arange(16, dtype=np.uint8)
    vals = F.e2m1_value(codes)                        # +-{0 .. 6}, includes 6.0 so amax = 6 * 2^k
    for k in range(-120, 121, 7):
        x = np.concatenate([vals, vals[::-1]]) * 2.0 ** k
        packed, sc = WS.encode_mxfp4_block(x.astype(np.float32))
        assert sc == k + 127, k
        got = F.unpack_e2m1_codes(packed)
        want = np.concatenate([codes, codes[::-1]])
        # -0 encodes with its sign
        assert np.array_equal(got, want), k


def test_e2m1_ties_go_to_the_even_code():
    # scale 1 (amax = 6); each midpoint lies halfway between two grid values
    table = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    mids = list(table)
    x = np.zeros(32, np.float32)
    x[0] = 6.0
    x[1:1 + len(mids)] = mids
    x[8:8 + len(mids)] = [-m for m in mids]
    packed, sc = WS.encode_mxfp4_block(x)
    c = F.unpack_e2m1_codes(packed)
    assert sc == 127
    assert list(c[1:1 + len(mids)]) == [table[m] for m in mids]
    assert list(c[8:8 + len(mids)]) == [table[m] | 8 for m in mids]


def test_e2m1_scale_exponent_and_saturation_edges():
    # amax in [6, 8) * 2^k: shared exponent k, values above 6 * 2^k saturate
    x = np.zeros(32, np.float32)
    x[0], x[1], x[2] = 7.0, 6.5, -7.99
    packed, sc = WS.encode_mxfp4_block(x)
    c = F.unpack_e2m1_codes(packed)
    assert sc == 127 and c[0] == 7 and c[1] == 7 and c[2] == 15
    # amax = 8: floor(log2 8) - 2 = 1, so 8 -> 4 * 2^1
    x[0] = 8.0
    packed, sc = WS.encode_mxfp4_block(x)
    assert sc == 128 and F.unpack_e2m1_codes(packed)[0] == 6
    # amax just below a power of two: 3.999 -> floor(log2) = 1, shared -1, 3.999 * 2 = 7.998 -> 6
    x[:] = 0
    x[0] = 3.999
    packed, sc = WS.encode_mxfp4_block(x)
    assert sc == 126 and F.unpack_e2m1_codes(packed)[0] == 7


def test_e2m1_zero_block_and_negative_zero():
    packed, sc = WS.encode_mxfp4_block(np.zeros(32, np.float32))
    assert sc == 127 and not packed.any()
    x = np.zeros(32, np.float32)
    x[0], x[1], x[2] = 6.0, -0.0, -0.1            # -0.1 rounds to zero and keeps its sign
    c = F.unpack_e2m1_codes(WS.encode_mxfp4_block(x)[0])
    assert c[1] == 8 and c[2] == 8


def test_mxfp4_nearest_value_brute_force():
    rng = np.random.default_rng(5)
    for trial in range(300):
        scale_exp = rng.integers(-30, 30)
        x = (rng.standard_normal(32) * 2.0 ** scale_exp).astype(np.float32)
        if trial % 7 == 0:
            x[rng.integers(32)] *= 40.0            # a large outlier
        packed, sc = WS.encode_mxfp4_block(x)
        s = 2.0 ** (int(sc) - 127)
        amax = float(np.max(np.abs(x.astype(np.float64))))
        assert s <= amax / 4 < 2 * s               # shared = floor(log2 amax) - 2
        got = F.e2m1_value(F.unpack_e2m1_codes(packed)) * s
        cand = np.array(E2M1_VALUES) * s
        for v, g in zip(x.astype(np.float64), got):
            best = np.min(np.abs(np.abs(v) - cand))
            assert abs(abs(v) - abs(g)) == best or (abs(v) > 6 * s and abs(g) == 6 * s)
            assert g == 0 or np.sign(g) == np.sign(v)


def test_mxfp4_rows_match_the_generators_encoder():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((40, 512)) * np.exp(rng.uniform(-8, 8, (40, 1)))).astype(np.float32)
    x[3, :32] = 0.0
    gp, gs = synth.encode_mxfp4(x)
    for r in range(40):
        p, s = WS.encode_mxfp4_row(x[r])
        assert np.array_equal(p, gp[r]) and np.array_equal(s, gs[r]), r


def test_e4m3_every_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    got = WS.encode_e4m3(F.e4m3_value(codes).astype(np.float32))
    assert np.array_equal(got, codes)


def test_e4m3_ties_and_clamp():
    g = WS.E4M3_GRID
    mids = (g[:-1] + g[1:]) / 2                    # exactly representable in float32
    got = WS.encode_e4m3(mids.astype(np.float32))
    lo = np.arange(len(mids))
    want = np.where(lo % 2 == 0, lo, lo + 1)        # the even code of each pair
    assert np.array_equal(got.astype(np.int64), want)
    assert WS.encode_e4m3(np.float32(1e6)) == 0x7E and WS.encode_e4m3(np.float32(-1e6)) == 0xFE


def test_e4m3_matches_torch_cast():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(20000) * np.exp(rng.uniform(-14, 8, 20000)),
                        rng.uniform(-600, 600, 2000), [0.0, -0.0, 2.0 ** -10, 448.0, 464.0]])
    x = x.astype(np.float32)
    want = torch.from_numpy(x).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(WS.encode_e4m3(x), want)


def test_append_pool_brute_force():
    rng = np.random.default_rng(2)
    B, M, T = 2, 5, 4
    lat = rng.integers(0, 256, (B, M, 256), dtype=np.uint8)
    sc = rng.integers(100, 140, (B, M, 16), dtype=np.uint8)
    key = rng.integers(0, 126, (B, M, 8, 64), dtype=np.uint8)
    xl = rng.standard_normal((B, T, 512)).astype(np.float32)
    xk = rng.standard_normal((B, T, 8, 64)).astype(np.float32)
    slot = np.array([[3, -1, 0, 7], [4, 1, 5, 2]])
    nl, ns, nk = WS.append_pool(lat, sc, key, xl, xk, slot)
    for b in range(B):
        written = {int(e): t for t, e in enumerate(slot[b]) if 0 <= e < M}
        for e in range(M):
            if e in written:
                t = written[e]
                v = F.dequant_latent(nl[b, e], ns[b, e])
                # every element within half an E2M1 step (or saturated) of the input
                s = np.repeat(F.e8m0_value(ns[b, e]), 32)
                assert np.all(np.abs(v - xl[b, t]) <= np.maximum(s, 2 * s * (np.abs(xl[b, t]) >= 4 * s)))
                assert np.array_equal(nk[b, e], WS.encode_e4m3(xk[b, t]))
            else:
                assert np.array_equal(nl[b, e], lat[b, e]) and np.array_equal(ns[b, e], sc[b, e])
                assert np.array_equal(nk[b, e], key[b, e])


def test_append_window_ring():
    rng = np.random.default_rng(4)
    B, W, D = 2, 4, 512
    ring = rng.integers(0, 126, (B, W, D), dtype=np.uint8)
    x = rng.standard_normal((B, 6, D)).astype(np.float32)
    out = WS.append_window(ring, x, pos0=3)          # tokens 3..8: rows of tokens 5..8 survive
    for p in range(5, 9):
        assert np.array_equal(out[:, p % W], WS.encode_e4m3(x[:, p - 3]))
    out2 = WS.append_window(ring, x[:, :2], pos0=10)  # tokens 10, 11 -> rows 2, 3
    assert np.array_equal(out2[:, 2], WS.encode_e4m3(x[:, 0]))
    assert np.array_equal(out2[:, 3], WS.encode_e4m3(x[:, 1]))
    assert np.array_equal(out2[:, :2], ring[:, :2])
