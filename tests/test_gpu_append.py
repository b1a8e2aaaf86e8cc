"""GPU parity of the write side (csa2_pool_append, csa2_swa_append) against the oracle.

The encodings are byte work, so the bar is bit-exact: whole pool arrays and
window rings after the GPU append equal the oracle's (oracle/write_side.py) on
the same inputs.  Inputs mix wide magnitudes (fp32 subnormals up to 1e38),
exact E2M1 and E4M3 ties, values past 448, all-zero blocks, -0, skipped slots
(-1 and >= M), ring wrap-around and more new tokens than ring rows; one case
encodes a full-size batch and checks sampled rows.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import write_side as WS

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_kv_cache_score_amd import _lib
    _lib.lib()
    yield


def _rows(rng, n, d):
    """fp32 rows with the awkward cases of both encodings."""
    x = rng.standard_normal((n, d)) * np.exp2(rng.integers(-40, 40, (n, 1)))
    for r in range(n):
        kind = r % 8
        if kind == 1:          # E2M1 ties at the block scale of amax = 6 * 2^k
            k = int(rng.integers(-20, 20))
            mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
            x[r] = np.tile(np.concatenate([mids, -mids]), d // 16) * 2.0 ** k
        elif kind == 2:        # E4M3 ties and values beyond 448
            g = WS.E4M3_GRID
            m = (g[:-1] + g[1:]) / 2
            x[r] = np.resize(np.concatenate([m, -m, [500.0, -1e6, 448.0]]), d)
        elif kind == 3:        # fp32 subnormals and zeros
            x[r] = rng.integers(-50, 50, d) * 2.0 ** -149
            x[r, :32] = 0.0
            x[r, 32] = -0.0
        elif kind == 4:        # huge
            x[r] = rng.standard_normal(d) * 1e37
        elif kind == 5:        # a block with one outlier
            x[r, rng.integers(d)] *= 300.0
    return x.astype(np.float32)


def test_pool_append_bit_exact():
    from fp4_kv_cache_score_amd import _lib as C
    say("case: pool append B=3 M=200 T=56")
    rng = np.random.default_rng(21)
    B, M, T = 3, 200, 56
    lat = rng.integers(0, 256, (B, M, 256), dtype=np.uint8)
    sc = rng.integers(0, 253, (B, M, 16), dtype=np.uint8)
    key = rng.integers(0, 256, (B, M, 8, 64), dtype=np.uint8)
    xl = _rows(rng, B * T, 512).reshape(B, T, 512)
    xk = _rows(rng, B * T, 512).reshape(B, T, 8, 64)
    slot = np.stack([rng.permutation(M)[:T] for _ in range(B)]).astype(np.int32)
    slot[0, 3], slot[1, 7], slot[2, 0] = -1, M, M + 100          # skipped rows
    want = WS.append_pool(lat, sc, key, xl, xk, slot)
    g = [torch.from_numpy(a.copy()).cuda() for a in (lat, sc, key)]
    C.csa2_pool_append(g[0], g[1], g[2], B, M, torch.from_numpy(xl).cuda(),
                       torch.from_numpy(xk).cuda(), torch.from_numpy(slot).cuda(), T)
    torch.cuda.synchronize()
    for name, got, w in zip(("latent", "scale", "idx_key"), g, want):
        got = got.cpu().numpy()
        bad = np.argwhere(got != w)
        assert bad.size == 0, (name, bad[:5], got[tuple(bad[0])], w[tuple(bad[0])])


@pytest.mark.parametrize("W,T,pos0", [(128, 5, 100), (128, 300, 7), (16, 16, 0), (7, 3, 12345678901)])
def test_swa_append_ring_bit_exact(W, T, pos0):
    from fp4_kv_cache_score_amd import _lib as C
    say("case: window append W=%d T=%d pos0=%d" % (W, T, pos0))
    rng = np.random.default_rng(W * 7 + T)
    B = 2
    ring = rng.integers(0, 126, (B, W, 512), dtype=np.uint8)
    x = _rows(rng, B * T, 512).reshape(B, T, 512)
    want = WS.append_window(ring, x, pos0)
    g = torch.from_numpy(ring.copy()).cuda()
    C.csa2_swa_append(g, B, W, torch.from_numpy(x).cuda(), pos0, T)
    torch.cuda.synchronize()
    assert np.array_equal(g.cpu().numpy(), want)


def test_pool_append_full_size_sampled():
    from fp4_kv_cache_score_amd import _lib as C
    B, M, T = 32, 32768, 1024
    say("case: pool append full size B=%d M=%d T=%d" % (B, M, T))
    rng = np.random.default_rng(33)
    xl = (rng.standard_normal((B, T, 512)) * np.exp2(rng.integers(-6, 6, (B, T, 1)))).astype(np.float32)
    xk = rng.standard_normal((B, T, 8, 64)).astype(np.float32)
    slot = np.broadcast_to((np.arange(T) * 31 + 5) % M, (B, T)).astype(np.int32).copy()
    lat = torch.zeros((B, M, 256), dtype=torch.uint8, device="cuda")
    sc = torch.zeros((B, M, 16), dtype=torch.uint8, device="cuda")
    key = torch.zeros((B, M, 8, 64), dtype=torch.uint8, device="cuda")
    C.csa2_pool_append(lat, sc, key, B, M, torch.from_numpy(xl).cuda(), torch.from_numpy(xk).cuda(),
                       torch.from_numpy(slot).cuda(), T)
    torch.cuda.synchronize()
    for b, t in [(0, 0), (0, T - 1), (31, 17), (13, 512), (7, 1000), (20, 3)]:
        e = slot[b, t]
        p, s = WS.encode_mxfp4_row(xl[b, t])
        assert np.array_equal(lat[b, e].cpu().numpy(), p), (b, t)
        assert np.array_equal(sc[b, e].cpu().numpy(), s), (b, t)
        assert np.array_equal(key[b, e].cpu().numpy(), WS.encode_e4m3(xk[b, t])), (b, t)
    # entries no row named stay zero
    assert int(lat[:, 1].sum()) == 0 and int(key[:, 2].sum()) == 0
