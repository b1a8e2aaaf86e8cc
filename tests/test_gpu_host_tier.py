"""GPU checks of the host tier (csa2_pool_restore / _offload, csa2_swa_restore / _offload).

The calls move stored bytes unchanged, so the bar is bit-exact: a restored
range equals the host bytes and nothing outside it changes; an offloaded range
equals the device bytes; and a decode step after offloading a sequence,
scrambling its device copy and restoring it gives bit-identical outputs.  The
copies run on a second stream (default priority) beside the decode launches.
"""
import sys

import numpy as np
import pytest
import torch

from fp4_kv_cache_score_amd import synth
from fp4_kv_cache_score_amd.configs import CONFIGS

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


def _pinned(a: np.ndarray) -> torch.Tensor:
    t = torch.empty(a.shape, dtype=torch.uint8, pin_memory=True)
    t.copy_(torch.from_numpy(a))
    return t


def test_pool_restore_and_offload_ranges():
    from fp4_kv_cache_score_amd import _lib as C
    say("case: pool restore / offload B=3 M=500")
    rng = np.random.default_rng(3)
    B, M = 3, 500
    dev = [rng.integers(0, 256, (B, M, w), dtype=np.uint8) for w in (256, 16, 512)]
    g = [torch.from_numpy(a.copy()).cuda() for a in dev]
    n, seq, e0 = 123, 1, 250
    host = [_pinned(rng.integers(0, 256, (n, a.shape[2]), dtype=np.uint8)) for a in dev]
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        C.csa2_pool_restore(g[0], g[1], g[2], B, M, seq, e0, n, host[0], host[1], host[2], side)
    side.synchronize()
    for a, t, h in zip(dev, g, host):
        want = a.copy()
        want[seq, e0:e0 + n] = h.numpy()
        assert np.array_equal(t.cpu().numpy(), want)
    out = [torch.empty((77, a.shape[2]), dtype=torch.uint8, pin_memory=True) for a in dev]
    C.csa2_pool_offload(g[0], g[1], g[2], B, M, 2, 400, 77, out[0], out[1], out[2], side)
    side.synchronize()
    for t, o in zip(g, out):
        assert np.array_equal(o.numpy(), t[2, 400:477].cpu().numpy())


def test_swa_ring_round_trip():
    from fp4_kv_cache_score_amd import _lib as C
    say("case: window ring restore / offload")
    rng = np.random.default_rng(4)
    B, W = 4, 128
    ring = torch.from_numpy(rng.integers(0, 126, (B, W, 512), dtype=np.uint8)).cuda()
    before = ring.cpu().numpy()
    h = torch.empty((W, 512), dtype=torch.uint8, pin_memory=True)
    C.csa2_swa_offload(ring, B, W, 2, h)
    torch.cuda.synchronize()
    assert np.array_equal(h.numpy(), before[2])
    new = _pinned(rng.integers(0, 126, (W, 512), dtype=np.uint8))
    C.csa2_swa_restore(ring, B, W, 0, new)
    torch.cuda.synchronize()
    after = ring.cpu().numpy()
    assert np.array_equal(after[0], new.numpy()) and np.array_equal(after[1:], before[1:])


def test_decode_after_offload_scramble_restore_is_identical():
    from fp4_kv_cache_score_amd import _lib as C
    from fp4_kv_cache_score_amd.device import DeviceCase
    cfg = CONFIGS[1].scaled(name="tier", B=4, M=4096, K=128)
    say("case: decode after a restore", cfg.name, "B=%d M=%d" % (cfg.B, cfg.M))
    dc = DeviceCase(synth.make_case(cfg))
    dc.prepare_decode()
    dc.decode_layers()
    torch.cuda.synchronize()
    ref = [(d["idx"].clone(), d["o"].clone(), d["lse"].clone()) for d in dc.layers]
    seq = 2
    host = [torch.empty((cfg.M, w), dtype=torch.uint8, pin_memory=True) for w in (256, 16, 512)]
    side = torch.cuda.Stream()
    C.csa2_pool_offload(dc.latent, dc.scale, dc.idx_key, cfg.B, cfg.M, seq, 0, cfg.M,
                        host[0], host[1], host[2], side)
    side.synchronize()
    for t in (dc.latent, dc.scale, dc.idx_key):       # lose the device copy of the sequence
        t[seq].random_(0, 126)
    C.csa2_pool_restore(dc.latent, dc.scale, dc.idx_key, cfg.B, cfg.M, seq, 0, cfg.M,
                        host[0], host[1], host[2], side)
    side.synchronize()
    dc.decode_layers()
    torch.cuda.synchronize()
    for (i0, o0, l0), d in zip(ref, dc.layers):
        assert torch.equal(i0, d["idx"]) and torch.equal(o0, d["o"]) and torch.equal(l0, d["lse"])
