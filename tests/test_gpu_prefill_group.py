"""GPU parity of the chunked-prefill group select (csa2_prefill_layers on many
rows longer than one work-group's select).

The score kernel writes, beside each query's scores, the largest visible
score of every run of 16 entries; the select keeps the K best runs (ties to
the earlier run), which hold the row's Top-K, and selects from their
entries.  Each row's Top-K must be exactly the Top-K of the scores the same
kernel writes through csa2_index_score (equal scores to the lower entry, -0
equal to +0), for every layer that scores:
* random inputs, K = 512 and K = 64, one and two sequences;
* keys repeated from a set of 16, so that run maxima tie at the K-th run
  (several hundred runs share it) and entries tie inside the kept runs;
* rows whose head weights are all zero (every score +0: every run ties, the
  first K entries win) mixed with ordinary rows;
* a chunk whose tokens see different counts, with ragged query tiles;
* a ragged batch (sequence lengths 17000 and 100: rows with fewer runs than K).
"""
import sys

import numpy as np
import pytest
import torch

from fp4_kv_cache_score_amd import synth
from fp4_kv_cache_score_amd.configs import CONFIGS, FULL, REINDEX

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


def exact_topk(s, n, K):
    """Ascending positions of the K largest of s[:n] (ties to the lower position,
    -0 equal to +0), -1 padded."""
    v = s[:n].astype(np.float64)
    v = np.where(v == 0.0, 0.0, v)
    order = np.lexsort((np.arange(n), -v))
    top = np.sort(order[:K])
    out = np.full(K, -1, np.int32)
    out[:len(top)] = top
    return out


CASES = [
    dict(name="random_k512", B=1, Q=256, M=20000, K=512),
    dict(name="random_k64_b2", B=2, Q=128, M=24000, K=64),
    dict(name="repeated_keys", B=1, Q=256, M=20000, K=512, repeat=16),
    dict(name="zero_weight_rows", B=1, Q=256, M=20000, K=512, zero_rows=3),
    dict(name="ragged_visible", B=1, Q=300, M=40000, K=256, chunk_pos=4 * 30000),
    dict(name="ragged_lengths", B=2, Q=128, M=24000, K=512, lens=[17000, 100]),
]


@pytest.mark.parametrize("kw", CASES, ids=[c["name"] for c in CASES])
def test_prefill_group_select_exact(kw):
    from fp4_kv_cache_score_amd.device import DeviceCase
    kw = dict(kw)
    name = kw.pop("name")
    repeat = kw.pop("repeat", 0)
    zero_rows = kw.pop("zero_rows", 0)
    chunk_pos = kw.pop("chunk_pos", -1)
    lens = kw.pop("lens", None)
    cfg = CONFIGS[4].scaled(name=name, seed=300 + len(name), W=16, modes=(FULL, REINDEX),
                            causal=True, chunk_pos=chunk_pos, **kw)
    say("case: prefill group select", name, "B=%d Q=%d M=%d K=%d pos0=%d"
        % (cfg.B, cfg.Q, cfg.M, cfg.K, cfg.pos0))
    case = synth.make_case(cfg)
    if repeat:
        rng = np.random.default_rng(5)
        pick = rng.integers(0, repeat, (cfg.B, cfg.M))
        base = case.pool.idx_key[:, :repeat].copy()
        case.pool.idx_key[:] = np.take_along_axis(base, pick[:, :, None, None], axis=1)
    if zero_rows:
        for L in case.layers:
            L.w_idx[:, ::zero_rows, :] = 0.0
    dc = DeviceCase(case)
    if lens is not None:
        dc.use_lengths(lens)
    dc.prefill_layers()
    torch.cuda.synchronize()
    vis = dc.visible_counts().cpu().numpy().reshape(cfg.B, cfg.Q)
    assert vis.min() > 16384, "the chunk must take the group select"
    if lens is not None:   # sequence b holds its first lens[b] entries
        vis = np.minimum(vis, np.asarray(lens, dtype=np.int64)[:, None])
    for ell in range(cfg.L):
        scores = dc.index_scores(ell).cpu().numpy()
        got = dc.layers[ell]["idx"].cpu().numpy()
        bad = 0
        for b in range(cfg.B):
            for t in range(cfg.Q):
                want = exact_topk(scores[b, t], int(vis[b, t]), cfg.K)
                if not np.array_equal(got[b, t], want):
                    bad += 1
                    if bad <= 3:
                        d = np.setxor1d(got[b, t], want)
                        say("  layer %d b=%d t=%d differs at %s" % (ell, b, t, d[:8]))
        assert bad == 0, "layer %d: %d rows differ" % (ell, bad)
    say("  exact on %d rows x %d layers" % (cfg.B * cfg.Q, cfg.L))


def test_prefill_group_select_full_size_every_row():
    """The 2048-token chunk over 65536 entries (the prefill workload's shape): the
    group select's Top-K of every row equals the exact Top-K of the scores the
    score kernel writes for the same chunk."""
    from fp4_kv_cache_score_amd.device import DeviceCase
    cfg = CONFIGS[4].scaled(modes=(FULL,))
    say("case: prefill group select full size Q=%d M=%d K=%d pos0=%d" % (cfg.Q, cfg.M, cfg.K, cfg.pos0))
    case = synth.make_case(cfg)
    dc = DeviceCase(case)
    dc.prefill_layers()
    torch.cuda.synchronize()
    got = dc.layers[0]["idx"].cpu().numpy()[0]
    vis = dc.visible_counts().cpu().numpy()
    scores = dc.index_scores(0).cpu().numpy()[0]
    bad = 0
    for t in range(cfg.Q):
        if not np.array_equal(got[t], exact_topk(scores[t], int(vis[t]), cfg.K)):
            bad += 1
    assert bad == 0, "%d of %d rows differ" % (bad, cfg.Q)
    say("  exact on all %d rows" % cfg.Q)
