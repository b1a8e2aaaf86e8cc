"""GPU parity of the fused score -> Top-K (csa2_score_topk).

Each work-group scores 4096 entries of a row into LDS and keeps a superset
of their Top-K; one work-group per row selects the Top-K from the keepers.
Checked on long rows (several slices; ragged lengths around the slice and
K boundaries: 0, 1, K - 1, K, K + 1, 4095, 4096, 4097, M):
* the indices equal those of the two-pass path (csa2_index_score, then
  csa2_topk on the written scores) and the oracle's Top-K of those GPU
  scores, bit for bit (the two kernels compute every score identically);
* all-equal scores select the lowest positions;
* a paged pool gives the contiguous pool's indices bit for bit;
* short rows (one slice), and the largest K whose keepers fit.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import csa2 as O
from fp4_kv_cache_score_amd import _lib as C
from fp4_kv_cache_score_amd import synth
from fp4_kv_cache_score_amd.configs import CONFIGS, FULL, REINDEX

pytestmark = pytest.mark.gpu

SLICE = 4096


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    C.lib()
    yield


def _lengths(seed, B, M, K):
    edge = [M, 0, 1, K - 1, K, K + 1, SLICE - 1, SLICE, SLICE + 1, 2 * SLICE, M - 1, M - SLICE]
    edge = [min(max(e, 0), M) for e in edge][:B]
    rng = np.random.default_rng(seed)
    rest = rng.integers(0, M + 1, B - len(edge))
    return np.concatenate([edge, rest]).astype(np.int32)


def _device(seed, B, M, K, lens=None, pages=None, zero_keys=False):
    from fp4_kv_cache_score_amd.device import DeviceCase
    cfg = CONFIGS[1].scaled(name="fused", seed=seed, B=B, M=M, K=K, P=0, W=8,
                            modes=(FULL, REINDEX))
    case = synth.make_case(cfg)
    if zero_keys:
        case.pool.idx_key[:] = 0
    dc = DeviceCase(case)
    if lens is not None:
        dc.use_lengths(lens)
    if pages is not None:
        dc.use_pages(pages, seed=pages)
    return dc


@pytest.mark.parametrize("B,M,K", [(64, 16448, 256), (8, 40000, 512), (3, 3000, 64),
                                   (2, 9000, 3008)])
def test_fused_topk_equals_two_pass_and_oracle(B, M, K):
    lens = _lengths(11 + B, B, M, K)
    say("case: fused score->Top-K B=%d M=%d K=%d, ragged lengths" % (B, M, K))
    dc = _device(90 + B, B, M, K, lens=lens)
    nv = torch.from_numpy(lens).cuda()
    for ell in range(2):
        got = dc.score_topk(ell).cpu().numpy()
        s = dc.index_scores(ell).view(B, M)
        two = dc.topk(s, K, n_valid=nv).cpu().numpy()
        sn = s.cpu().numpy()
        for b in range(B):
            want, _ = O.topk(sn[b].astype(np.float64), K, n_valid=int(lens[b]))
            assert np.array_equal(two[b], want), (ell, b, int(lens[b]))
            assert np.array_equal(got[b], want), (ell, b, int(lens[b]))


def test_fused_all_scores_equal_take_the_lowest_positions():
    B, M, K = 16, 20000, 300
    lens = _lengths(12, B, M, K)
    say("case: fused select, all index scores 0")
    dc = _device(91, B, M, K, lens=lens, zero_keys=True)
    got = dc.score_topk(0).cpu().numpy()
    for b in range(B):
        n = min(int(lens[b]), K)
        want = np.concatenate([np.arange(n), -np.ones(K - n)]).astype(np.int32)
        assert np.array_equal(got[b], want), b


def test_fused_paged_equals_contiguous():
    B, M, K = 32, 32768, 512
    lens = _lengths(13, B, M, K)
    say("case: fused select on a paged pool (pages of 64 entries)")
    a = _device(92, B, M, K, lens=lens).score_topk(0)
    b = _device(92, B, M, K, lens=lens, pages=6).score_topk(0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
