"""GPU checks of paged pools (csa2_pool.pages: a page table into shared arrays).

A paged pool holds the same entries as a contiguous one, only at other rows,
so every result over it must be bit-identical to the contiguous run (which the
other parity tests hold to the oracle): the decode schedule (flat,
hierarchical, ragged), the scores, chunked prefill through the schedule (short
rows, and rows long enough for the group select) and the write side (entries
appended into pages land where the table says).
Pages are shuffled among spare ones, so a wrong row would read other data.
"""
import sys

import numpy as np
import pytest
import torch

from fp4_kv_cache_score_amd import synth
from fp4_kv_cache_score_amd.configs import CONFIGS, FULL, REINDEX, REUSE

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


def _outputs(dc):
    return [(d["idx"].clone(), d["o"].clone(), d["lse"].clone()) for d in dc.layers]


@pytest.mark.parametrize("ci,kw,lg2,lens", [
    (1, dict(B=4, M=4096), 8, None),
    (2, dict(B=2, M=32768), 10, None),
    (1, dict(B=5, M=3072), 6, [3072, 0, 1, 2000, 64]),
])
def test_paged_decode_equals_contiguous(ci, kw, lg2, lens):
    from fp4_kv_cache_score_amd.device import DeviceCase
    cfg = CONFIGS[ci].scaled(name="pg", **kw)
    say("case: paged decode", CONFIGS[ci].name, kw, "page 2^%d" % lg2, "lens" if lens else "")
    case = synth.make_case(cfg)
    runs = []
    for paged in (False, True):
        dc = DeviceCase(case)
        if lens:
            dc.use_lengths(lens)
        if paged:
            dc.use_pages(lg2, seed=lg2)
        dc.prepare_decode()
        dc.decode_layers()
        torch.cuda.synchronize()
        runs.append(_outputs(dc))
        if not paged:
            s0 = dc.index_scores(0).clone()
        else:
            s1 = dc.index_scores(0).clone()
    for ell, (a, b) in enumerate(zip(*runs)):
        for x, y in zip(a, b):
            assert torch.equal(x, y), ell
    assert torch.equal(s0, s1)


@pytest.mark.parametrize("kw", [
    dict(Q=160, M=4096, K=96, chunk_pos=4 * 4096 - 3000),
    # rows over 16384 entries on 256 rows: the group select from the run maxima
    dict(Q=128, M=24576, K=512, chunk_pos=-1),
], ids=["short_rows", "group_select"])
def test_paged_prefill_equals_contiguous(kw):
    from fp4_kv_cache_score_amd.device import DeviceCase
    cfg = CONFIGS[4].scaled(name="pgp", seed=81, B=2, W=40, modes=(FULL, REINDEX, REUSE), **kw)
    say("case: paged prefill Q=%d M=%d K=%d" % (cfg.Q, cfg.M, cfg.K))
    case = synth.make_case(cfg)
    runs = []
    for paged in (False, True):
        dc = DeviceCase(case)
        if paged:
            dc.use_pages(7, seed=5)
        dc.prefill_layers()
        torch.cuda.synchronize()
        runs.append(_outputs(dc))
    for ell, (a, b) in enumerate(zip(*runs)):
        for x, y in zip(a, b):
            assert torch.equal(x, y), ell


def test_paged_append_writes_the_mapped_rows():
    from fp4_kv_cache_score_amd import _lib as C
    say("case: paged append")
    rng = np.random.default_rng(6)
    B, M, T, lg2 = 2, 512, 40, 6
    ps, npg = 1 << lg2, M >> 6
    perm = rng.permutation(B * npg + 2).astype(np.int32)[:B * npg]
    table = torch.from_numpy(perm.reshape(B, npg)).cuda()
    rows = (B * npg + 2) * ps
    xl = torch.from_numpy((rng.standard_normal((B, T, 512)) * 3).astype(np.float32)).cuda()
    xk = torch.from_numpy(rng.standard_normal((B, T, 8, 64)).astype(np.float32)).cuda()
    slot = torch.from_numpy(np.stack([rng.permutation(M)[:T] for _ in range(B)]).astype(np.int32)).cuda()
    cont = [torch.zeros((B * M, w), dtype=torch.uint8, device="cuda") for w in (256, 16, 512)]
    paged = [torch.zeros((rows, w), dtype=torch.uint8, device="cuda") for w in (256, 16, 512)]
    C.csa2_pool_append(cont[0], cont[1], cont[2], B, M, xl, xk, slot, T)
    C.csa2_pool_append(paged[0], paged[1], paged[2], B, M, xl, xk, slot, T, pages=table,
                       page_log2=lg2)
    torch.cuda.synchronize()
    e = np.arange(M)
    for b in range(B):
        prow = perm[b * npg + (e >> lg2)] * ps + (e & (ps - 1))
        for c, p in zip(cont, paged):
            assert torch.equal(c[b * M:(b + 1) * M], p[torch.from_numpy(prow).long().cuda()]), b
