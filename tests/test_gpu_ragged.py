"""GPU parity of ragged batches: per-sequence pool lengths (csa2_pool.len).

Sequence b of a ragged batch holds its first len[b] entries; the oracle runs
each sequence on its pool sliced to those entries (the definition of the
ragged batch), so no new oracle function is involved.  Checked: the decode
schedule (flat and hierarchical, one-work-group and multi-work-group
selects) with lengths that are full, 0, 1, below K and below P; scores past
a sequence's length are -inf; chunked prefill within a shorter sequence.
Top-K exact except near ties (counted), attention within 2e-3 on the GPU's
own selection.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import csa2 as O
from fp4_kv_cache_score_amd import synth
from fp4_kv_cache_score_amd.configs import CONFIGS, FULL, REINDEX, REUSE
from parity import ATTN_TOL, TieReport, attn_rel_err, score_bound

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


def _check_decode(case, dc, lens, P):
    cfg = case.cfg
    res = dc.results()
    rep = TieReport()
    worst = 0.0
    p = case.pool
    for b in range(cfg.B):
        n = int(lens[b])
        lat, sc, key = p.latent[b, :n], p.scale[b, :n], p.idx_key[b, :n]
        layers = [dict(mode=L.mode,
                       q_idx=None if L.q_idx is None else L.q_idx[b, 0],
                       w_idx=None if L.w_idx is None else L.w_idx[b, 0],
                       q=L.q[b, 0], swa=L.swa[b]) for L in case.layers]
        want = O.decode_sequence(lat, sc, key, layers, cfg.K, P)
        for ell, (w, g) in enumerate(zip(want, res)):
            gi = g["idx"][b, 0]                  # decode outputs are [B][Q = 1][...]
            assert (gi[gi >= 0] < max(n, 1)).all() and (n > 0 or (gi == -1).all()), (b, ell)
            if w["mode"] != REUSE:
                rep.check(gi, w["idx"], w.get("gap"), "b=%d layer %d" % (b, ell))
            keys = O.gather_keys(lat, sc, gi, layers[ell]["swa"])
            wo, wl = O.attend(layers[ell]["q"], keys)
            err = attn_rel_err(g["o"][b, 0], wo)
            worst = max(worst, err)
            assert err < ATTN_TOL, (b, ell, err)
            assert np.allclose(g["lse"][b, 0], wl, rtol=1e-5, atol=1e-5), (b, ell)
    say("  top-k:", rep, " worst attention rel err %.3g" % worst)


@pytest.mark.parametrize("name,B,M,K,P,lens,modes", [
    ("flat", 5, 3000, 128, 0, [3000, 1, 1777, 0, 100], (FULL, REINDEX, REUSE)),
    ("hier", 4, 4000, 64, 256, [4000, 200, 30, 0], (FULL, REINDEX, REINDEX)),
    ("multi-wg", 2, 40000, 96, 0, [40000, 12345], (FULL, REUSE, REINDEX)),
    # hierarchical with the multi-work-group joint Top-P / Top-K: lengths full,
    # between P and 32768, below P, below K and 0
    ("hier-multi-wg", 5, 40000, 128, 2048, [40000, 30001, 1500, 100, 0],
     (FULL, REINDEX, REUSE, REINDEX)),
    # the threshold-bin joint select: lengths full, between P and M, below P,
    # below K and 0
    ("hier-bin", 5, 70000, 256, 8192, [70000, 40001, 5000, 100, 0], (FULL, REINDEX, REUSE)),
])
def test_ragged_decode(name, B, M, K, P, lens, modes):
    from fp4_kv_cache_score_amd.device import DeviceCase
    say("case: ragged decode %s B=%d M=%d K=%d P=%d lens=%s" % (name, B, M, K, P, lens))
    cfg = CONFIGS[1].scaled(name="rg", seed=60 + B, B=B, M=M, K=K, P=P, W=32, modes=modes)
    case = synth.make_case(cfg)
    dc = DeviceCase(case)
    dc.use_lengths(lens)
    dc.prepare_decode()
    dc.decode_layers()
    torch.cuda.synchronize()
    _check_decode(case, dc, lens, P)


def test_ragged_scores_are_minus_inf_past_length():
    from fp4_kv_cache_score_amd.device import DeviceCase
    say("case: ragged scores")
    lens = [700, 0, 1024]
    cfg = CONFIGS[1].scaled(name="rs", seed=71, B=3, M=1024, K=16, W=8, modes=(FULL,))
    case = synth.make_case(cfg)
    dc = DeviceCase(case)
    dc.use_lengths(lens)
    s = dc.index_scores(0).cpu().numpy().reshape(3, 1024)
    L = case.layers[0]
    for b, n in enumerate(lens):
        assert np.all(s[b, n:] == -np.inf)
        if n:
            want = O.index_scores(case.pool.idx_key[b, :n], L.q_idx[b, 0], L.w_idx[b, 0])
            bound = score_bound(case.pool.idx_key[b, :n], L.q_idx[b, 0], L.w_idx[b, 0], want)
            assert np.all(np.abs(s[b, :n] - want) <= bound), b


def test_ragged_prefill_layers():
    from fp4_kv_cache_score_amd.device import DeviceCase
    lens = [2000, 300]
    say("case: ragged prefill lens=%s" % lens)
    cfg = CONFIGS[4].scaled(name="rp", seed=72, B=2, Q=100, M=2000, K=64, W=16,
                            modes=(FULL, REUSE), chunk_pos=7000)
    case = synth.make_case(cfg)
    dc = DeviceCase(case)
    dc.use_lengths(lens)
    dc.prefill_layers()
    torch.cuda.synchronize()
    rep = TieReport()
    p = case.pool
    for b, n in enumerate(lens):
        gi = dc.layers[0]["idx"][b].cpu().numpy()
        go = [d["o"][b].cpu().numpy() for d in dc.layers]
        L = case.layers
        for t in range(0, cfg.Q, 7):
            lay = [dict(mode=X.mode, q_idx=None if X.q_idx is None else X.q_idx[b, t:t + 1],
                        w_idx=None if X.w_idx is None else X.w_idx[b, t:t + 1],
                        q=X.q[b, t:t + 1], swa=X.swa[b, t:t + cfg.W]) for X in L]
            recs = O.prefill_layers(p.latent[b, :n], p.scale[b, :n], p.idx_key[b, :n], lay, 1,
                                    cfg.pos0 + t, cfg.ratio, cfg.K, cfg.W)
            rep.check(gi[t], recs[0]["idx"][0], recs[0]["gap"][0], "b=%d t=%d" % (b, t))
            for ell in range(2):
                keys = O.gather_keys(p.latent[b, :n], p.scale[b, :n], gi[t], L[ell].swa[b, t:t + cfg.W])
                wo, _ = O.attend(L[ell].q[b, t], keys)
                assert attn_rel_err(go[ell][t], wo) < ATTN_TOL, (b, t, ell)
    say("  top-k:", rep)


@pytest.mark.parametrize("R,N,K,finite", [(3, 300, 64, 20), (2, 40000, 96, 50), (4, 5000, 128, 0)])
def test_topk_takes_minus_inf_positions_when_few_scores_are_finite(R, N, K, finite):
    # fewer finite scores than K: every finite one is selected, then -inf
    # positions by the lower-position tie-break (scores compare as reals)
    from fp4_kv_cache_score_amd import _lib as C
    say("case: top-k with -inf ties R=%d N=%d K=%d finite=%d" % (R, N, K, finite))
    rng = np.random.default_rng(N + K)
    s = np.full((R, N), -np.inf, np.float32)
    for r in range(R):
        s[r, rng.choice(N, finite, replace=False)] = rng.random(finite, dtype=np.float32)
    nb = C.csa2_workspace_bytes(C.CSA2_OP_TOPK, R, 1, N, K, 0, 0, 0)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((R, K), dtype=torch.int32, device="cuda")
    C.csa2_topk(torch.from_numpy(s).cuda(), R, N, None, None, K, out, ws, nb)
    torch.cuda.synchronize()
    for r in range(R):
        want, _ = O.topk(s[r].astype(np.float64), K)
        assert np.array_equal(out[r].cpu().numpy(), want), r
