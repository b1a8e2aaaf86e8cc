"""GPU parity at the sizes the ABI allows at most, and past the points where
the kernels change how they hold things:

* the decode step with K = 4096 and K = 16384 (the limit; beyond the entry
  numbers a work-group keeps on chip) and windows of 300 and 4096 rows (the
  limit; not multiples of a key chunk);
* chunked prefill through the schedule with K = 1500 and W = 300;
* Top-K with K = 16384 on rows of 40000 (several work-groups per row) and
  of 20000 (one).

Top-K exact except near ties (counted), attention within 2e-3 on the GPU's
own selection, as in the other parity tests.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import csa2 as O
from fp4_kv_cache_score_amd import synth
from fp4_kv_cache_score_amd.configs import CONFIGS, FULL, REINDEX, REUSE
from parity import ATTN_TOL, TieReport, attn_rel_err

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


@pytest.mark.parametrize("B,M,K,W", [(2, 20000, 4096, 300), (1, 40000, 16384, 4096)])
def test_decode_large_k_and_window(B, M, K, W):
    from fp4_kv_cache_score_amd.device import DeviceCase
    say("case: decode limits B=%d M=%d K=%d W=%d" % (B, M, K, W))
    cfg = CONFIGS[1].scaled(name="lim", seed=90 + B, B=B, M=M, K=K, W=W,
                            modes=(FULL, REINDEX, REUSE))
    case = synth.make_case(cfg)
    dc = DeviceCase(case)
    dc.prepare_decode()
    dc.decode_layers()
    torch.cuda.synchronize()
    res = dc.results()
    rep = TieReport()
    worst = 0.0
    p = case.pool
    for b in range(B):
        layers = [dict(mode=L.mode,
                       q_idx=None if L.q_idx is None else L.q_idx[b, 0],
                       w_idx=None if L.w_idx is None else L.w_idx[b, 0],
                       q=L.q[b, 0], swa=L.swa[b]) for L in case.layers]
        want = O.decode_sequence(p.latent[b], p.scale[b], p.idx_key[b], layers, K)
        for ell, (w, g) in enumerate(zip(want, res)):
            gi = g["idx"][b, 0]
            if w["mode"] != REUSE:
                rep.check(gi, w["idx"], w.get("gap"), "b=%d layer %d" % (b, ell))
            keys = O.gather_keys(p.latent[b], p.scale[b], gi, layers[ell]["swa"])
            wo, wl = O.attend(layers[ell]["q"], keys)
            err = attn_rel_err(g["o"][b, 0], wo)
            worst = max(worst, err)
            assert err < ATTN_TOL, (b, ell, err)
            assert np.allclose(g["lse"][b, 0], wl, rtol=1e-5, atol=1e-5), (b, ell)
    say("  top-k:", rep, " worst attention rel err %.3g" % worst)


def test_prefill_layers_large_k_and_window():
    from fp4_kv_cache_score_amd.device import DeviceCase
    K, W, Q = 1500, 300, 70
    say("case: prefill limits Q=%d K=%d W=%d" % (Q, K, W))
    cfg = CONFIGS[4].scaled(name="plim", seed=95, B=1, Q=Q, M=6000, K=K, W=W,
                            modes=(FULL, REUSE), chunk_pos=4 * 6000 - Q)
    case = synth.make_case(cfg)
    dc = DeviceCase(case)
    dc.prefill_layers()
    torch.cuda.synchronize()
    p = case.pool
    rep = TieReport()
    gi = dc.layers[0]["idx"][0].cpu().numpy()
    go = [d["o"][0].cpu().numpy() for d in dc.layers]
    L = case.layers
    for t in range(0, Q, 5):
        lay = [dict(mode=X.mode, q_idx=None if X.q_idx is None else X.q_idx[0, t:t + 1],
                    w_idx=None if X.w_idx is None else X.w_idx[0, t:t + 1],
                    q=X.q[0, t:t + 1], swa=X.swa[0, t:t + W]) for X in L]
        recs = O.prefill_layers(p.latent[0], p.scale[0], p.idx_key[0], lay, 1, cfg.pos0 + t,
                                cfg.ratio, K, W)
        rep.check(gi[t], recs[0]["idx"][0], recs[0]["gap"][0], "t=%d" % t)
        for ell in range(2):
            keys = O.gather_keys(p.latent[0], p.scale[0], gi[t], L[ell].swa[0, t:t + W])
            wo, _ = O.attend(L[ell].q[0, t], keys)
            assert attn_rel_err(go[ell][t], wo) < ATTN_TOL, (t, ell)
    say("  top-k:", rep)


@pytest.mark.parametrize("R,N", [(2, 40000), (3, 20000)])
def test_topk_largest_k(R, N):
    from fp4_kv_cache_score_amd import _lib as C
    K = 16384
    say("case: top-k K=%d R=%d N=%d" % (K, R, N))
    rng = np.random.default_rng(N)
    s = rng.random((R, N), dtype=np.float32)
    s[:, ::7] = s[:, 3:4]                     # ties straddling the boundary
    nb = C.csa2_workspace_bytes(C.CSA2_OP_TOPK, R, 1, N, K, 0, 0, 0)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((R, K), dtype=torch.int32, device="cuda")
    C.csa2_topk(torch.from_numpy(s).cuda(), R, N, None, None, K, out, ws, nb)
    torch.cuda.synchronize()
    for r in range(R):
        want, _ = O.topk(s[r].astype(np.float64), K)
        assert np.array_equal(out[r].cpu().numpy(), want), r
