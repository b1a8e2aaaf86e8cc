"""GPU parity of csa2_prefill_layers (chunked prefill through the layer schedule).

Every layer of a Full / Reindex / Reuse schedule runs over a chunk of Q tokens
in one call: matrix-core scores of the entries the chunk can see, Top-K per
token within its visible count, and one attention pass per token over its
selected FP4 entries and its FP8 window rows.  Checked against the oracle's
prefill schedule:
* Top-K exact per token and layer (near ties counted, as elsewhere), Reuse
  layers equal to their source layer's indices;
* attention within 2e-3 of the oracle on the GPU's own selection, including
  tokens that see no pool entry and window rows before position 0;
* one chunk at several positions (the first chunk of a context, a chunk
  where tokens cross K visible entries, Q = 1 without causal limit, ragged
  query tiles), a whole context prefilled chunk by chunk into a pool that
  grows by csa2_pool_append (ragged chunk sizes, Q = 1 among them) with the
  pool bit-exact against the oracle's write side at the end, and the
  2048-token / 65536-entry shape at sampled tokens.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import csa2 as O
from oracle import write_side as WS
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


def _check_token(p, layers, got, b, t, pos0, ratio, K, W, rep, tag=""):
    """One token of sequence b through the oracle schedule, against the GPU's
    per-layer (idx, o, lse) arrays got[l] (each [Q][...] of sequence b).
    layers: host inputs with [B][Q]... arrays.  Returns the worst attention error."""
    lay = [dict(mode=L["mode"],
                q_idx=None if L["q_idx"] is None else L["q_idx"][b, t:t + 1],
                w_idx=None if L["w_idx"] is None else L["w_idx"][b, t:t + 1],
                q=L["q"][b, t:t + 1], swa=L["swa"][b, t:t + W]) for L in layers]
    recs = O.prefill_layers(p[0][b], p[1][b], p[2][b], lay, 1, pos0 + t if pos0 >= 0 else -1,
                            ratio, K, W)
    r0 = O.window_first_row(t, W, pos0)
    worst = 0.0
    src = None
    for ell, (L, rec) in enumerate(zip(layers, recs)):
        gi, go, gl = got[ell]
        where = "%s b=%d t=%d layer %d" % (tag, b, t, ell)
        if L["mode"] == REUSE:
            assert np.array_equal(gi[t], got[src][0][t]), where
        else:
            rep.check(gi[t], rec["idx"][0], rec["gap"][0], where)
            src = ell
        keys = O.gather_keys(p[0][b], p[1][b], gi[t], L["swa"][b, t + r0:t + W])
        wo, wl = O.attend(L["q"][b, t], keys)
        err = attn_rel_err(go[t], wo)
        worst = max(worst, err)
        assert err < ATTN_TOL, (where, err)
        assert np.allclose(gl[t], wl, rtol=1e-5, atol=1e-5), where
    return worst


def _host_layers(case):
    return [dict(mode=L.mode, q_idx=L.q_idx, w_idx=L.w_idx, q=L.q, swa=L.swa)
            for L in case.layers]


def _got(dc, b):
    return [(d["idx"][b].cpu().numpy(), d["o"][b].cpu().numpy(), d["lse"][b].cpu().numpy())
            for d in dc.layers]


@pytest.mark.parametrize("B,Q,M,K,W,pos0", [
    (2, 200, 1000, 64, 64, 150),      # tokens cross K visible entries
    (1, 300, 4096, 64, 128, 0),       # first chunk: no entry at first, window rows before 0
    (2, 3, 64, 8, 4, 0),              # no entry visible to any token of the chunk
    (1, 2, 64, 8, 0, 0),              # and no window: empty key set
    (2, 1, 600, 32, 16, -1),          # one token, no causal limit (the decode shape)
    (1, 129, 2051, 100, 33, 9000),    # ragged tiles, every entry visible, M not a multiple of 4
])
def test_prefill_layers_one_chunk(B, Q, M, K, W, pos0):
    from fp4_kv_cache_score_amd.device import DeviceCase
    modes = (FULL, REINDEX, REUSE, REUSE)
    say("case: prefill layers B=%d Q=%d M=%d K=%d W=%d pos0=%d" % (B, Q, M, K, W, pos0))
    cfg = CONFIGS[4].scaled(name="pfl", seed=40 + Q, B=B, Q=Q, M=M, K=K, W=W, modes=modes,
                            causal=pos0 >= 0, chunk_pos=max(pos0, 0))
    case = synth.make_case(cfg)
    dc = DeviceCase(case)
    dc.prefill_layers()
    torch.cuda.synchronize()
    assert dc.src_layer == [0, 1, 1, 1]
    p = (case.pool.latent, case.pool.scale, case.pool.idx_key)
    rep = TieReport()
    worst = 0.0
    layers = _host_layers(case)
    for b in range(B):
        got = _got(dc, b)
        for t in range(Q):
            worst = max(worst, _check_token(p, layers, got, b, t, cfg.pos0, cfg.ratio, K, W, rep))
    say("  top-k:", rep, " worst attention rel err %.3g" % worst)


def test_prefill_layers_growing_pool_chunks():
    """A context of 1024 tokens prefilled in ragged chunks; before each chunk the
    entries it completes are appended to the pool (GPU and oracle write sides)."""
    from fp4_kv_cache_score_amd import _lib as C
    B, Mcap, ratio, K, W = 2, 256, 4, 24, 40
    ctx = ratio * Mcap
    modes = (FULL, REUSE, REINDEX)
    bounds = [0, 200, 456, 457, 700, 1024]
    say("case: growing pool B=%d ctx=%d chunks=%s" % (B, ctx, bounds))
    rng = np.random.default_rng(77)
    dev = "cuda"
    # pool storage: random (valid) codes where no entry has been written yet
    lat = rng.integers(0, 256, (B, Mcap, 256), dtype=np.uint8)
    sc = rng.integers(100, 150, (B, Mcap, 16), dtype=np.uint8)
    key = rng.integers(0, 126, (B, Mcap, 8, 64), dtype=np.uint8)
    g_lat, g_sc, g_key = (torch.from_numpy(a.copy()).to(dev) for a in (lat, sc, key))
    pool = C.make_pool(g_lat, g_sc, g_key, B, Mcap)
    x_lat = (rng.standard_normal((B, Mcap, 512)) * np.exp2(rng.integers(-3, 3, (B, Mcap, 1)))
             ).astype(np.float32)
    x_key = rng.standard_normal((B, Mcap, 8, 64)).astype(np.float32)
    # per-layer inputs of every context token; window rows indexed by position + W - 1
    layers = []
    for ell, mode in enumerate(modes):
        idx_q = mode != REUSE
        layers.append(dict(
            mode=mode,
            q_idx=synth.encode_e4m3(rng.standard_normal((B, ctx, 8, 64)).astype(np.float32))
            if idx_q else None,
            w_idx=rng.random((B, ctx, 8), dtype=np.float32) if idx_q else None,
            q=synth.encode_bf16((rng.standard_normal((B, ctx, 16, 512)) / np.sqrt(512.0))
                                .astype(np.float32)),
            swa=rng.integers(0, 126, (B, ctx + W - 1, 512), dtype=np.uint8)))
    rep = TieReport()
    worst = 0.0
    for p0, p1 in zip(bounds[:-1], bounds[1:]):
        Q = p1 - p0
        j0, j1 = p0 // ratio, p1 // ratio          # entries whose last token lies in the chunk
        T = j1 - j0
        if T > 0:
            slot = np.broadcast_to(np.arange(j0, j1, dtype=np.int32), (B, T)).copy()
            xl = np.ascontiguousarray(x_lat[:, j0:j1])
            xk = np.ascontiguousarray(x_key[:, j0:j1])
            C.csa2_pool_append(g_lat, g_sc, g_key, B, Mcap, torch.from_numpy(xl).to(dev),
                               torch.from_numpy(xk).to(dev), torch.from_numpy(slot).to(dev), T)
            lat, sc, key = WS.append_pool(lat, sc, key, xl, xk, slot)
        chunk = []
        structs = []
        for L in layers:
            d = dict(mode=L["mode"],
                     q_idx=None if L["q_idx"] is None else np.ascontiguousarray(L["q_idx"][:, p0:p1]),
                     w_idx=None if L["w_idx"] is None else np.ascontiguousarray(L["w_idx"][:, p0:p1]),
                     q=np.ascontiguousarray(L["q"][:, p0:p1]),
                     swa=np.ascontiguousarray(L["swa"][:, p0:p1 + W - 1]))
            chunk.append(d)
            t_ = {k: (None if v is None or k == "mode" else
                      torch.from_numpy(v.view(np.int16) if v.dtype == np.uint16 else v).to(dev))
                  for k, v in d.items()}
            t_["o"] = torch.empty((B, Q, 16, 512), dtype=torch.float32, device=dev)
            t_["lse"] = torch.empty((B, Q, 16), dtype=torch.float32, device=dev)
            t_["idx"] = torch.empty((B, Q, K), dtype=torch.int32, device=dev)
            d["dev"] = t_
            structs.append(C.csa2_layer(L["mode"], C._p(t_["q_idx"]), C._p(t_["w_idx"]),
                                        C._p(t_["q"]), C._p(t_["swa"]), C._p(t_["o"]),
                                        C._p(t_["lse"]), C._p(t_["idx"])))
        nb = C.csa2_workspace_bytes(C.CSA2_OP_PREFILL_LAYERS, B, Q, Mcap, K, 0, W, 16)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        say("  chunk [%d, %d): %d new entries" % (p0, p1, T))
        _, src = C.csa2_prefill_layers(pool, structs, Q, p0, ratio, 16, K, W, ws, nb)
        torch.cuda.synchronize()
        assert src == [0, 0, 2]
        for b in range(B):
            got = [(d["dev"]["idx"][b].cpu().numpy(), d["dev"]["o"][b].cpu().numpy(),
                    d["dev"]["lse"][b].cpu().numpy()) for d in chunk]
            for t in range(Q):
                worst = max(worst, _check_token((lat, sc, key), chunk, got, b, t, p0, ratio, K, W,
                                                rep, "chunk %d" % p0))
    for name, g, w in (("latent", g_lat, lat), ("scale", g_sc, sc), ("idx_key", g_key, key)):
        assert np.array_equal(g.cpu().numpy(), w), name
    say("  top-k:", rep, " worst attention rel err %.3g" % worst)


@pytest.mark.parametrize("first", [False, True])
def test_prefill_layers_full_size_sampled(first):
    from fp4_kv_cache_score_amd.device import DeviceCase
    cfg = CONFIGS[4].scaled(modes=(FULL, REINDEX, REUSE, REUSE), chunk_pos=0 if first else -1)
    say("case: prefill layers full size Q=%d M=%d pos0=%d" % (cfg.Q, cfg.M, cfg.pos0))
    case = synth.make_case(cfg)
    dc = DeviceCase(case)
    dc.prefill_layers()
    torch.cuda.synchronize()
    p = (case.pool.latent, case.pool.scale, case.pool.idx_key)
    rep = TieReport()
    got = _got(dc, 0)
    layers = _host_layers(case)
    worst = 0.0
    for t in (0, 1, 3, 4, 127, 128, 1024, 2046, 2047):
        worst = max(worst, _check_token(p, layers, got, 0, t, cfg.pos0, cfg.ratio, cfg.K, cfg.W,
                                        rep))
    say("  top-k:", rep, " worst attention rel err %.3g" % worst)
