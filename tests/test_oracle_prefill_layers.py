"""Pins of the oracle's chunked prefill through the layer schedule (CPU only).

Closed forms at the start of a context: the first token attends to its own
window row alone (o = that row, lse = q . row), a token that sees fewer than K
pool entries selects all of them, and no token sees a window row before
position 0.  Brute-force causality: changing a pool entry or a window row
changes exactly the tokens that can see it.  Invariants: a chunk split in two
(the second starting where the first ends) gives the same results as one
chunk, Q = 1 with no causal limit reproduces the decode schedule, and a Reuse
layer takes its source layer's indices token by token.
"""
import numpy as np
import pytest

from oracle import csa2 as O
from oracle import formats as F
from fp4_kv_cache_score_amd import synth
from fp4_kv_cache_score_amd.configs import CONFIGS, FULL, REINDEX, REUSE


def _case(M=64, K=8, W=8, Q=24, pos0=0, modes=(FULL,), seed=5, ratio=4):
    cfg = CONFIGS[0].scaled(name="pf", seed=seed, B=1, M=M, K=K, W=W, Q=Q, modes=tuple(modes),
                            causal=True, chunk_pos=pos0, ratio=ratio)
    return synth.make_case(cfg)


def _layers(case, t0=0, t1=None, W=None):
    """Per-layer inputs of tokens t0 .. t1-1 (window buffer rows t0 .. t1-1+W-1)."""
    cfg = case.cfg
    t1 = cfg.Q if t1 is None else t1
    W = cfg.W if W is None else W
    out = []
    for L in case.layers:
        out.append(dict(mode=L.mode,
                        q_idx=None if L.q_idx is None else L.q_idx[0, t0:t1],
                        w_idx=None if L.w_idx is None else L.w_idx[0, t0:t1],
                        q=L.q[0, t0:t1], swa=L.swa[0, t0:t1 + W - 1]))
    return out


def _run(case, pool=None, layers=None, Q=None, pos0=None):
    cfg = case.cfg
    p = case.pool if pool is None else pool
    return O.prefill_layers(p.latent[0], p.scale[0], p.idx_key[0],
                            _layers(case) if layers is None else layers,
                            cfg.Q if Q is None else Q, cfg.pos0 if pos0 is None else pos0,
                            cfg.ratio, cfg.K, cfg.W)


def test_first_token_attends_to_its_own_window_row_only():
    case = _case(W=8, pos0=0)
    rec = _run(case)[0]
    L = case.layers[0]
    row = F.e4m3_value(L.swa[0, 7])                 # token 0's own row: t + W - 1
    q = F.bf16_value(L.q[0, 0])
    assert rec["vis"][0] == 0 and (rec["idx"][0] == -1).all()
    for h in range(q.shape[0]):
        assert np.array_equal(rec["o"][0, h], row)
        z = sum(float(a) * float(b) for a, b in zip(q[h], row))
        assert abs(rec["lse"][0, h] - z) <= 1e-12 * max(1.0, abs(z))


def test_second_token_sees_two_window_rows():
    case = _case(W=8, pos0=0)
    rec = _run(case)[0]
    L = case.layers[0]
    k = F.e4m3_value(L.swa[0, 7:9])                 # positions 0 and 1
    q = F.bf16_value(L.q[0, 1])
    z = q @ k.T
    m = z.max(1, keepdims=True)
    e = np.exp(z - m)
    want = (e[:, :1] * k[0] + e[:, 1:] * k[1]) / e.sum(1, keepdims=True)
    assert np.allclose(rec["o"][1], want, rtol=1e-13, atol=1e-15)


def test_tokens_seeing_fewer_than_k_entries_select_all_of_them():
    case = _case(M=64, K=8, Q=48, pos0=0, ratio=4)
    rec = _run(case)[0]
    for t in range(48):
        vis = (t + 1) // 4
        assert rec["vis"][t] == vis
        if vis <= 8:
            assert rec["idx"][t].tolist() == list(range(vis)) + [-1] * (8 - vis), t
        else:
            sel = rec["idx"][t]
            assert (sel >= 0).all() and sel.max() < vis and (np.diff(sel) > 0).all(), t


def test_window_rows_before_position_zero_are_never_used():
    case = _case(W=16, Q=20, pos0=3)
    base = _run(case)
    case.layers[0].swa[0, :12] ^= 0x11               # rows of positions -12 .. -1
    again = _run(case)
    assert np.array_equal(base[0]["o"], again[0]["o"])
    assert np.array_equal(base[0]["lse"], again[0]["lse"])


def test_causality_pool_entry_brute_force():
    # K above every token's visible count: each token selects all it can see
    case = _case(M=40, K=32, Q=40, pos0=60, ratio=4, W=4)
    base = _run(case)[0]
    e = 20                                            # visible from position 83 = token 23
    pool = synth.HostPool(case.pool.latent.copy(), case.pool.scale.copy(),
                          case.pool.idx_key.copy(), case.pool.planted)
    pool.idx_key[0, e] ^= 0x01
    pool.latent[0, e] ^= 0x22
    pert = _run(case, pool=pool)[0]
    for t in range(40):
        same = np.array_equal(base["o"][t], pert["o"][t])
        if 60 + t < 4 * e + 3:
            assert same and np.array_equal(base["idx"][t], pert["idx"][t]), t
        else:
            assert e in pert["idx"][t] and not same, t


def test_causality_window_row_brute_force():
    W, Q = 8, 30
    case = _case(W=W, Q=Q, pos0=100)
    base = _run(case)[0]
    r = 15                                            # buffer row 15 = position 100 - 7 + 15
    case.layers[0].swa[0, r] ^= 0x08
    pert = _run(case)[0]
    for t in range(Q):
        same = np.array_equal(base["o"][t], pert["o"][t])
        assert same == (not (t <= r <= t + W - 1)), t


@pytest.mark.parametrize("pos0,split", [(0, 9), (37, 16)])
def test_chunk_split_matches_one_chunk(pos0, split):
    W, Q = 8, 32
    case = _case(M=48, K=6, W=W, Q=Q, pos0=pos0, modes=(FULL, REINDEX, REUSE))
    whole = _run(case)
    a = _run(case, layers=_layers(case, 0, split), Q=split, pos0=pos0)
    b = _run(case, layers=_layers(case, split, Q), Q=Q - split, pos0=pos0 + split)
    for ell in range(3):
        for key in ("idx", "o", "lse"):
            got = np.concatenate([a[ell][key], b[ell][key]])
            assert np.array_equal(got, whole[ell][key]), (ell, key)


def test_single_token_without_causal_limit_is_the_decode_schedule():
    cfg = CONFIGS[0].scaled(name="d", seed=8, B=1, M=96, K=8, W=8, modes=(FULL, REINDEX, REUSE))
    case = synth.make_case(cfg)
    p = case.pool
    dec = O.decode_sequence(p.latent[0], p.scale[0], p.idx_key[0],
                            [dict(mode=L.mode,
                                  q_idx=None if L.q_idx is None else L.q_idx[0, 0],
                                  w_idx=None if L.w_idx is None else L.w_idx[0, 0],
                                  q=L.q[0, 0], swa=L.swa[0]) for L in case.layers], K=8)
    pf = O.prefill_layers(p.latent[0], p.scale[0], p.idx_key[0],
                          [dict(mode=L.mode, q_idx=None if L.q_idx is None else L.q_idx[0],
                                w_idx=None if L.w_idx is None else L.w_idx[0],
                                q=L.q[0], swa=L.swa[0]) for L in case.layers],
                          Q=1, pos0=-1, ratio=4, K=8, W=8)
    for d, r in zip(dec, pf):
        assert np.array_equal(d["idx"], r["idx"][0])
        assert np.array_equal(d["o"], r["o"][0]) and np.array_equal(d["lse"], r["lse"][0])


def test_reuse_takes_the_source_indices_token_by_token():
    case = _case(M=64, K=6, Q=40, pos0=50, modes=(FULL, REUSE, REINDEX, REUSE))
    recs = _run(case)
    assert np.array_equal(recs[1]["idx"], recs[0]["idx"])
    assert np.array_equal(recs[3]["idx"], recs[2]["idx"])
    assert not np.array_equal(recs[2]["idx"], recs[0]["idx"])
    with pytest.raises(ValueError):
        _run(_case(modes=(REUSE,)))
