"""GPU parity of each C-ABI stage against the CPU oracle (needs an MI355X).

Covers: FP4 / FP8 dequantisation bit-exact through attention with one key;
indexer scores within the fp32 bound (flat, candidate pool, causal Q > 1,
ragged tails); Top-K exact on the GPU's own scores (ties, n_valid, candidate
maps, multi-segment rows, candidate-slot overflow); attention and the window
merge within 2e-3.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import csa2 as O
from oracle import formats as F
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
    _lib.lib()   # must load: no fallback exists
    yield


def _case(**kw):
    cfg = CONFIGS[0].scaled(name="t", **kw)
    return synth.make_case(cfg)


# --------------------------------------------------------------------------- dequant

def test_fp4_dequant_bit_exact_through_single_key_attention():
    from fp4_kv_cache_score_amd.device import DeviceCase
    say("case: fp4 dequant, M=512 all codes, scale codes 0..200")
    cfg = CONFIGS[0].scaled(name="deq", B=1, M=512, K=1, Q=513, W=0, modes=(FULL,))
    case = synth.make_case(cfg)
    rng = np.random.default_rng(0)
    case.pool.latent[:] = rng.integers(0, 256, size=case.pool.latent.shape, dtype=np.uint16)
    # codes 0..200: the subnormal range and beyond, while every logit stays finite
    case.pool.scale[:] = (np.arange(512 * 16).reshape(1, 512, 16) % 201).astype(np.uint8)
    dc = DeviceCase(case)
    idx = torch.arange(513, dtype=torch.int32, device="cuda").view(1, 513, 1).clone()
    idx[0, 512, 0] = -1
    o, lse = dc.sparse_attn(0, idx)
    torch.cuda.synchronize()
    o = o.cpu().numpy()
    lse = lse.cpu().numpy()
    want = F.dequant_latent(case.pool.latent[0], case.pool.scale[0])    # [512][512]
    assert np.array_equal(o[0, :512], np.broadcast_to(want[:, None, :], (512, 16, 512)))
    assert np.all(o[0, 512] == 0) and np.all(lse[0, 512] == -np.inf)
    q = F.bf16_value(case.layers[0].q[0, :512])                          # [512][16][512]
    z = np.einsum("thd,td->th", q, want)
    mag = np.einsum("thd,td->th", np.abs(q), np.abs(want))
    # any fp32 summation order of 512 exact products: |err| <= 512 * 2^-24 * sum |q c|
    assert np.all(np.abs(lse[0, :512] - z) <= 512 * 2.0 ** -24 * mag + 1e-30)


@pytest.mark.parametrize("gap", [23, 40, 80])
@pytest.mark.parametrize("big", [0, 40])
def test_sparse_attn_block_scale_spread(big, gap):
    """Entry `big` has block 0 at scale code 120 + gap while every other entry
    sits at 120, and q makes its logit hugely negative (weight ~0), so the
    output's block-0 dims come only from values `gap` binades below the
    largest scale in the same step (big = 0) or in the other split (big = 40,
    the second 32-key step).  The keys enter the products as bf16 with their
    true scale, so no spread of legal scale codes loses bits."""
    from fp4_kv_cache_score_amd.device import DeviceCase
    say("case: sparse attention, block scales %d binades apart, big entry %d" % (gap, big))
    cfg = CONFIGS[0].scaled(name="spread", B=1, M=64, K=64, W=0, modes=(FULL,))
    case = synth.make_case(cfg)
    rng = np.random.default_rng(23)
    case.pool.latent[:] = rng.integers(0, 256, size=case.pool.latent.shape, dtype=np.uint16)
    case.pool.scale[:] = 120
    case.pool.scale[0, big, 0] = 120 + gap
    cb = F.dequant_latent(case.pool.latent[0, big:big + 1], case.pool.scale[0, big:big + 1])[0, :32]
    q = case.layers[0].q                       # bf16 bits [1][1][16][512]
    q[0, 0, :, :32] = np.where(cb > 0, 0xBA80, np.where(cb < 0, 0x3A80, 0)).astype(np.uint16)
    dc = DeviceCase(case)
    idx = torch.arange(64, dtype=torch.int32, device="cuda").view(1, 1, 64)
    o, lse = dc.sparse_attn(0, idx)
    torch.cuda.synchronize()
    keys = O.gather_keys(case.pool.latent[0], case.pool.scale[0], np.arange(64))
    wo, wl = O.attend(q[0, 0], keys)
    assert np.abs(wo[:, :32]).max() > 0.1 * np.abs(wo).max()    # block 0 carries the output
    err = attn_rel_err(o[0, 0].cpu().numpy(), wo)
    say("  rel err %.3g" % err)
    assert err < ATTN_TOL
    assert np.allclose(lse[0, 0].cpu().numpy(), wl, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("gap", [40, 80])
def test_decode_step_block_scale_spread(gap):
    """The same spread inside a whole decode step (csa2_decode_layers: scan,
    Top-K of 512 among 2048 entries, attention in several splits per row).
    One entry of every sequence holds block 0 at code 125 + gap and an index
    key equal to the indexer query (so it is selected), and q gives it a
    hugely negative logit; every other entry has block 0 at 125 (about the
    size of the other blocks), and the attention weight sits on them."""
    from fp4_kv_cache_score_amd.device import DeviceCase
    say("case: decode step, block scales %d binades apart" % gap)
    cfg = CONFIGS[0].scaled(name="spread_step", B=4, M=2048, K=512, W=0, modes=(FULL, REUSE))
    case = synth.make_case(cfg)
    p = case.pool
    p.scale[:, :, 0] = 125
    bigs = [37 + 100 * b for b in range(cfg.B)]
    for b, big in enumerate(bigs):
        p.scale[b, big, 0] = 125 + gap
        p.idx_key[b, big] = case.layers[0].q_idx[b, 0]
        cb = F.dequant_latent(p.latent[b, big:big + 1], p.scale[b, big:big + 1])[0, :32]
        for L in case.layers:
            L.q[b, 0, :, :32] = np.where(cb > 0, 0xBA80, np.where(cb < 0, 0x3A80, 0)).astype(np.uint16)
    dc = DeviceCase(case)
    dc.prepare_decode()
    dc.decode_layers()
    torch.cuda.synchronize()
    res = dc.results()
    worst = 0.0
    for ell, L in enumerate(case.layers):
        for b, big in enumerate(bigs):
            g_idx = res[ell]["idx"][b, 0]
            assert big in g_idx
            keys = O.gather_keys(p.latent[b], p.scale[b], g_idx)
            wo, wl = O.attend(L.q[b, 0], keys)
            # block 0 carries a share well above the tolerance: losing it would fail
            assert np.abs(wo[:, :32]).max() > 5 * ATTN_TOL * np.abs(wo).max()
            err = attn_rel_err(res[ell]["o"][b, 0], wo)
            worst = max(worst, err)
            assert err < ATTN_TOL, "layer %d seq %d err %g" % (ell, b, err)
            assert np.allclose(res[ell]["lse"][b, 0], wl, rtol=1e-5, atol=1e-5)
    say("  worst rel err %.3g" % worst)


def test_fp8_window_rows_bit_exact_and_merge():
    from fp4_kv_cache_score_amd.device import DeviceCase
    say("case: fp8 window, W=1 exact; W=128 merge vs oracle")
    cfg = CONFIGS[0].scaled(name="swa1", B=2, M=64, K=1, Q=40, W=1, modes=(FULL,))
    case = synth.make_case(cfg)
    rng = np.random.default_rng(1)
    b = rng.integers(0, 256, size=case.layers[0].swa.shape, dtype=np.uint16).astype(np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x7E
    case.layers[0].swa[:] = b
    dc = DeviceCase(case)
    o = torch.zeros((2, 40, 16, 512), dtype=torch.float32, device="cuda")
    lse = torch.full((2, 40, 16), -float("inf"), dtype=torch.float32, device="cuda")
    dc.swa_merge(0, o, lse)
    torch.cuda.synchronize()
    want = F.e4m3_value(b)                                              # [2][40][512]
    assert np.array_equal(o.cpu().numpy(), np.broadcast_to(want[:, :, None, :], (2, 40, 16, 512)))

    cfg = CONFIGS[0].scaled(name="swa", B=3, M=64, K=1, Q=5, W=128, modes=(FULL,))
    case = synth.make_case(cfg)
    dc = DeviceCase(case)
    o_in = rng.standard_normal((3, 5, 16, 512)).astype(np.float32)
    lse_in = (rng.standard_normal((3, 5, 16)) * 3).astype(np.float32)
    lse_in[0, 0, :4] = -np.inf
    o = torch.from_numpy(o_in.copy()).cuda()
    lse = torch.from_numpy(lse_in.copy()).cuda()
    dc.swa_merge(0, o, lse)
    torch.cuda.synchronize()
    go, gl = o.cpu().numpy(), lse.cpu().numpy()
    for bb in range(3):
        for t in range(5):
            wo, wl = O.swa_merge(case.layers[0].q[bb, t], case.layers[0].swa[bb, t:t + 128],
                                 o_in[bb, t], lse_in[bb, t])
            assert attn_rel_err(go[bb, t], wo) < ATTN_TOL
            assert np.allclose(gl[bb, t], wl, rtol=1e-5, atol=1e-5)


# --------------------------------------------------------------------------- scores

@pytest.mark.parametrize("B,M", [(1, 1024), (2, 3001), (3, 513)])
def test_index_scores_within_fp32_bound_flat(B, M):
    from fp4_kv_cache_score_amd.device import DeviceCase
    say("case: scores flat B=%d M=%d" % (B, M))
    case = _case(B=B, M=M)
    dc = DeviceCase(case)
    s = dc.index_scores(0).cpu().numpy()                  # [B][1][M]
    L = case.layers[0]
    for b in range(B):
        ex = O.index_scores(case.pool.idx_key[b], L.q_idx[b, 0], L.w_idx[b, 0])
        bound = score_bound(case.pool.idx_key[b], L.q_idx[b, 0], L.w_idx[b, 0], ex)
        assert np.all(np.abs(s[b, 0].astype(np.float64) - ex) <= bound)
        assert not np.signbit(s[b, 0]).any()


def test_index_scores_candidate_pool_and_padding():
    from fp4_kv_cache_score_amd.device import DeviceCase
    say("case: scores over candidate pool with -1 padding")
    case = _case(B=2, M=5000)
    dc = DeviceCase(case)
    rng = np.random.default_rng(3)
    P = 1500
    cand = np.full((2, P), -1, np.int32)
    for b, nv in enumerate((1500, 1111)):
        cand[b, :nv] = np.sort(rng.choice(5000, nv, replace=False))
    s = dc.index_scores(0, cand=torch.from_numpy(cand).cuda(), P=P).cpu().numpy()
    L = case.layers[0]
    for b, nv in enumerate((1500, 1111)):
        ex = O.index_scores(case.pool.idx_key[b], L.q_idx[b, 0], L.w_idx[b, 0], rows=cand[b, :nv])
        bound = score_bound(case.pool.idx_key[b], L.q_idx[b, 0], L.w_idx[b, 0], ex, rows=cand[b, :nv])
        assert np.all(np.abs(s[b, 0, :nv] - ex) <= bound)
        assert np.all(s[b, 0, nv:] == -np.inf)


def test_index_scores_causal_multi_query():
    from fp4_kv_cache_score_amd.device import DeviceCase
    say("case: scores causal Q=37 M=700")
    cfg = CONFIGS[4].scaled(name="pf", M=700, Q=37, K=16, W=8)
    case = synth.make_case(cfg)
    dc = DeviceCase(case)
    s = dc.index_scores(0).cpu().numpy()                  # [1][37][700]
    L = case.layers[0]
    for t in range(37):
        vis = O.visible_entries(700, cfg.pos0 + t, 4)
        ex = O.index_scores(case.pool.idx_key[0], L.q_idx[0, t], L.w_idx[0, t], rows=np.arange(vis))
        bound = score_bound(case.pool.idx_key[0], L.q_idx[0, t], L.w_idx[0, t], ex, rows=np.arange(vis))
        assert np.all(np.abs(s[0, t, :vis] - ex) <= bound)
        assert np.all(s[0, t, vis:] == -np.inf)


# --------------------------------------------------------------------------- top-k

def _gpu_topk(scores_np, K, n_valid=None, cand=None):
    from fp4_kv_cache_score_amd import _lib as C
    R, N = scores_np.shape
    s = torch.from_numpy(np.ascontiguousarray(scores_np, np.float32)).cuda()
    nb = C.csa2_workspace_bytes(C.CSA2_OP_TOPK, R, 1, N, K, 0, 0, 0)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    idx = torch.empty((R, K), dtype=torch.int32, device="cuda")
    nv = None if n_valid is None else torch.from_numpy(np.asarray(n_valid, np.int32)).cuda()
    cd = None if cand is None else torch.from_numpy(np.asarray(cand, np.int32)).cuda()
    C.csa2_topk(s, R, N, nv, cd, K, idx, ws, nb)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


def _oracle_rows(scores_np, K, n_valid=None, cand=None):
    out = []
    for r in range(scores_np.shape[0]):
        nv = None if n_valid is None else n_valid[r]
        pos, _ = O.topk(scores_np[r].astype(np.float64), K, n_valid=nv)
        out.append(pos if cand is None else O.map_positions(pos, cand[r]))
    return np.stack(out)


@pytest.mark.parametrize("R,N,K,kind", [
    (1, 1, 1, "cont"), (3, 7, 3, "ties"), (5, 100, 100, "cont"), (4, 100, 150, "ties"),
    (8, 4097, 64, "ties"), (6, 33333, 512, "cont"), (6, 40960, 512, "cont"), (2, 33000, 64, "ties"),
    (2, 9000, 8192, "cont"),
    (3, 300001, 512, "cont"), (2, 300001, 8192, "ties"), (64, 4096, 1, "ties"),
    (16, 2000, 77, "zeros"), (4, 5000, 300, "negzero")])
def test_topk_exact_vs_oracle(R, N, K, kind):
    say("case: topk R=%d N=%d K=%d %s" % (R, N, K, kind))
    rng = np.random.default_rng(R * 7 + N + K)
    if kind == "cont":
        s = (rng.standard_normal((R, N)) ** 2).astype(np.float32)
    elif kind == "ties":
        s = rng.integers(0, 40, size=(R, N)).astype(np.float32) * np.float32(0.25)
    elif kind == "zeros":
        s = np.zeros((R, N), np.float32)
        s[:, ::97] = 1.0
    else:
        s = rng.integers(-2, 3, size=(R, N)).astype(np.float32)
        s[s == 0] = -0.0
        s[:, ::2] = np.where(s[:, ::2] == -0.0, 0.0, s[:, ::2])
    g = _gpu_topk(s, K)
    assert np.array_equal(g, _oracle_rows(s, K))


def test_topk_n_valid_and_candidate_map():
    say("case: topk with n_valid and cand map")
    rng = np.random.default_rng(11)
    R, N, K = 7, 6000, 200
    s = rng.integers(0, 1000, size=(R, N)).astype(np.float32)
    nv = np.array([0, 1, 199, 200, 201, 5999, 6000], np.int32)
    cand = np.stack([np.sort(rng.choice(10 ** 6, N, replace=False)) for _ in range(R)]).astype(np.int32)
    g = _gpu_topk(s, K, n_valid=nv, cand=cand)
    assert np.array_equal(g, _oracle_rows(s, K, n_valid=nv, cand=cand))


def test_topk_candidate_slot_overflow_path():
    say("case: topk overflow R=2048 N=16500")
    R, N, K = 2048, 16500, 100
    s = np.zeros((R, N), np.float32)             # one bin holds every position
    s[1::2, 7::11] = 2.0
    g = _gpu_topk(s, K)
    assert np.array_equal(g, _oracle_rows(s, K))


@pytest.mark.parametrize("N,K,kind", [
    (65536, 512, "cont"), (40000, 1, "cont"), (262144, 512, "cont"), (65536, 512, "sorted"),
    (65536, 300, "ties"), (65536, 512, "const"), (65536, 513, "cont"), (50000, 64, "mixed")])
def test_topk_streamed_rows_sampled_bound(N, K, kind):
    """256 rows longer than 32768 take the one-work-group select that streams
    its row from memory (a histogram pass, then a collection pass): continuous,
    sorted, tied and constant rows, K around 512, valid counts around 32768
    and an unaligned tail."""
    R = 256
    say("case: topk streamed rows R=%d N=%d K=%d %s" % (R, N, K, kind))
    rng = np.random.default_rng(N + K)
    nv = None
    if kind == "cont":
        s = (rng.standard_normal((R, N)) ** 2).astype(np.float32)
    elif kind == "sorted":
        s = np.sort(rng.random((R, N), dtype=np.float32), axis=1)
        s[1::2] = s[1::2, ::-1]
    elif kind == "ties":
        s = rng.integers(0, 40, size=(R, N)).astype(np.float32) * np.float32(0.25)
    elif kind == "const":
        s = np.full((R, N), 0.5, np.float32)
        s[::3, ::5000] = 1.0
    else:   # valid counts around the sampling threshold and an unaligned tail
        s = rng.random((R, N), dtype=np.float32)
        nv = rng.integers(30000, N + 1, size=R).astype(np.int32)
        nv[:4] = [32767, 32768, 32769, N]
    g = _gpu_topk(s, K, n_valid=nv)
    assert np.array_equal(g, _oracle_rows(s, K, n_valid=nv))


@pytest.mark.parametrize("K", [512, 8192])
def test_topk_multi_group_bin_overflow(K):
    """Rows longer than 2^18 go to the several-work-groups-per-row select; at
    140 rows each row has fewer candidate slots than positions, so a row whose
    threshold bin holds (nearly) every position takes the finish step's
    re-scan of the row.  Rows: constant; zeros with a spike every 1000
    positions; three values; continuous."""
    R, N = 140, 262145
    say("case: topk multi-group overflow R=%d N=%d K=%d" % (R, N, K))
    rng = np.random.default_rng(K)
    s = np.full((R, N), 0.25, np.float32)
    for r in range(R):
        if r % 4 == 1:
            s[r] = 0.0
            s[r, ::1000] = 1.0
        elif r % 4 == 2:
            s[r] = rng.integers(0, 3, N).astype(np.float32)
        elif r % 4 == 3:
            s[r] = rng.random(N, dtype=np.float32)
    g = _gpu_topk(s, K)
    assert np.array_equal(g[0], np.arange(K, dtype=np.int32))
    assert np.array_equal(g, _oracle_rows(s, K))


# --------------------------------------------------------------------------- attention

def test_sparse_attn_dense_and_random_selection():
    from fp4_kv_cache_score_amd.device import DeviceCase
    say("case: sparse attention K=M dense and random K with -1")
    case = _case(B=2, M=1024, K=1024)
    dc = DeviceCase(case)
    idx = torch.arange(1024, dtype=torch.int32, device="cuda").repeat(2, 1).view(2, 1, 1024)
    o, lse = dc.sparse_attn(0, idx)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    for b in range(2):
        dense = F.dequant_latent(case.pool.latent[b], case.pool.scale[b])
        wo, wl = O.attend(case.layers[0].q[b, 0], dense)
        assert attn_rel_err(o[b, 0], wo) < ATTN_TOL
        assert np.allclose(lse[b, 0], wl, rtol=1e-5, atol=1e-5)
    rng = np.random.default_rng(4)
    K = 77
    sel = np.full((2, 1, K), -1, np.int32)
    sel[0, 0, :60] = np.sort(rng.choice(1024, 60, replace=False))
    sel[1, 0, :] = np.sort(rng.choice(1024, K, replace=False))
    o, lse = dc.sparse_attn(0, torch.from_numpy(sel).cuda())
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    for b in range(2):
        keys = O.gather_keys(case.pool.latent[b], case.pool.scale[b], sel[b, 0])
        wo, wl = O.attend(case.layers[0].q[b, 0], keys)
        assert attn_rel_err(o[b, 0], wo) < ATTN_TOL
        assert np.allclose(lse[b, 0], wl, rtol=1e-5, atol=1e-5)
