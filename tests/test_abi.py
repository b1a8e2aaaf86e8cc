"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, sizes workspaces, and rejects bad arguments on the host
before any HIP call (so these calls never touch a device)."""
import ctypes
import os
import re

import pytest

from fp4_kv_cache_score_amd import _lib as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")

if not os.path.exists(C.LIB_PATH):
    pytest.skip("libcsa2.so not built (run python -m fp4_kv_cache_score_amd.build)",
                allow_module_level=True)

A = 0x10000   # a 16-byte-aligned fake device address: never dereferenced here
A2 = 0x20000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(C.EXPORTS)
    L = ctypes.CDLL(C.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert "gfx950" in C.csa2_version()


def test_library_resolves_its_own_symbols():
    """Every symbol of the library's own namespace is defined inside it (a
    shared library links with undefined symbols, which would only fail at the
    first call): loading with immediate binding resolves every one."""
    ctypes.CDLL(C.LIB_PATH, mode=ctypes.RTLD_GLOBAL | os.RTLD_NOW)


def test_status_strings():
    for s in range(8):
        assert C.csa2_status_string(s)
    assert C.csa2_status_string(0) == "ok"
    assert "unknown" in C.csa2_status_string(99)


def test_workspace_bytes():
    ws = C.csa2_workspace_bytes
    assert ws(C.CSA2_OP_TOPK, 32, 1, 32768, 512, 0, 0, 0) > 0
    assert ws(C.CSA2_OP_TOPK, 4, 1, 300001, 512, 0, 0, 0) > 4 * 4096 * 4
    assert ws(C.CSA2_OP_TOPK, 32, 1, 32768, 0, 0, 0, 0) == 0
    assert ws(C.CSA2_OP_TOPK, 32, 1, 32768, 16385, 0, 0, 0) == 0
    # decode rows are split: at least two partials of [16][512] floats per row
    part = 16 * 512 * 4
    assert ws(C.CSA2_OP_SPARSE_ATTN, 32, 1, 32768, 512, 0, 0, 16) >= 32 * 2 * part
    assert ws(C.CSA2_OP_SPARSE_ATTN, 32, 1, 32768, 512, 0, 0, 8) == 0
    # at most one partial per step (four window steps per row)
    assert 256 <= ws(C.CSA2_OP_SWA_MERGE, 32, 1, 0, 0, 0, 128, 16) <= 32 * 4 * (part + 128) + 512
    assert ws(C.CSA2_OP_SPARSE_ATTN, 1, 2048, 65536, 512, 0, 0, 16) == 256   # prefill: none
    # sized by the splits the launch uses, not by one split per step
    assert ws(C.CSA2_OP_SPARSE_ATTN, 32, 1, 32768, 512, 0, 0, 16) < 32 * 16 * part
    d = ws(C.CSA2_OP_DECODE_LAYERS, 8, 1, 262144, 512, 8192, 128, 16)
    assert d >= 8 * 262144 * 4
    assert ws(C.CSA2_OP_DECODE_LAYERS, 8, 1, 262144, 512, 256, 128, 16) == 0  # P < K
    assert ws(99, 1, 1, 1, 1, 0, 0, 16) == 0


def test_prefill_workspace_holds_the_run_maxima():
    """A prefill chunk of 256 or more rows longer than 16384 entries with K <= 512
    selects from run maxima: its workspace holds, beyond the scores and visible
    counts, [ceil(M / 128)][B Q][8] floats of them (nothing for K > 512 or for
    rows of at most 16384 entries)."""
    ws = C.csa2_workspace_bytes
    al = lambda x: (x + 255) // 256 * 256

    def pf(B, Q, M, K):
        return ws(C.CSA2_OP_PREFILL_LAYERS, B, Q, M, K, 0, 128, 16)
    for B, Q, M in ((1, 256, 20000), (2, 128, 65536), (1, 2048, 65536)):
        R = B * Q
        runs = al(R * 8 * ((M + 127) // 128) * 4)
        assert pf(B, Q, M, 512) - pf(B, Q, M, 513) == runs, (B, Q, M)
        assert pf(B, Q, M, 512) == al(R * M * 4) + al(R * 4) + runs, (B, Q, M)
    assert pf(1, 256, 16384, 512) == al(256 * 16384 * 4) + al(256 * 4)   # short rows: none


def _pool(**kw):
    d = dict(latent=A, scale=A, idx_key=A, B=2, M=1024)
    d.update(kw)
    return C.make_pool(d["latent"], d["scale"], d["idx_key"], d["B"], d["M"],
                       d.get("D", 512), d.get("HI", 8), d.get("DI", 64))


def _score(pool, **kw):
    a = dict(q_idx=A, w_idx=A, Q=1, pos0=-1, ratio=4, cand=None, P=0, scores=A, hist=None)
    a.update(kw)
    return C.csa2_index_score(pool, a["q_idx"], a["w_idx"], a["Q"], a["pos0"], a["ratio"],
                              a["cand"], a["P"], a["scores"], a["hist"], 0,
                              raise_on_error=False)


def test_index_score_argument_errors():
    assert _score(_pool(latent=None)) == C.CSA2_ERR_NULL
    assert _score(_pool(), q_idx=None) == C.CSA2_ERR_NULL
    assert _score(_pool(), scores=None) == C.CSA2_ERR_NULL
    assert _score(_pool(B=0)) == C.CSA2_ERR_SHAPE
    assert _score(_pool(M=0)) == C.CSA2_ERR_SHAPE
    assert _score(_pool(D=256)) == C.CSA2_ERR_SHAPE
    assert _score(_pool(HI=4)) == C.CSA2_ERR_SHAPE
    assert _score(_pool(), Q=0) == C.CSA2_ERR_SHAPE
    assert _score(_pool(B=40000), Q=2) == C.CSA2_ERR_SHAPE
    assert _score(_pool(), pos0=10, ratio=0) == C.CSA2_ERR_SHAPE
    assert _score(_pool(), cand=A, P=0) == C.CSA2_ERR_SHAPE
    assert _score(_pool(idx_key=A + 4)) == C.CSA2_ERR_ALIGN
    assert _score(_pool(), q_idx=A + 8) == C.CSA2_ERR_ALIGN
    assert _score(_pool(), scores=A + 2) == C.CSA2_ERR_ALIGN


def test_topk_argument_errors():
    f = lambda **kw: C.csa2_topk(kw.get("scores", A), kw.get("R", 4), kw.get("N", 100),
                                 kw.get("n_valid"), kw.get("cand"), kw.get("K", 8),
                                 kw.get("idx", A2), kw.get("ws", A), kw.get("ws_bytes", 0),
                                 0, raise_on_error=False)
    need = C.csa2_workspace_bytes(C.CSA2_OP_TOPK, 4, 1, 100, 8, 0, 0, 0)
    assert f(scores=None) == C.CSA2_ERR_NULL
    assert f(idx=None) == C.CSA2_ERR_NULL
    assert f(R=0) == C.CSA2_ERR_SHAPE
    assert f(N=0) == C.CSA2_ERR_SHAPE
    assert f(K=0) == C.CSA2_ERR_SHAPE
    assert f(K=16385) == C.CSA2_ERR_SHAPE
    assert f(ws_bytes=need - 1) == C.CSA2_ERR_WORKSPACE
    assert f(ws=None, ws_bytes=need) == C.CSA2_ERR_WORKSPACE
    assert f(ws=A + 4, ws_bytes=need) == C.CSA2_ERR_ALIGN
    assert f(scores=A + 2, ws_bytes=need) == C.CSA2_ERR_ALIGN


def test_attention_argument_errors():
    need = C.csa2_workspace_bytes(C.CSA2_OP_SPARSE_ATTN, 2, 1, 1024, 64, 0, 0, 16)
    g = lambda pool=None, **kw: C.csa2_sparse_attn(pool or _pool(), kw.get("q", A), kw.get("Q", 1),
                                                   kw.get("H", 16), kw.get("idx", A), kw.get("K", 64),
                                                   kw.get("o", A), kw.get("lse", A), kw.get("ws", A),
                                                   kw.get("ws_bytes", need - 1), 0,
                                                   raise_on_error=False)
    assert g(q=None) == C.CSA2_ERR_NULL
    assert g(H=8) == C.CSA2_ERR_SHAPE
    assert g(K=0) == C.CSA2_ERR_SHAPE
    assert g(o=A + 4) == C.CSA2_ERR_ALIGN
    assert g() == C.CSA2_ERR_WORKSPACE
    needw = C.csa2_workspace_bytes(C.CSA2_OP_SWA_MERGE, 2, 1, 0, 0, 0, 128, 16)
    h = lambda **kw: C.csa2_swa_merge(kw.get("q", A), kw.get("B", 2), 1, kw.get("H", 16),
                                      kw.get("D", 512), kw.get("swa", A), kw.get("W", 128), A, A,
                                      A, kw.get("ws_bytes", needw - 1), 0, raise_on_error=False)
    assert h(q=None) == C.CSA2_ERR_NULL
    assert h(swa=None) == C.CSA2_ERR_NULL
    assert h(D=256) == C.CSA2_ERR_SHAPE
    assert h(W=-1) == C.CSA2_ERR_SHAPE
    assert h(W=5000) == C.CSA2_ERR_SHAPE
    assert h() == C.CSA2_ERR_WORKSPACE


def test_append_argument_errors():
    # every case returns before any HIP call, so fake aligned addresses are fine
    f = lambda **kw: C.csa2_pool_append(kw.get("lat", A), kw.get("sc", A), kw.get("key", A),
                                        kw.get("B", 2), kw.get("M", 100), kw.get("xl", A),
                                        kw.get("xk", A), kw.get("slot", A), kw.get("T", 0), 0,
                                        raise_on_error=False)
    assert f() == C.CSA2_OK                     # T == 0: nothing to do, no launch
    assert f(lat=None) == C.CSA2_ERR_NULL
    assert f(slot=None) == C.CSA2_ERR_NULL
    assert f(B=0) == C.CSA2_ERR_SHAPE
    assert f(M=0) == C.CSA2_ERR_SHAPE
    assert f(T=-1) == C.CSA2_ERR_SHAPE
    assert f(xl=A + 4) == C.CSA2_ERR_ALIGN
    assert f(key=A + 4) == C.CSA2_ERR_ALIGN
    g = lambda **kw: C.csa2_swa_append(kw.get("swa", A), kw.get("B", 2), kw.get("W", 128),
                                       kw.get("x", A), kw.get("pos0", 0), kw.get("T", 0), 0,
                                       raise_on_error=False)
    assert g() == C.CSA2_OK
    assert g(x=None) == C.CSA2_ERR_NULL
    assert g(W=0) == C.CSA2_ERR_SHAPE
    assert g(pos0=-1) == C.CSA2_ERR_SHAPE
    assert g(T=-2) == C.CSA2_ERR_SHAPE
    assert g(x=A + 8) == C.CSA2_ERR_ALIGN
    assert g(swa=A + 4) == C.CSA2_ERR_ALIGN


def _layer(mode, **kw):
    d = dict(q_idx=A, w_idx=A, q=A, swa=A, o=A, lse=A, idx_out=A2)
    d.update(kw)
    return C.csa2_layer(mode, d["q_idx"], d["w_idx"], d["q"], d["swa"], d["o"], d["lse"],
                        d["idx_out"])


def test_decode_layers_schedule_and_argument_errors():
    pool = _pool()
    need = C.csa2_workspace_bytes(C.CSA2_OP_DECODE_LAYERS, 2, 1, 1024, 64, 0, 128, 16)

    def run(layers, K=64, P=0, W=128, H=16, ws=A, nb=need - 1, pool=pool):
        st, _ = C.csa2_decode_layers(pool, layers, H, K, P, W, ws, nb, 0, raise_on_error=False)
        return st

    F, RI, RU = C.CSA2_FULL, C.CSA2_REINDEX, C.CSA2_REUSE
    assert run([_layer(RI)]) == C.CSA2_ERR_SCHEDULE
    assert run([_layer(RU), _layer(F)]) == C.CSA2_ERR_SCHEDULE
    assert run([_layer(F), _layer(7)]) == C.CSA2_ERR_SCHEDULE
    assert run([_layer(F, idx_out=None)]) == C.CSA2_ERR_NULL
    assert run([_layer(F), _layer(RI, q_idx=None)]) == C.CSA2_ERR_NULL
    assert run([_layer(F), _layer(RU, swa=None)]) == C.CSA2_ERR_NULL
    assert run([_layer(F, o=None)]) == C.CSA2_ERR_NULL
    assert run([_layer(F)], K=0) == C.CSA2_ERR_SHAPE
    assert run([_layer(F)], P=32) == C.CSA2_ERR_SHAPE       # P < K
    assert run([_layer(F)], H=8) == C.CSA2_ERR_SHAPE
    assert run([_layer(F)], W=4097) == C.CSA2_ERR_SHAPE
    assert run([_layer(F, q=A + 2)]) == C.CSA2_ERR_ALIGN
    assert run([_layer(F), _layer(RU, idx_out=None)]) == C.CSA2_ERR_WORKSPACE
    assert run([_layer(F)], ws=None, nb=need) == C.CSA2_ERR_WORKSPACE
    assert run([_layer(F)], pool=_pool(scale=None)) == C.CSA2_ERR_NULL


def test_decode_layer_argument_errors():
    """The per-layer call checks the whole schedule and the layer number."""
    pool = _pool()
    need = C.csa2_workspace_bytes(C.CSA2_OP_DECODE_LAYERS, 2, 1, 1024, 64, 0, 128, 16)
    F, RI, RU = C.CSA2_FULL, C.CSA2_REINDEX, C.CSA2_REUSE

    def run(layers, l, nb=need - 1, **kw):
        st, _ = C.csa2_decode_layer(pool, layers, l, 16, kw.get("K", 64), 0, 128, A, nb, 0,
                                    raise_on_error=False)
        return st

    good = [_layer(F), _layer(RI), _layer(RU)]
    assert run(good, -1) == C.CSA2_ERR_SHAPE
    assert run(good, 3) == C.CSA2_ERR_SHAPE
    assert run(good, 0, K=0) == C.CSA2_ERR_SHAPE
    assert run([_layer(RU), _layer(F)], 1) == C.CSA2_ERR_SCHEDULE     # layer 0 not Full
    assert run([_layer(F), _layer(RI, q_idx=None)], 0) == C.CSA2_ERR_NULL
    assert run(good, 2) == C.CSA2_ERR_WORKSPACE


def test_decode_layers_noalloc_argument_errors():
    """The static-scratch decode checks its arguments as csa2_decode_layers does
    and refuses a step larger than its scratch, all before any HIP call."""
    F, RI, RU = C.CSA2_FULL, C.CSA2_REINDEX, C.CSA2_REUSE

    def run(layers, pool=None, K=64, P=0, W=128, H=16):
        st, _ = C.csa2_decode_layers_noalloc(pool or _pool(), layers, H, K, P, W, 0,
                                             raise_on_error=False)
        return st

    assert run([_layer(RU), _layer(F)]) == C.CSA2_ERR_SCHEDULE
    assert run([_layer(F)], K=0) == C.CSA2_ERR_SHAPE
    assert run([_layer(F)], H=8) == C.CSA2_ERR_SHAPE
    assert run([_layer(F)], P=32) == C.CSA2_ERR_SHAPE          # P < K
    assert run([_layer(F, lse=None)]) == C.CSA2_ERR_NULL
    assert run([_layer(F)], pool=_pool(idx_key=None)) == C.CSA2_ERR_NULL
    ws = C.csa2_workspace_bytes
    lim = C.CSA2_NOALLOC_SCRATCH_BYTES
    assert ws(C.CSA2_OP_DECODE_LAYERS, 64, 1, 262144, 512, 0, 128, 16) > lim
    assert run([_layer(F)], pool=_pool(B=64, M=262144), K=512) == C.CSA2_ERR_SCRATCH
    # the workloads it is meant for fit
    assert ws(C.CSA2_OP_DECODE_LAYERS, 64, 1, 65536, 512, 0, 128, 16) <= lim
    assert ws(C.CSA2_OP_DECODE_LAYERS, 8, 1, 262144, 512, 8192, 128, 16) <= lim
    assert ws(C.CSA2_OP_DECODE_LAYERS, 32, 1, 32768, 512, 0, 128, 16) <= lim


def test_score_topk_argument_errors():
    ws = C.csa2_workspace_bytes
    need = ws(C.CSA2_OP_SCORE_TOPK, 2, 1, 1024, 64, 0, 0, 0)
    assert need >= 2 * 2 * 64 * 4                      # keys and positions of the keepers
    assert ws(C.CSA2_OP_SCORE_TOPK, 32, 1, 32768, 512, 0, 0, 0) > 0
    assert ws(C.CSA2_OP_SCORE_TOPK, 8, 1, 262144, 512, 0, 0, 0) == 0   # keepers overflow
    assert ws(C.CSA2_OP_SCORE_TOPK, 2, 1, 1024, 0, 0, 0, 0) == 0

    def run(pool=None, q=A, w=A, K=64, idx=A2, w_=A, nb=need):
        return C.csa2_score_topk(pool or _pool(), q, w, K, idx, w_, nb, 0, raise_on_error=False)

    assert run(q=None) == C.CSA2_ERR_NULL
    assert run(idx=None) == C.CSA2_ERR_NULL
    assert run(K=0) == C.CSA2_ERR_SHAPE
    assert run(pool=_pool(B=8, M=262144), K=512) == C.CSA2_ERR_SHAPE
    assert run(q=A + 4) == C.CSA2_ERR_ALIGN
    assert run(nb=need - 1) == C.CSA2_ERR_WORKSPACE
    assert run(w_=None) == C.CSA2_ERR_WORKSPACE


def test_prefill_layers_schedule_and_argument_errors():
    pool = _pool()
    need = C.csa2_workspace_bytes(C.CSA2_OP_PREFILL_LAYERS, 2, 64, 1024, 64, 0, 128, 16)
    assert need >= 2 * 64 * 1024 * 4
    assert C.csa2_workspace_bytes(C.CSA2_OP_PREFILL_LAYERS, 2, 64, 1024, 64, 0, 128, 8) == 0
    assert C.csa2_workspace_bytes(C.CSA2_OP_PREFILL_LAYERS, 2, 40000, 1024, 64, 0, 128, 16) == 0

    def run(layers, Q=64, pos0=0, ratio=4, K=64, W=128, H=16, ws=A, nb=need - 1, pool=pool):
        st, _ = C.csa2_prefill_layers(pool, layers, Q, pos0, ratio, H, K, W, ws, nb, 0,
                                      raise_on_error=False)
        return st

    F, RI, RU = C.CSA2_FULL, C.CSA2_REINDEX, C.CSA2_REUSE
    assert run([_layer(RI)]) == C.CSA2_ERR_SCHEDULE
    assert run([_layer(RU), _layer(F)]) == C.CSA2_ERR_SCHEDULE
    assert run([_layer(F), _layer(5)]) == C.CSA2_ERR_SCHEDULE
    assert run([_layer(F, idx_out=None)]) == C.CSA2_ERR_NULL
    assert run([_layer(F), _layer(RI, w_idx=None)]) == C.CSA2_ERR_NULL
    assert run([_layer(F, swa=None)]) == C.CSA2_ERR_NULL
    assert run([_layer(F, lse=None)]) == C.CSA2_ERR_NULL
    assert run([_layer(F)], Q=0) == C.CSA2_ERR_SHAPE
    assert run([_layer(F)], Q=40000) == C.CSA2_ERR_SHAPE      # B * Q rows above the limit
    assert run([_layer(F)], ratio=0) == C.CSA2_ERR_SHAPE
    assert run([_layer(F)], K=16385) == C.CSA2_ERR_SHAPE
    assert run([_layer(F)], H=8) == C.CSA2_ERR_SHAPE
    assert run([_layer(F)], W=-1) == C.CSA2_ERR_SHAPE
    assert run([_layer(F, o=A + 4)]) == C.CSA2_ERR_ALIGN
    assert run([_layer(F)]) == C.CSA2_ERR_WORKSPACE
    assert run([_layer(F)], ws=None, nb=need) == C.CSA2_ERR_WORKSPACE
    assert run([_layer(F)], ws=A + 8, nb=need) == C.CSA2_ERR_ALIGN
    assert run([_layer(F)], pool=_pool(M=0)) == C.CSA2_ERR_SHAPE
    # no causal limit: ratio is not used
    assert run([_layer(F)], pos0=-1, ratio=0) == C.CSA2_ERR_WORKSPACE


def test_host_tier_argument_errors():
    H = 0x30000   # a fake host address: never dereferenced here

    def restore(**kw):
        a = dict(latent=A, scale=A, idx_key=A, B=2, M=100, seq=1, entry0=10, n=5, h=H)
        a.update(kw)
        return C.csa2_pool_restore(a["latent"], a["scale"], a["idx_key"], a["B"], a["M"], a["seq"],
                                   a["entry0"], a["n"], a["h"], a["h"], a["h"], 0,
                                   raise_on_error=False)

    assert restore(latent=None) == C.CSA2_ERR_NULL
    assert restore(h=None) == C.CSA2_ERR_NULL
    assert restore(seq=2) == C.CSA2_ERR_SHAPE
    assert restore(seq=-1) == C.CSA2_ERR_SHAPE
    assert restore(entry0=96) == C.CSA2_ERR_SHAPE           # entry0 + n > M
    assert restore(n=-1) == C.CSA2_ERR_SHAPE
    assert restore(M=0) == C.CSA2_ERR_SHAPE
    assert restore(n=0) == C.CSA2_OK                        # nothing to copy, no HIP call
    assert C.csa2_pool_offload(A, A, A, 2, 100, 0, 0, 101, H, H, H, 0,
                               raise_on_error=False) == C.CSA2_ERR_SHAPE
    assert C.csa2_swa_restore(A, 2, 128, 2, H, 0, raise_on_error=False) == C.CSA2_ERR_SHAPE
    assert C.csa2_swa_restore(A, 2, 0, 0, H, 0, raise_on_error=False) == C.CSA2_ERR_SHAPE
    assert C.csa2_swa_offload(A, 2, 128, 0, None, 0, raise_on_error=False) == C.CSA2_ERR_NULL


def test_pool_length_array_alignment():
    pool = _pool()
    pool.len = A + 2
    assert _score(pool) == C.CSA2_ERR_ALIGN


def test_paged_pool_argument_errors():
    pool = _pool(M=1024)
    pool.pages = A
    pool.page_log2 = 5                                 # pages smaller than a scan wave's 64 entries
    assert _score(pool) == C.CSA2_ERR_SHAPE
    pool.page_log2 = 11                                # 2048 does not divide M = 1024
    assert _score(pool) == C.CSA2_ERR_SHAPE
    pool.page_log2 = 8
    pool.pages = A + 2
    assert _score(pool) == C.CSA2_ERR_ALIGN
    f = lambda lg2, pages=A: C.csa2_pool_append(A, A, A, 2, 1024, A, A, A, 4, 0,
                                                raise_on_error=False, pages=pages, page_log2=lg2)
    assert f(4) == C.CSA2_ERR_SHAPE
    assert f(8, pages=A + 1) == C.CSA2_ERR_ALIGN
