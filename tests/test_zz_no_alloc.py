"""csa2_decode_layers_noalloc (the decode step in the library's static
scratch) against csa2_decode_layers (the same step in a caller's workspace).

Two calls in a row through the C ABI, the second on a smaller input whose
multi-work-group select keeps its histogram and counters where the first
call left scores, then a third, flat call: every index, output and lse equal
the workspace call's bit for bit (the two entry points run the same kernels
in the same order).
"""
import sys

import numpy as np
import pytest
import torch

from fp4_kv_cache_score_amd import _lib as C
from fp4_kv_cache_score_amd import synth
from fp4_kv_cache_score_amd.configs import CONFIGS, FULL, REINDEX, REUSE

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    C.lib()
    yield


# larger first, then smaller: (seed, B, M, K, P, modes)
CASES = [
    (500, 8, 60000, 512, 8192, (FULL, REINDEX, REUSE, REINDEX)),
    (501, 3, 40000, 256, 8192, (FULL, REUSE, REINDEX)),
    (502, 2, 5000, 128, 0, (FULL, REUSE, REINDEX)),
]


def _device_case(seed, B, M, K, P, modes):
    from fp4_kv_cache_score_amd.device import DeviceCase
    cfg = CONFIGS[0].scaled(name="noalloc_%d" % seed, seed=seed, B=B, M=M, K=K, P=P, modes=modes)
    need = C.csa2_workspace_bytes(C.CSA2_OP_DECODE_LAYERS, cfg.B, 1, cfg.M, cfg.K, cfg.P, cfg.W,
                                  cfg.H)
    assert 0 < need <= C.CSA2_NOALLOC_SCRATCH_BYTES
    dc = DeviceCase(synth.make_case(cfg))
    dc.prepare_decode()
    return dc


def test_noalloc_equals_workspace_call():
    dcs = [_device_case(*c) for c in CASES]
    ref, ref_src = [], []
    for c, dc in zip(CASES, dcs):
        say("case: workspace call", c[:5])
        ref_src.append(dc.decode_layers())
        torch.cuda.synchronize()
        ref.append(dc.results())
        for d in dc.layers:   # scramble the outputs before the second run
            d["o"].fill_(7.0)
            d["lse"].fill_(7.0)
            d["idx"].fill_(-7)
    torch.cuda.synchronize()
    for i, (c, dc) in enumerate(zip(CASES, dcs)):
        say("case: static-scratch call", c[:5])
        cfg = dc.cfg
        st, src = C.csa2_decode_layers_noalloc(dc.pool, dc._structs, cfg.H, cfg.K, cfg.P, cfg.W)
        assert st == C.CSA2_OK
        assert src == ref_src[i]
    torch.cuda.synchronize()
    for c, dc, want in zip(CASES, dcs, ref):
        got = dc.results()
        for ell, (a, b) in enumerate(zip(want, got)):
            for k in ("idx", "o", "lse"):
                assert np.array_equal(a[k], b[k]), (c[:5], ell, k)


def test_noalloc_refuses_a_step_beyond_the_scratch():
    dc = _device_case(*CASES[2])
    cfg = dc.cfg
    # a pool header that claims more sequences and entries than the buffers
    # hold: the size check refuses it before any HIP call
    big = C.make_pool(dc.latent, dc.scale, dc.idx_key, 64, 262144, cfg.D, cfg.HI, cfg.DI)
    assert C.csa2_workspace_bytes(C.CSA2_OP_DECODE_LAYERS, 64, 1, 262144, cfg.K, 0, cfg.W,
                                  cfg.H) > C.CSA2_NOALLOC_SCRATCH_BYTES
    st, _ = C.csa2_decode_layers_noalloc(big, dc._structs, cfg.H, cfg.K, 0, cfg.W,
                                         raise_on_error=False)
    assert st == C.CSA2_ERR_SCRATCH
