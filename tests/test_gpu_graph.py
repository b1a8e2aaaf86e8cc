"""A decode step captured into a HIP graph (torch.cuda.CUDAGraph around
csa2_decode_layers) replays to the eager call's results bit for bit.

The step launches kernels only (the Top-K scratch is cleared by a fill
kernel, not by a memset), so it can be captured.  Each replay follows eager
work that overwrites every output and a synchronisation; after the inputs are
changed in place, a replay must equal a new eager call on the changed inputs.
Two steps issued from two host threads onto two streams at once must give the
results of the same steps run one after the other.  The chunked-prefill chain
is captured and replayed the same way, and so is csa2_prefill_layers on rows
long enough for the group select (its run maxima recomputed on every replay).
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


CASES = [
    dict(name="graph_flat", B=8, M=20000, K=256, W=128, modes=(FULL, REINDEX, REUSE, REUSE)),
    dict(name="graph_hier", B=4, M=40000, K=256, P=4096, W=64, modes=(FULL, REINDEX, REUSE, REINDEX)),
]


def _same(want, got, what):
    for ell, (a, b) in enumerate(zip(want, got)):
        for k in ("idx", "o", "lse"):
            assert np.array_equal(a[k], b[k]), "%s: layer %d %s differs" % (what, ell, k)


def _clobber(dc):
    for d in dc.layers:
        d["o"].fill_(12345.0)
        d["lse"].fill_(-3.0)
        d["idx"].fill_(-7)


@pytest.mark.parametrize("kw", CASES, ids=[c["name"] for c in CASES])
def test_decode_step_graph_replay(kw):
    from fp4_kv_cache_score_amd.device import DeviceCase
    cfg = CONFIGS[0].scaled(seed=90 + len(kw["name"]), **kw)
    say("case: graph replay", cfg.name, cfg.modes)
    case = synth.make_case(cfg)
    dc = DeviceCase(case)
    dc.prepare_decode()
    dc.decode_layers()                       # eager (also loads every kernel before capture)
    torch.cuda.synchronize()
    want = dc.results()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        dc.decode_layers()
    torch.cuda.synchronize()

    for rep in range(3):
        _clobber(dc)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(want, dc.results(), "replay %d" % rep)

    # Inputs changed in place (queries of sequence b moved to sequence B-1-b):
    # the graph reads them at replay time.
    for d in dc.layers:
        for k in ("q_idx", "w_idx"):
            if d[k] is not None:         # Reuse layers carry no indexer query
                d[k].copy_(d[k].flip(0))
        qv = d["q"].view(torch.int16)
        qv.copy_(qv.flip(0))
    torch.cuda.synchronize()
    _clobber(dc)
    g.replay()
    torch.cuda.synchronize()
    got = dc.results()
    _clobber(dc)
    dc.decode_layers()
    torch.cuda.synchronize()
    want2 = dc.results()
    _same(want2, got, "replay on changed inputs")
    assert not np.array_equal(want2[0]["idx"], want[0]["idx"])


def test_decode_two_streams_two_host_threads():
    """No global state: two decode steps with their own workspaces, issued
    from two host threads onto two streams at once, give the results of the
    same steps run one after the other."""
    import threading
    from fp4_kv_cache_score_amd.device import DeviceCase
    say("case: two streams, two host threads")
    dcs, want = [], []
    for kw in CASES:
        cfg = CONFIGS[0].scaled(seed=70 + len(kw["name"]), **kw)
        dc = DeviceCase(synth.make_case(cfg))
        dc.prepare_decode()
        dc.decode_layers()
        torch.cuda.synchronize()
        want.append(dc.results())
        _clobber(dc)
        dcs.append(dc)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in dcs]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    errors = []

    def run(dc, s):
        try:
            with torch.cuda.stream(s):
                for _ in range(5):
                    dc.decode_layers()
        except Exception as e:       # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(dc, s)) for dc, s in zip(dcs, streams)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for dc, w, kw in zip(dcs, want, CASES):
        _same(w, dc.results(), kw["name"] + " on its own stream")


@pytest.mark.parametrize("M", [4096, 40000])
def test_prefill_chain_graph_replay(M):
    """The chunked-prefill chain (causal scores, Top-K over the visible
    entries, attention, window merge) captured into a graph: every replay
    equals the eager chain (rows held in registers at M = 4096, streamed rows
    at M = 40000)."""
    from fp4_kv_cache_score_amd.device import DeviceCase
    cfg = CONFIGS[4].scaled(name="graph_pf", seed=55, B=1, Q=256, M=M, K=128, W=128)
    say("case: prefill chain graph replay Q=%d M=%d" % (cfg.Q, cfg.M))
    dc = DeviceCase(synth.make_case(cfg))
    dc.prefill()                             # eager; allocates the chain's buffers
    torch.cuda.synchronize()
    outs = (dc.pf_idx, dc.pf_o, dc.pf_lse)
    want = [t.cpu().numpy() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        dc.prefill()
    torch.cuda.synchronize()
    for rep in range(3):
        dc.pf_idx.fill_(-7)
        dc.pf_o.fill_(12345.0)
        dc.pf_lse.fill_(-3.0)
        dc.pf_scores.fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, t in zip(("idx", "o", "lse"), want, outs):
            assert np.array_equal(a, t.cpu().numpy()), "replay %d: %s differs" % (rep, name)


def test_prefill_layers_graph_replay_group_select():
    """csa2_prefill_layers on rows long enough for the group select (256 tokens,
    40000 entries: the score kernel writes run maxima, the select reads them)
    captured into a graph: every replay, after the outputs and the whole
    workspace (scores and run maxima) are overwritten, equals the eager call."""
    from fp4_kv_cache_score_amd.device import DeviceCase
    cfg = CONFIGS[4].scaled(name="graph_pfl", seed=57, B=1, Q=256, M=40000, K=512, W=64,
                            modes=(FULL, REINDEX, REUSE))
    say("case: prefill layers graph replay Q=%d M=%d (group select)" % (cfg.Q, cfg.M))
    dc = DeviceCase(synth.make_case(cfg))
    dc.prefill_layers()                      # eager; allocates the workspace
    torch.cuda.synchronize()
    want = dc.results()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        dc.prefill_layers()
    torch.cuda.synchronize()
    for rep in range(3):
        _clobber(dc)
        dc.ws.fill_(0x7F)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(want, dc.results(), "replay %d" % rep)
