#!/usr/bin/env python3
"""CSA2 decode benchmark on one MI355X: query-tokens/s and achieved HBM bandwidth.

A step is one decode token for every sequence of the batch through the whole
layer schedule (indexer scan, Top-K, FP4 gather + attention, FP8 window merge
per layer) with all inputs resident in HBM.  The headline is the MALL-cold
step: before every layer a 512 MiB read-write sweep evicts the 256 MB
last-level cache (outside the timed region), the layer alone
(csa2_decode_layer) is timed between HIP events on the stream it runs on, and
a step's time is the sum of its layers' times; the median over the timed
steps is reported.  (In a model the weights read between two layers evict
that cache.)  Back-to-back whole steps (csa2_decode_layers, warm) are reported
beside it.  The default workload is the 128K-context decode (batch 32, pool
M = 32768, K = 512, W = 128, layers Full / Reindex / Reuse / Reuse); the
1M-context hierarchical decode (batch 8, M = 262144, P = 8192, Full + 3
Reindex) and the 20-layer schedule are measured the same way under "extra".

Prints ONE JSON line.  `roofline` is for the dominant kernel (the indexer
scan): algorithmic bytes per launch / its mean duration, timed with HIP
events on the stream it runs on; `traffic` is the counter-measured HBM bytes
per launch recorded under profiles/ for the same kernel source (null when the
kernel changed since).  `cpu_baseline` times the CPU oracle on bounded samples
of the 128K, 1M and prefill workloads on one host core.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
SCORE_SRC = [os.path.join(ROOT, "fp4_kv_cache_score_amd", "csrc", f)
             for f in ("index_score.hip", "index_math.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    """Hash of the scan kernel's sources (its body and its arithmetic)."""
    h = hashlib.sha256()
    for f in SCORE_SRC:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


# The scan as the decode step launches it: 64 entries per wave, flat, no histogram.
SCAN_VARIANT = "k_index_score<64, false, false>"


def recorded_traffic(workload: str):
    """HBM bytes per scan launch from the counter summary of this workload.

    The summary (profiles/index_score_<workload>.txt) records the scan
    kernel's source hash; a summary taken on another version of the kernel
    does not count (None).
    """
    try:
        text = open(os.path.join(PROFILES, "index_score_%s.txt" % workload)).read()
    except OSError:
        return None
    fields = dict(m.groups() for m in re.finditer(r"^(\w+):\s*(.+?)\s*$", text, re.M))
    if fields.get("kernel_sha256_16") != kernel_hash() or fields.get("kernel_variant") != SCAN_VARIANT:
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_decode(dc, steps: int, warmup: int):
    import torch
    dc.prepare_decode(idx_for_reuse=False)
    for _ in range(warmup):
        dc.decode_layers()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        dc.decode_layers()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def time_structs(dc, structs, steps: int, warmup: int) -> float:
    """Back-to-back mean ms of one decode_layers call over the given layer structs."""
    import torch
    from fp4_kv_cache_score_amd import _lib as C
    cfg = dc.cfg
    stream = torch.cuda.current_stream()

    def run():
        C.csa2_decode_layers(dc.pool, structs, cfg.H, cfg.K, cfg.P, cfg.W, dc.ws, dc.ws_bytes,
                             stream)
    for _ in range(warmup):
        run()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def cold_layers_ms(dc, steps: int, sweep_mib: int = 512, write: bool = False):
    """MALL-cold steps: before every layer a sweep of sweep_mib MiB (outside the
    timed region), then the layer alone (csa2_decode_layer) between HIP events.
    Returns (median step ms, per-layer median ms, all step ms), a step's time
    being the sum of its layers' times.

    The sweep reads (write=False), as the weights a model streams between two
    layers are read: it evicts the cache and leaves it clean.  A written sweep
    (write=True) leaves up to the cache's size in dirty lines, whose write-back
    to HBM then lands inside the next layer's timed region."""
    import torch
    stream = torch.cuda.current_stream()
    sweep = torch.zeros(sweep_mib << 20, dtype=torch.uint8, device="cuda")
    sweep_f = sweep.view(torch.float32)
    sink = torch.zeros((), dtype=torch.float32, device="cuda")
    L = dc.cfg.L
    dc.prepare_decode(idx_for_reuse=False)
    dc.decode_layers()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(L)] for _ in range(steps)]
    for row in evs:
        for ell, (a, b) in enumerate(row):
            if write:
                sweep.add_(1)
            else:
                torch.sum(sweep_f, dim=0, out=sink)
            a.record(stream)
            dc.decode_layer(ell)
            b.record(stream)
    torch.cuda.synchronize()
    del sweep, sweep_f, sink
    per = np.array([[a.elapsed_time(b) for a, b in row] for row in evs])   # [steps][L]
    T = per.sum(axis=1)
    return float(np.median(T)), np.median(per, axis=0).tolist(), T.tolist()


def all_full_ms(dc, steps: int, warmup: int) -> float:
    """The same layers with every layer in Full mode (each one scans and selects):
    the per-layer indexing that Reindex / Reuse layers avoid.  Layers without an
    indexer query of their own use the first layer's."""
    from fp4_kv_cache_score_amd import _lib as C
    first = next(d for d in dc.layers if d["q_idx"] is not None)
    structs = []
    for d in dc.layers:
        qi = d["q_idx"] if d["q_idx"] is not None else first["q_idx"]
        wi = d["w_idx"] if d["w_idx"] is not None else first["w_idx"]
        structs.append(C.csa2_layer(C.CSA2_FULL, C._p(qi), C._p(wi), C._p(d["q"]),
                                    C._p(d["swa"]), C._p(d["o"]), C._p(d["lse"]),
                                    C._p(d["idx"])))
    return time_structs(dc, structs, steps, warmup)


def time_score_kernel(dc, launches: int):
    """Mean duration of the scan kernel as decode launches it (flat, no histogram)."""
    import torch
    from fp4_kv_cache_score_amd import _lib as C
    cfg = dc.cfg
    d = dc.layers[0]
    scores = torch.empty((cfg.B, cfg.M), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(3):
        C.csa2_index_score(dc.pool, d["q_idx"], d["w_idx"], 1, -1, 1, None, 0, scores, None, stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(launches)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(stream)
        C.csa2_index_score(dc.pool, d["q_idx"], d["w_idx"], 1, -1, 1, None, 0, scores, None, stream)
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    return float(np.mean(ms)), float(np.min(ms))


def _time_calls(fn, steps: int, warmup: int) -> float:
    """Mean milliseconds of fn() on the current stream (HIP events around each call)."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def _prefill_flops(cfg, pos0: int):
    t = np.arange(cfg.Q)
    vis = np.minimum(cfg.M, (pos0 + t + 1) // cfg.ratio)
    idx_flop = 2.0 * cfg.B * float(vis.sum()) * cfg.HI * cfg.DI
    # S = q C^T and O = P C (P as bf16 hi + lo, two products) over the selected + window keys
    keys = np.minimum(cfg.K, vis) + np.minimum(cfg.W, pos0 + t + 1)
    attn_flop = 2.0 * cfg.B * cfg.H * cfg.D * float(keys.sum()) * 3
    return idx_flop, attn_flop


def measure_prefill(ci: int, steps: int, warmup: int, context: bool = True):
    """Chunked prefill: csa2_prefill_layers on the chunk of `ci` (one Full layer), its
    stages, the unfused four-call chain, a 4-layer schedule, the first chunk of a
    context, and a whole context prefilled chunk by chunk into a growing pool."""
    import torch
    from fp4_kv_cache_score_amd import _lib as C
    from fp4_kv_cache_score_amd import synth
    from fp4_kv_cache_score_amd.configs import CONFIGS, FULL, REINDEX, REUSE
    from fp4_kv_cache_score_amd.device import DeviceCase
    cfg = CONFIGS[ci]
    case = synth.make_case(cfg)
    dc = DeviceCase(case)
    dc.prepare_prefill()
    dc.prepare_prefill_layers()
    ms = _time_calls(dc.prefill_layers, steps, warmup)
    stage_ms = [_time_calls(lambda st=st: dc.prefill_stage(st), steps, warmup) for st in range(4)]
    # the attention work (selected entries, then window rows) as the separate
    # calls do it; the chunk runs both in one pass (its kernel time is in the
    # kernel trace)
    attn_ms = stage_ms[2] + stage_ms[3]
    idx_flop, attn_flop = _prefill_flops(cfg, cfg.pos0)
    res = dict(workload=cfg.name, case=case,
               query_tokens_per_s=cfg.B * cfg.Q / (ms * 1e-3), ms_per_step=ms,
               path="csa2_prefill_layers (score, Top-K, one attention pass over K + W keys)",
               select_note="csa2_prefill_layers selects each token's Top-K from the runs of 16 "
                           "entries with the largest maxima (written by its score kernel); "
                           "stage_ms times the separate calls, whose csa2_topk reads every score",
               stage_ms={"index_score_mfma": stage_ms[0], "topk": stage_ms[1],
                         "sparse_attn_mfma": stage_ms[2], "swa_merge_mfma": stage_ms[3]},
               unfused_chain_ms=sum(stage_ms),
               index_score_tflops=idx_flop / (stage_ms[0] * 1e-3) / 1e12,
               index_score_frac_of_bf16_mfma_peak=idx_flop / (stage_ms[0] * 1e-3) / 2.5e15,
               attention_tflops=attn_flop / (attn_ms * 1e-3) / 1e12,
               attention_frac_of_bf16_mfma_peak=attn_flop / (attn_ms * 1e-3) / 2.5e15)
    log("prefill %s: %.3f ms (unfused chain %.3f ms)" % (cfg.name, ms, sum(stage_ms)))
    del dc

    # the same chunk through a Full, Reindex, Reuse, Reuse schedule
    sched = (FULL, REINDEX, REUSE, REUSE)
    c4 = cfg.scaled(modes=sched)
    dc = DeviceCase(synth.make_case(c4))
    dc.prepare_prefill_layers(idx_for_reuse=False)     # Reuse layers alias their source's indices
    ms4 = _time_calls(dc.prefill_layers, steps, warmup)
    res["schedule_F_Ri_Ru_Ru"] = dict(ms_per_chunk=ms4,
                                      query_tokens_per_s=c4.B * c4.Q / (ms4 * 1e-3))
    # the first chunk of a context (positions 0 .. Q-1): it sees a prefix of the pool
    ms0 = _time_calls(lambda: dc.prefill_layers(pos0=0), steps, warmup)
    res["schedule_F_Ri_Ru_Ru"]["first_chunk_ms"] = ms0
    log("prefill schedule F,Ri,Ru,Ru: %.3f ms per chunk, first chunk %.3f ms" % (ms4, ms0))

    if not context:
        del dc
        torch.cuda.empty_cache()
        return res
    # a whole context of ratio * M tokens in chunks of Q: before each chunk the
    # Q / ratio entries it completes are appended (MXFP4 / E4M3 encode), then the
    # schedule runs over the chunk at its position
    B, Q, M, ratio = c4.B, c4.Q, c4.M, c4.ratio
    n_chunks = ratio * M // Q
    per = Q // ratio
    g = torch.Generator(device="cuda").manual_seed(5)
    xl = torch.randn((B, per, c4.D), generator=g, device="cuda")
    xk = torch.randn((B, per, c4.HI, c4.DI), generator=g, device="cuda")
    slots = [torch.arange(c * per, (c + 1) * per, dtype=torch.int32, device="cuda")
             .expand(B, per).contiguous() for c in range(n_chunks)]

    def context():
        for c in range(n_chunks):
            C.csa2_pool_append(dc.latent, dc.scale, dc.idx_key, B, M, xl, xk, slots[c], per)
            dc.prefill_layers(pos0=c * Q)

    ctx_ms = _time_calls(context, 2, 1)
    res["schedule_F_Ri_Ru_Ru"]["whole_context"] = dict(
        tokens=ratio * M, chunks=n_chunks, ms=ctx_ms,
        query_tokens_per_s=B * ratio * M / (ctx_ms * 1e-3))
    log("prefill whole context %d tokens in %d chunks: %.1f ms" % (ratio * M, n_chunks, ctx_ms))
    del dc
    torch.cuda.empty_cache()
    return res


def host_info() -> dict:
    """The host the CPU baseline runs on: logical CPUs, CPU model, BLAS threads."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = {i.get("internal_api", i.get("prefix", "?")): i.get("num_threads")
                for i in threadpool_info()}
    except Exception:
        pass
    return dict(host_cpu_count=os.cpu_count(), cpu_model=model, blas_threads_default=blas)


def cpu_decode(case, budget_s: float) -> dict:
    """The CPU oracle, single-threaded, on whole sequences of a decode workload
    (all layers) until the budget is used."""
    from threadpoolctl import threadpool_limits
    from oracle import csa2 as O
    cfg = case.cfg
    p = case.pool
    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        for b in range(cfg.B):
            layers = [dict(mode=L.mode,
                           q_idx=None if L.q_idx is None else L.q_idx[b, 0],
                           w_idx=None if L.w_idx is None else L.w_idx[b, 0],
                           q=L.q[b, 0], swa=L.swa[b]) for L in case.layers]
            O.decode_sequence(p.latent[b], p.scale[b], p.idx_key[b], layers, cfg.K, cfg.P)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
    el = time.perf_counter() - t0
    return dict(value=done / el, unit="query-tokens/s", cores=1, kind="oracle",
                sample="%d of %d sequences of %s through all %d layers (%.1f s, NumPy fp64, "
                       "BLAS limited to 1 thread)" % (done, cfg.B, cfg.name, cfg.L, el))


def cpu_prefill(case, budget_s: float) -> dict:
    """The CPU oracle, single-threaded, on query tokens of a prefill chunk
    (Full layer: score the visible entries, Top-K, attention with the window)
    until the budget is used."""
    from threadpoolctl import threadpool_limits
    from oracle import csa2 as O
    cfg = case.cfg
    p = case.pool
    L = case.layers[0]
    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        for t in range(cfg.Q - 1, -1, -1):
            O.prefill_query(p.latent[0], p.scale[0], p.idx_key[0], L.q_idx[0, t], L.w_idx[0, t],
                            L.q[0, t], L.swa[0], t, cfg.pos0, cfg.ratio, cfg.K, cfg.W)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
    el = time.perf_counter() - t0
    return dict(value=done / el, unit="query-tokens/s", cores=1, kind="oracle",
                sample="%d of %d query tokens of %s (the newest first; %.1f s, NumPy fp64, "
                       "BLAS limited to 1 thread)" % (done, cfg.Q, cfg.name, el))


def measure(ci: int, steps: int, warmup: int, score_launches: int, detail: bool = False):
    import torch
    from fp4_kv_cache_score_amd import synth
    from fp4_kv_cache_score_amd.configs import CONFIGS, algorithmic_bytes
    from fp4_kv_cache_score_amd.device import DeviceCase
    cfg = CONFIGS[ci]
    t0 = time.perf_counter()
    case = synth.make_case(cfg)
    log("generated %s in %.1f s" % (cfg.name, time.perf_counter() - t0))
    dc = DeviceCase(case)
    torch.cuda.synchronize()
    dc.prepare_decode(idx_for_reuse=False)
    for _ in range(warmup):
        dc.decode_layers()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms, per_layer, all_steps = cold_layers_ms(dc, steps)
    wall = time.perf_counter() - t0
    log("%s: MALL-cold step %.3f ms (median of %d; layers %s ms; wall %.2f s with the sweeps)" % (
        cfg.name, ms, steps, ["%.4f" % x for x in per_layer], wall))
    warm_ms, _ = time_decode(dc, steps, 2)
    log("%s: warm back-to-back step %.3f ms" % (cfg.name, warm_ms))
    ab = algorithmic_bytes(cfg)
    k_ms, k_min = time_score_kernel(dc, score_launches)
    per_launch = cfg.B * cfg.M * cfg.HI * cfg.DI + cfg.B * (cfg.HI * cfg.DI + cfg.HI * 4)
    log("%s: scan kernel mean %.3f ms (min %.3f) per launch" % (cfg.name, k_ms, k_min))
    res = dict(cfg=cfg, case=case, ms=ms, per_layer_ms=per_layer, step_ms_all=all_steps,
               warm_ms=warm_ms, wall=wall, bytes=ab, k_ms=k_ms, per_launch=per_launch)
    if detail:
        rw_ms, rw_layers, _ = cold_layers_ms(dc, max(10, steps // 2), write=True)
        res["rw_sweep_ms"], res["rw_sweep_layers_ms"] = rw_ms, rw_layers
        log("%s: step after read-write sweeps %.3f ms (layers %s)" % (
            cfg.name, rw_ms, ["%.4f" % x for x in rw_layers]))
        dc.prepare_decode(idx_for_reuse=False)
        res["all_full_ms"] = all_full_ms(dc, max(5, steps // 2), 2)
        log("%s: all-Full schedule %.3f ms (warm)" % (cfg.name, res["all_full_ms"]))
    del dc
    torch.cuda.empty_cache()
    return res


def measure_append(ci: int, launches: int = 10):
    """Write side at a decode workload's pool shape: a bulk append of 4096 new
    entries per sequence (GB/s of fp32 inputs read + encoded bytes written), one
    new entry per sequence (latency), and 4096 window rows per sequence."""
    import torch
    from fp4_kv_cache_score_amd import _lib as C
    from fp4_kv_cache_score_amd.configs import CONFIGS
    cfg = CONFIGS[ci]
    B, M, T = cfg.B, cfg.M, 4096
    lat = torch.zeros((B, M, cfg.D // 2), dtype=torch.uint8, device="cuda")
    sc = torch.zeros((B, M, cfg.D // 32), dtype=torch.uint8, device="cuda")
    key = torch.zeros((B, M, cfg.HI, cfg.DI), dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(1)
    xl = torch.randn((B, T, cfg.D), device="cuda", generator=g)
    xk = torch.randn((B, T, cfg.HI, cfg.DI), device="cuda", generator=g)
    slot = torch.arange(T, dtype=torch.int32, device="cuda").repeat(B, 1).contiguous()
    ring = torch.zeros((B, cfg.W, cfg.D), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(2):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(launches):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / launches

    bulk = timed(lambda: C.csa2_pool_append(lat, sc, key, B, M, xl, xk, slot, T, stream))
    one = timed(lambda: C.csa2_pool_append(lat, sc, key, B, M, xl, xk, slot, 1, stream))
    win = timed(lambda: C.csa2_swa_append(ring, B, cfg.W, xl, 0, T, stream))
    per_entry = cfg.D * 4 + cfg.HI * cfg.DI * 4 + 4 + cfg.D // 2 + cfg.D // 32 + cfg.HI * cfg.DI
    bulk_bytes = B * T * per_entry
    win_bytes = B * cfg.W * cfg.D * 5        # only the last W rows are encoded
    return dict(entries=B * T, bulk_ms=bulk, bulk_gbs=bulk_bytes / (bulk * 1e-3) / 1e9,
                bulk_frac_of_peak=bulk_bytes / (bulk * 1e-3) / 1e9 / HBM_PEAK_GBS,
                one_entry_per_sequence_us=one * 1e3, window_rows=B * T,
                window_ms=win, window_gbs=win_bytes / (win * 1e-3) / 1e9)


def measure_ragged(ci: int, steps: int, warmup: int):
    """A ragged batch at a decode workload's shape: sequence b holds a seeded
    uniform share of the M entry slots (M/8 .. M); step time and the step's
    algorithmic bytes (scans and candidate gathers scale with each length)."""
    import torch
    from fp4_kv_cache_score_amd import synth
    from fp4_kv_cache_score_amd.configs import CONFIGS, algorithmic_bytes
    from fp4_kv_cache_score_amd.device import DeviceCase
    cfg = CONFIGS[ci]
    rng = np.random.default_rng(cfg.seed + 1000)
    lens = rng.integers(cfg.M // 8, cfg.M + 1, cfg.B)
    dc = DeviceCase(synth.make_case(cfg))
    dc.use_lengths(lens)
    ms, _ = time_decode(dc, steps, warmup)
    full = algorithmic_bytes(cfg)
    frac = float(lens.sum()) / (cfg.B * cfg.M)
    ragged_bytes = full["total"] - full["scan"] * (1.0 - frac)
    del dc
    torch.cuda.empty_cache()
    return dict(lengths_mean=float(lens.mean()), lengths_min=int(lens.min()),
                lengths_max=int(lens.max()), ms_per_step=ms,
                query_tokens_per_s=cfg.B / (ms * 1e-3),
                step_hbm_gbs=ragged_bytes / (ms * 1e-3) / 1e9)


def measure_paged(ci: int, steps: int, warmup: int, page_log2: int = 8):
    """A paged pool at a decode workload's shape: every sequence's entries in
    pages of 2^page_log2 entries at shuffled places of one shared array, read
    through a page table; step time against the same pool laid out contiguously."""
    import torch
    from fp4_kv_cache_score_amd import synth
    from fp4_kv_cache_score_amd.configs import CONFIGS, algorithmic_bytes
    from fp4_kv_cache_score_amd.device import DeviceCase
    cfg = CONFIGS[ci]
    dc = DeviceCase(synth.make_case(cfg))
    dc.use_pages(page_log2, seed=cfg.seed)
    ms, _ = time_decode(dc, steps, warmup)
    del dc
    torch.cuda.empty_cache()
    return dict(page_entries=1 << page_log2, ms_per_step=ms,
                query_tokens_per_s=cfg.B / (ms * 1e-3),
                step_hbm_gbs=algorithmic_bytes(cfg)["total"] / (ms * 1e-3) / 1e9)


def measure_fused_select(ci: int, steps: int, warmup: int):
    """The Full layer's index work at a decode workload's shape, two ways: the
    scan writing the scores then the Top-K select (what csa2_decode_layers
    runs), and the fused single pass of csa2_score_topk (no score round trip)."""
    import torch
    from fp4_kv_cache_score_amd import _lib as C
    from fp4_kv_cache_score_amd import synth
    from fp4_kv_cache_score_amd.configs import CONFIGS
    from fp4_kv_cache_score_amd.device import DeviceCase
    cfg = CONFIGS[ci]
    if C.csa2_workspace_bytes(C.CSA2_OP_SCORE_TOPK, cfg.B, 1, cfg.M, cfg.K, 0, 0, 0) == 0:
        return None
    dc = DeviceCase(synth.make_case(cfg))
    d = dc.layers[0]
    scores = torch.empty((cfg.B, cfg.M), dtype=torch.float32, device="cuda")
    nb = C.csa2_workspace_bytes(C.CSA2_OP_TOPK, cfg.B, 1, cfg.M, cfg.K, 0, 0, 0)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
    idx = torch.empty((cfg.B, cfg.K), dtype=torch.int32, device="cuda")

    def two_pass():
        C.csa2_index_score(dc.pool, d["q_idx"], d["w_idx"], 1, -1, 1, None, 0, scores, None)
        C.csa2_topk(scores, cfg.B, cfg.M, None, None, cfg.K, idx, ws, nb)

    two = _time_calls(two_pass, steps, warmup)
    fused = _time_calls(lambda: dc.score_topk(0), steps, warmup)
    del dc
    torch.cuda.empty_cache()
    return dict(two_pass_ms=two, fused_ms=fused,
                note="csa2_decode_layers runs the two-pass form (the faster one here)")


def measure_host_tier(ci: int, reps: int = 5):
    """Host tier at a decode workload's pool shape: one sequence's whole pool
    (M entries x 784 B) restored from / offloaded to page-locked host memory,
    alone, and restored on a second stream while decode steps run."""
    import torch
    from fp4_kv_cache_score_amd import _lib as C
    from fp4_kv_cache_score_amd import synth
    from fp4_kv_cache_score_amd.configs import CONFIGS
    from fp4_kv_cache_score_amd.device import DeviceCase
    cfg = CONFIGS[ci]
    dc = DeviceCase(synth.make_case(cfg))
    dc.prepare_decode()
    B, M = cfg.B, cfg.M
    widths = (cfg.D // 2, cfg.D // 32, cfg.HI * cfg.DI)
    host = [torch.empty((M, w), dtype=torch.uint8, pin_memory=True) for w in widths]
    seq_bytes = M * sum(widths)
    side = torch.cuda.Stream()

    def copy_ms(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        fn(0)
        side.synchronize()
        e0.record(side)
        for k in range(n):
            fn(k % B)
        e1.record(side)
        side.synchronize()
        return e0.elapsed_time(e1) / n

    off = copy_ms(lambda b: C.csa2_pool_offload(dc.latent, dc.scale, dc.idx_key, B, M, b, 0, M,
                                                host[0], host[1], host[2], side), reps)
    res = copy_ms(lambda b: C.csa2_pool_restore(dc.latent, dc.scale, dc.idx_key, B, M, b, 0, M,
                                                host[0], host[1], host[2], side), reps)
    # decode alone, then decode while restores stream in on the side stream
    steps = 40
    alone, _ = time_decode(dc, steps, 3)
    main = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    r0 = torch.cuda.Event(enable_timing=True)
    r1 = torch.cuda.Event(enable_timing=True)
    n_res = max(1, int(round(steps * alone / max(res, 1e-3))))
    torch.cuda.synchronize()
    r0.record(side)
    for k in range(n_res):
        C.csa2_pool_restore(dc.latent, dc.scale, dc.idx_key, B, M, k % B, 0, M,
                            host[0], host[1], host[2], side)
    r1.record(side)
    e0.record(main)
    for _ in range(steps):
        dc.decode_layers(main)
    e1.record(main)
    torch.cuda.synchronize()
    busy = e0.elapsed_time(e1) / steps
    rtime = r0.elapsed_time(r1)
    del dc
    torch.cuda.empty_cache()
    return dict(sequence_bytes=seq_bytes, bytes_per_token=sum(widths) / cfg.ratio,
                restore_ms=res, restore_gbs=seq_bytes / (res * 1e-3) / 1e9,
                offload_ms=off, offload_gbs=seq_bytes / (off * 1e-3) / 1e9,
                decode_ms_alone=alone, decode_ms_with_restores=busy,
                restores_during_decode=n_res,
                restore_gbs_during_decode=n_res * seq_bytes / (rtime * 1e-3) / 1e9)


def step_detail(r) -> dict:
    """Cold per-layer, warm and all-Full figures of a decode workload."""
    B = r["cfg"].B
    d = dict(mall_cold_ms_per_step=r["ms"], mall_cold_query_tokens_per_s=B / (r["ms"] * 1e-3),
             mall_cold_per_layer_ms=r["per_layer_ms"],
             mall_cold_step_ms_min_max=[min(r["step_ms_all"]), max(r["step_ms_all"])],
             warm_ms_per_step=r["warm_ms"], warm_query_tokens_per_s=B / (r["warm_ms"] * 1e-3),
             warm_step_frac_of_peak=r["bytes"]["total"] / (r["warm_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS)
    if "rw_sweep_ms" in r:
        d.update(read_write_sweep_ms_per_step=r["rw_sweep_ms"],
                 read_write_sweep_per_layer_ms=r["rw_sweep_layers_ms"])
    if "all_full_ms" in r:
        d.update(all_full_ms_per_step=r["all_full_ms"],
                 all_full_query_tokens_per_s=B / (r["all_full_ms"] * 1e-3))
    return d


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1, help="headline workload (config index)")
    ap.add_argument("--extra", type=int, nargs="*", default=[2, 3],
                    help="further decode configs measured into 'extra'")
    ap.add_argument("--prefill", type=int, nargs="*", default=[4],
                    help="chunked-prefill configs measured into 'extra'")
    ap.add_argument("--score-launches", type=int, default=20)
    ap.add_argument("--cpu-budget", type=float, default=8.0,
                    help="seconds of CPU oracle work per baseline workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the chunked-prefill measurement of --prefill configs, without "
                         "the whole-context loop (for a counter pass)")
    ap.add_argument("--step-only", action="store_true",
                    help="only time --steps decode steps of --config (for a counter pass)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="first run a 1 GiB device-to-device copy 3 times (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(decode would shard by sequence, one process per GPU). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    from fp4_kv_cache_score_amd import _lib
    _lib.lib()
    if args.copy_calib:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("copy calibration: 3 x 1 GiB device copies done")

    if args.prefill_only:   # a counter pass over prefill chunks alone
        for ci in args.prefill:
            r = measure_prefill(ci, args.steps, args.warmup, context=False)
            r.pop("case")
            print(json.dumps({"workload": r.pop("workload"), **r}), flush=True)
        return

    if args.step_only:   # a counter pass over decode steps alone
        from fp4_kv_cache_score_amd import synth
        from fp4_kv_cache_score_amd.configs import CONFIGS
        from fp4_kv_cache_score_amd.device import DeviceCase
        dc = DeviceCase(synth.make_case(CONFIGS[args.config]))
        ms, _ = time_decode(dc, args.steps, args.warmup)
        print(json.dumps({"workload": CONFIGS[args.config].name, "steps": args.steps,
                          "warmup": args.warmup, "ms_per_step": ms}), flush=True)
        return

    head = measure(args.config, args.steps, args.warmup, args.score_launches, detail=True)
    cfg = head["cfg"]
    value = cfg.B / (head["ms"] * 1e-3)      # the MALL-cold step (sum of per-layer times)
    cpu_cases = {cfg.name: head["case"]}
    achieved = head["per_launch"] / (head["k_ms"] * 1e-3) / 1e9
    traffic = recorded_traffic(cfg.name)
    step_gbs = head["bytes"]["total"] / (head["ms"] * 1e-3) / 1e9
    extra = {}
    for ci in args.extra:
        if ci == args.config:
            continue
        r = measure(ci, args.steps, args.warmup, args.score_launches, detail=ci in (1, 2))
        c = r["cfg"]
        if ci == 2:
            cpu_cases[c.name] = r["case"]
        extra[c.name] = dict(
            query_tokens_per_s=c.B / (r["ms"] * 1e-3), ms_per_step=r["ms"],
            step_hbm_gbs=r["bytes"]["total"] / (r["ms"] * 1e-3) / 1e9,
            step_frac_of_peak=r["bytes"]["total"] / (r["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            algorithmic_bytes_per_step=r["bytes"]["total"],
            scan_kernel_ms=r["k_ms"],
            scan_kernel_gbs=r["per_launch"] / (r["k_ms"] * 1e-3) / 1e9)
        extra[c.name].update(step_detail(r))
        del r
    for ci in args.prefill:
        r = measure_prefill(ci, max(3, args.steps // 5), 2)
        cpu_cases[r["workload"]] = r.pop("case")
        extra[r.pop("workload")] = r
        log("prefill: %.3f ms/step %s" % (r["ms_per_step"], r["stage_ms"]))
    extra[cfg.name] = step_detail(head)
    ap_res = measure_append(args.config)
    extra["pool_append_" + cfg.name] = ap_res
    rg = measure_ragged(args.config, args.steps, args.warmup)
    extra["ragged_" + cfg.name] = rg
    log("ragged batch (mean length %.0f of %d): %.3f ms/step, %.1f GB/s" % (
        rg["lengths_mean"], cfg.M, rg["ms_per_step"], rg["step_hbm_gbs"]))
    pg = measure_paged(args.config, args.steps, args.warmup)
    extra["paged_" + cfg.name] = pg
    log("paged pool (pages of %d entries): %.3f ms/step against %.3f contiguous (warm)" % (
        pg["page_entries"], pg["ms_per_step"], head["warm_ms"]))
    fz = measure_fused_select(args.config, args.steps, args.warmup)
    if fz:
        extra["fused_score_topk_" + cfg.name] = fz
        log("Full-layer index work: scan + select %.3f ms, fused single pass %.3f ms" % (
            fz["two_pass_ms"], fz["fused_ms"]))
    ht = measure_host_tier(args.config)
    extra["host_tier_" + cfg.name] = ht
    log("host tier: restore %.1f GB/s, offload %.1f GB/s; decode %.3f ms alone, %.3f ms beside "
        "restores (%.1f GB/s)" % (ht["restore_gbs"], ht["offload_gbs"], ht["decode_ms_alone"],
                                  ht["decode_ms_with_restores"], ht["restore_gbs_during_decode"]))
    log("pool append: %.1f GB/s bulk, %.1f us one entry per sequence" % (
        ap_res["bulk_gbs"], ap_res["one_entry_per_sequence_us"]))
    cpu = None
    if not args.no_cpu_baseline:
        per = {}
        for name, case in cpu_cases.items():
            per[name] = (cpu_prefill(case, args.cpu_budget) if case.cfg.Q > 1
                         else cpu_decode(case, args.cpu_budget))
            log("cpu oracle %s: %.3g query-tokens/s" % (name, per[name]["value"]))
        cpu = dict(per[cfg.name])
        cpu.update(host_info())
        cpu["per_workload"] = per

    out = {
        "metric": "CSA2 decode query-tokens/s at 128K ctx (achieved HBM GB/s vs peak)",
        "value": value,
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "operand_formats": "E4M3 index keys and window, E2M1 + E8M0 latent, bf16 queries; "
                           "f32 accumulation (attention: bf16 matrix products of exactly "
                           "dequantised keys, softmax weights split into bf16 hi + lo)",
        "data": "synthetic (seeded N(0,1) pool and queries, MXFP4 / E4M3 encoded)",
        "config": {"workload": cfg.name, "batch": cfg.B, "pool_entries": cfg.M, "K": cfg.K,
                   "P": cfg.P, "W": cfg.W, "heads": cfg.H, "d": cfg.D,
                   "layers": "/".join({0: "Full", 1: "Reindex", 2: "Reuse"}[m] for m in cfg.modes)},
        "timing": "MALL-cold: a 512 MiB read sweep before every layer (outside the timed "
                  "region), each layer alone between HIP events, a step = the sum of its "
                  "layers, median of the timed steps; warm back-to-back steps and steps after "
                  "read-write sweeps in extra",
        "step_hbm_gbs": step_gbs,
        "step_frac_of_peak": step_gbs / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": head["bytes"]["total"],
        "roofline": {"bound": "hbm", "kernel": SCAN_VARIANT,
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "bytes_per_launch": head["per_launch"], "mean_launch_ms": head["k_ms"]},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
