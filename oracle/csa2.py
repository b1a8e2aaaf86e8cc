"""CPU oracle of the CSA2 decode / chunked-prefill hot path (NumPy, fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What the pages fix, restated:
* One global KV pool serves every layer, and Top-K indices are reused across
  layers ("Inside the DeepSeek-V4.1-Flash Tech Report", section "KV Cache:
  Three Techniques to 890 Bytes per Token"; "DeepSeek V4.1-Flash Cuts KV Cache
  by 437x", paragraph on CSA2 storage).
* Each layer runs in one static mode: Full scores the whole context with the
  indexer and selects Top-K; Reindex keeps the Full layer's KV but re-scores
  with its own indexer and selects a new Top-K; Reuse does no index work and
  takes the indices of an earlier layer ("... Cuts KV Cache by 437x",
  paragraph on the three operating modes; "DeepSeek V4.1 Flash Architecture
  Breakdown", section "How does the cache compress along three dimensions at
  once?").
* For very long contexts the Full layer builds a reduced candidate pool and
  later layers retrieve and score only inside it (same two passages).
* Global entries are FP4 (E2M1) restored to real values for the computation;
  the sliding-window rows are FP8 (paragraph on FP4 quantisation; section "How
  are cache precision and storage arranged?").
* The window handles nearby tokens next to the sparse global entries
  ("... Cuts KV Cache by 437x", paragraph on sliding window attention); no
  absolute-position scheme is applied (paragraph on CSA2 storage).

Readings where the pages are silent (each is a choice, not a quotation):
* Indexer score of pool entry j: s_j = sum_h w_h * ReLU(sum_i qI[h,i]*kI[j,h,i])
  over 8 indexer heads of width 64, E4M3 keys and queries, fp32 head weights.
* Top-K: the K largest scores, equal scores broken toward the lower *global*
  pool index, returned as ascending global indices padded with -1 when fewer
  than K entries are eligible.
* Reuse takes the indices of the most recent Full or Reindex layer; the first
  layer must be Full.  All layers read the same pool.
* Attention per head h over the union of the selected latent rows and the W
  window rows, keys and values both the 512-wide row (shared K/V), logit
  z = q_h . key with scale 1 (the query already carries 1/sqrt(d)):
  o_h = sum softmax(z) * key, lse_h = log sum exp(z).  No de-duplication.
* Chunked prefill: query t of a chunk of Q sits at position pos0 + t; pool
  entry j covers tokens [ratio*j, ratio*j + ratio - 1] and is visible once its
  last token is, so the query sees the first min(M, (pos0+t+1)//ratio) entries;
  its window is rows t .. t+W-1 of a [Q+W-1] buffer of the newest tokens,
  of which rows before the context's first token do not exist (a first
  chunk).  A chunk runs the whole layer schedule token by token; it builds no
  candidate pool (that serves one decode token's indexing cost, while a
  chunk's scan of the pool is shared by its Q queries).

Exactness: E4M3 values are integer multiples of 2^-9 with magnitude at most
448, so each product is a multiple of 2^-18 below 2^18 and any sum of 64 of
them is exactly representable in fp64 (below 2^42 < 2^53).  The per-head dot
is therefore exact whatever the summation order (including BLAS).
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_value, dequant_latent, e4m3_value

FULL, REINDEX, REUSE = 0, 1, 2


# ---------------------------------------------------------------------------
# Indexer score
# ---------------------------------------------------------------------------

def index_scores(idx_key, q_idx, w_idx, rows=None, chunk: int = 8192) -> np.ndarray:
    """Indexer scores of pool rows (all rows, or the given row numbers).

    idx_key: uint8 E4M3 [M][HI][DI]; q_idx: uint8 E4M3 [HI][DI];
    w_idx: float32 [HI]; rows: optional int array of pool rows.
    Returns fp64 [N].  The per-head dot is exact; ReLU maps x<=0 to +0.
    """
    q = e4m3_value(q_idx)                       # [HI][DI]
    w = np.asarray(w_idx, dtype=np.float64)     # [HI]
    n = idx_key.shape[0] if rows is None else len(rows)
    out = np.empty(n, np.float64)
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        sel = slice(a, b) if rows is None else np.asarray(rows[a:b])
        k = e4m3_value(idx_key[sel])            # [n][HI][DI]
        dots = np.einsum("nhi,hi->nh", k, q)    # exact
        relu = np.where(dots > 0, dots, 0.0)
        out[a:b] = (relu * w).sum(axis=1)
    return out


def index_dots_bruteforce(idx_key, q_idx) -> np.ndarray:
    """Per-head dots via int64 arithmetic on the integers v * 2^9 (tiny inputs)."""
    ki = np.rint(e4m3_value(idx_key) * 512).astype(np.int64)
    qi = np.rint(e4m3_value(q_idx) * 512).astype(np.int64)
    n, hi, di = ki.shape
    d = np.zeros((n, hi), np.int64)
    for j in range(n):
        for h in range(hi):
            acc = 0
            for i in range(di):
                acc += int(ki[j, h, i]) * int(qi[h, i])
            d[j, h] = acc
    return d  # true dot = d * 2^-18


# ---------------------------------------------------------------------------
# Top-K
# ---------------------------------------------------------------------------

def topk(scores, K: int, n_valid=None):
    """Positions of the K largest of scores[:n_valid], lower position first on ties.

    Returns (positions ascending, padded with -1 to length K; gap), where gap is
    (s_K - s_{K+1}) / s_K for the K-th and (K+1)-th largest, or None when no
    (K+1)-th entry exists.
    """
    s = np.asarray(scores, dtype=np.float64)
    n = len(s) if n_valid is None else max(0, min(int(n_valid), len(s)))
    if K <= 0:
        raise ValueError("K must be positive")
    order = np.argsort(-s[:n], kind="stable")   # descending, stable on ties
    take = np.sort(order[:min(K, n)])
    out = np.full(K, -1, np.int64)
    out[:len(take)] = take
    gap = None
    if n > K:
        a, b = s[order[K - 1]], s[order[K]]
        gap = (a - b) / a if a > 0 else (0.0 if a == b else np.inf)
    return out, gap


def topk_bruteforce(scores, K: int, n_valid=None) -> np.ndarray:
    """Tiny-input cross-check: pick the best remaining entry K times."""
    s = [float(x) for x in np.asarray(scores, dtype=np.float64)]
    n = len(s) if n_valid is None else min(int(n_valid), len(s))
    chosen = []
    for _ in range(min(K, n)):
        best = None
        for j in range(n):
            if j in chosen:
                continue
            if best is None or s[j] > s[best]:
                best = j
        chosen.append(best)
    out = sorted(chosen) + [-1] * (K - len(chosen))
    return np.asarray(out, np.int64)


def map_positions(pos, cand) -> np.ndarray:
    """Candidate-pool positions -> global pool indices (-1 stays -1)."""
    pos = np.asarray(pos)
    cand = np.asarray(cand)
    if cand.size == 0:                      # an empty candidate list selects nothing
        return np.full(pos.shape, -1, np.int64)
    return np.where(pos >= 0, cand[np.maximum(pos, 0)], -1)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def gather_keys(latent, scale, idx, swa_rows=None) -> np.ndarray:
    """Union of the selected FP4 global rows (idx != -1) and the FP8 window rows."""
    idx = np.asarray(idx)
    sel = idx[idx >= 0]
    parts = [dequant_latent(latent[sel], scale[sel])]
    if swa_rows is not None and len(swa_rows) > 0:
        parts.append(e4m3_value(swa_rows))
    return np.concatenate(parts, axis=0) if parts else np.zeros((0, latent.shape[-1] * 2))


def attend(q_bits, keys):
    """Single-softmax attention of every head over one key set (keys = values).

    q_bits: bf16 bit patterns [H][D]; keys: fp64 [N][D].
    Returns (o fp64 [H][D], lse fp64 [H]); an empty key set gives o = 0, lse = -inf.
    """
    q = bf16_value(q_bits)
    H, D = q.shape
    if keys.shape[0] == 0:
        return np.zeros((H, D)), np.full(H, -np.inf)
    z = q @ keys.T                               # [H][N]
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ keys) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def lse_merge(o1, lse1, o2, lse2):
    """Combine two attention results over disjoint key sets into one softmax."""
    lse = np.logaddexp(lse1, lse2)
    a = np.where(np.isfinite(lse1), np.exp(lse1 - lse), 0.0)[:, None]
    b = np.where(np.isfinite(lse2), np.exp(lse2 - lse), 0.0)[:, None]
    return a * o1 + b * o2, lse


def swa_merge(q_bits, swa_rows, o_in, lse_in):
    """Attention over the FP8 window merged into an earlier result (o_in, lse_in)."""
    o2, l2 = attend(q_bits, e4m3_value(swa_rows))
    return lse_merge(np.asarray(o_in, np.float64), np.asarray(lse_in, np.float64), o2, l2)


# ---------------------------------------------------------------------------
# Layer schedule (decode, one sequence)
# ---------------------------------------------------------------------------

def decode_sequence(latent, scale, idx_key, layers, K: int, P: int = 0):
    """Run the static mode schedule for one sequence's single decode token.

    latent [M][D/2], scale [M][D/32], idx_key [M][HI][DI] describe the pool;
    layers is a list of dicts with keys mode, q_idx [HI][DI], w_idx [HI],
    q [H][D] (bf16 bits) and swa [W][D].  P > 0 enables the hierarchical
    candidate pool built by the Full layer.
    Returns a list of per-layer dicts: idx (global, ascending, -1 padded),
    o, lse, and for indexing layers the scores, gap and (hierarchical Full)
    cand.
    """
    out = []
    src_idx = None
    cand = None
    for ell, L in enumerate(layers):
        rec = {"mode": L["mode"]}
        mode = L["mode"]
        if mode == FULL:
            s = index_scores(idx_key, L["q_idx"], L["w_idx"])
            if P > 0:
                cand, cand_gap = topk(s, P)
                rec["cand"] = cand
                rec["cand_gap"] = cand_gap
            idx, gap = topk(s, K)
            rec.update(scores=s, gap=gap)
        elif mode == REINDEX:
            if src_idx is None:
                raise ValueError("layer %d: Reindex before any Full layer" % ell)
            if P > 0:
                valid = cand[cand >= 0]
                s = index_scores(idx_key, L["q_idx"], L["w_idx"], rows=valid)
                pos, gap = topk(s, K)
                idx = map_positions(pos, valid)
            else:
                s = index_scores(idx_key, L["q_idx"], L["w_idx"])
                idx, gap = topk(s, K)
            rec.update(scores=s, gap=gap)
        elif mode == REUSE:
            if src_idx is None:
                raise ValueError("layer %d: Reuse before any Full layer" % ell)
            idx = src_idx.copy()
        else:
            raise ValueError("unknown mode %r" % (mode,))
        if mode != REUSE:
            src_idx = idx
        keys = gather_keys(latent, scale, idx, L["swa"])
        o, lse = attend(L["q"], keys)
        rec.update(idx=idx, o=o, lse=lse)
        out.append(rec)
    return out


# ---------------------------------------------------------------------------
# Causal chunked prefill (one sequence, one Full layer)
# ---------------------------------------------------------------------------

def visible_entries(M: int, pos: int, ratio: int) -> int:
    """Pool entries whose every token is at or before position pos."""
    return max(0, min(M, (pos + 1) // ratio))


def prefill_query(latent, scale, idx_key, q_idx_t, w_t, q_t, swa, t: int,
                  pos0: int, ratio: int, K: int, W: int):
    """One query token t of a causal prefill chunk (Full layer).

    q_idx_t [HI][DI], w_t [HI], q_t [H][D] bf16 bits, swa [Q+W-1][D].
    Returns dict(idx, o, lse, gap, vis).
    """
    M = idx_key.shape[0]
    vis = visible_entries(M, pos0 + t, ratio)
    s = index_scores(idx_key, q_idx_t, w_t, rows=np.arange(vis))
    idx, gap = topk(s, K)
    keys = gather_keys(latent, scale, idx, swa[t:t + W])
    o, lse = attend(q_t, keys)
    return dict(idx=idx, o=o, lse=lse, gap=gap, vis=vis, scores=s)


# ---------------------------------------------------------------------------
# Causal chunked prefill through the layer schedule (one sequence)
# ---------------------------------------------------------------------------

def window_first_row(t: int, W: int, pos0: int) -> int:
    """First of query t's window rows t .. t+W-1 that holds a token.

    Row t + r of the chunk's [Q+W-1] window buffer is token position
    pos0 + t - (W - 1) + r; positions below 0 do not exist (the start of the
    context).  pos0 < 0 means no causal limit: every row is a token.
    """
    if pos0 < 0:
        return 0
    return max(0, (W - 1) - (pos0 + t))


def prefill_layers(latent, scale, idx_key, layers, Q: int, pos0: int, ratio: int,
                   K: int, W: int):
    """The static mode schedule for a chunk of Q query tokens of one sequence.

    Every layer does what it does in decode, once per query token, with the
    causal limits of that token: query t at position pos0 + t selects among
    the first visible_entries(M, pos0 + t, ratio) pool entries (all M when
    pos0 < 0) and attends to its window rows from window_first_row on.  Full
    and Reindex layers score the visible entries with their own indexer and
    select Top-K; a Reuse layer takes, token by token, the indices of the most
    recent Full or Reindex layer.  (No candidate pool: see the hierarchical
    reading, which concerns one decode token's indexing cost.)

    layers: list of dicts with mode, q_idx [Q][HI][DI], w_idx [Q][HI],
    q [Q][H][D] bf16 bits, swa [Q+W-1][D] E4M3.
    Returns per layer a dict: idx [Q][K] (ascending, -1 padded), o [Q][H][D],
    lse [Q][H], gap [Q] (None where no (K+1)-th entry), vis [Q].
    """
    M = idx_key.shape[0]
    vis = np.array([M if pos0 < 0 else visible_entries(M, pos0 + t, ratio) for t in range(Q)])
    out = []
    src = None
    for ell, L in enumerate(layers):
        mode = L["mode"]
        rec = dict(mode=mode, vis=vis, gap=[None] * Q)
        if mode in (FULL, REINDEX):
            if mode == REINDEX and src is None:
                raise ValueError("layer %d: Reindex before any Full layer" % ell)
            idx = np.full((Q, K), -1, np.int64)
            for t in range(Q):
                s = index_scores(idx_key, L["q_idx"][t], L["w_idx"][t], rows=np.arange(vis[t]))
                idx[t], rec["gap"][t] = topk(s, K)
            src = idx
        elif mode == REUSE:
            if src is None:
                raise ValueError("layer %d: Reuse before any Full layer" % ell)
            idx = src.copy()
        else:
            raise ValueError("unknown mode %r" % (mode,))
        H, D = np.asarray(L["q"]).shape[1:]
        o = np.zeros((Q, H, D))
        lse = np.zeros((Q, H))
        for t in range(Q):
            r0 = window_first_row(t, W, pos0)
            keys = gather_keys(latent, scale, idx[t], L["swa"][t + r0:t + W])
            o[t], lse[t] = attend(L["q"][t], keys)
        rec.update(idx=idx, o=o, lse=lse)
        out.append(rec)
    return out
