"""Comparison rules shared by the GPU parity tests.

* Attention outputs: per (row, head) max_i |g_i - o_i| / max_i |o_i| <= 2e-3
  (the oracle is fp64; the kernels accumulate in fp32).
* Top-K sets: exact, except rows whose oracle K-th and (K+1)-th scores differ
  by less than 1e-4 relative; those are counted and their actual mismatches
  reported.  Exactness without that excuse is checked separately by running
  the oracle's Top-K on the GPU's own fp32 scores.
* Indexer scores: |g - s| <= 72 * 2^-24 * sum_h w_h sum_i |qI kI| + 2^-50 |s|,
  a bound that holds for any fp32 summation order: the E4M3 products are exact,
  a 64-term dot adds at most 63 roundings, then one for the head weight and
  seven for the 8-head sum.
"""
import numpy as np

from oracle import formats as F

ATTN_TOL = 2e-3
GAP_TOL = 1e-4


def attn_rel_err(g, o) -> float:
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    num = np.abs(g - o).max(axis=-1)
    den = np.abs(o).max(axis=-1)
    r = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return float(r.max()) if r.size else 0.0


def score_bound(idx_key, q_idx, w_idx, s_exact, rows=None):
    k = F.e4m3_value(idx_key if rows is None else idx_key[rows])
    q = F.e4m3_value(q_idx)
    mag = np.einsum("nhi,hi->nh", np.abs(k), np.abs(q))
    return 72 * 2.0 ** -24 * (mag * np.abs(np.asarray(w_idx, np.float64))).sum(1) + \
        2.0 ** -50 * np.abs(s_exact)


class TieReport:
    def __init__(self):
        self.rows = 0
        self.excused = 0
        self.excused_mismatch = 0

    def check(self, g_idx, o_idx, gap, where=""):
        self.rows += 1
        same = np.array_equal(np.asarray(g_idx), np.asarray(o_idx))
        if gap is not None and gap < GAP_TOL:
            self.excused += 1
            if not same:
                self.excused_mismatch += 1
            return
        assert same, "Top-K mismatch %s (gap %r)" % (where, gap)

    def __str__(self):
        return "rows=%d near-tie rows=%d mismatches among them=%d" % (
            self.rows, self.excused, self.excused_mismatch)
