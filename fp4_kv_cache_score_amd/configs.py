"""Workload shapes of the CSA2 decode / chunked-prefill hot path.

CSA2 gives every layer one of three static modes over one shared global KV
pool: Full (score the whole pool with the indexer and pick Top-K), Reindex
(re-score with the layer's own indexer query and pick a new Top-K) and Reuse
(take the indices of an earlier layer).  Sources: "DeepSeek V4.1-Flash Cuts KV
Cache by 437x With New CED and CSA2 Architecture" (paragraph on CSA2's three
operating modes and the hierarchical sparse indexer) and "DeepSeek V4.1 Flash
Architecture Breakdown" (section "How does the cache compress along three
dimensions at once?").  The pages give no sizes; the shapes below are the
synthetic workloads this library is measured on.
"""
from __future__ import annotations

from dataclasses import dataclass, field

FULL, REINDEX, REUSE = 0, 1, 2
MODE_NAMES = {FULL: "Full", REINDEX: "Reindex", REUSE: "Reuse"}


@dataclass(frozen=True)
class CaseConfig:
    name: str
    seed: int
    B: int                      # sequences in the batch
    M: int                      # global pool entries per sequence
    K: int                      # Top-K selected entries
    modes: tuple                # static per-layer schedule
    H: int = 16                 # attention heads
    D: int = 512                # latent width (shared K/V)
    HI: int = 8                 # indexer heads
    DI: int = 64                # indexer head width
    W: int = 128                # FP8 sliding-window rows
    P: int = 0                  # hierarchical candidate pool size (0: flat)
    Q: int = 1                  # query tokens per sequence (1: decode)
    ratio: int = 4              # tokens per compressed pool entry
    causal: bool = False        # prefill: restrict entries to those visible
    chunk_pos: int = -1         # prefill: first token's position (< 0: the newest Q tokens)
    plant_frac: float = 0.01    # share of planted (scaled) pool entries
    plant_mult: float = 3.0     # their pre-quantisation multiplier

    @property
    def L(self) -> int:
        return len(self.modes)

    @property
    def pos0(self) -> int:
        """Position of the first query token of the chunk (-1: no causal limit).

        The chunk starts at chunk_pos when that is given; otherwise it is the
        newest Q tokens of a context of ratio*M tokens.
        """
        if not self.causal:
            return -1
        return self.chunk_pos if self.chunk_pos >= 0 else self.ratio * self.M - self.Q

    def scaled(self, **kw) -> "CaseConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return CaseConfig(**d)


def _sched20():
    m = [REUSE] * 20
    m[0] = m[10] = FULL
    m[5] = m[15] = REINDEX
    return tuple(m)


CONFIGS = [
    CaseConfig("tiny_full_M1024", seed=0, B=1, M=1024, K=64, modes=(FULL,)),
    CaseConfig("decode_128k_B32", seed=1, B=32, M=32768, K=512,
               modes=(FULL, REINDEX, REUSE, REUSE)),
    CaseConfig("decode_1m_hier_B8", seed=2, B=8, M=262144, K=512, P=8192,
               modes=(FULL, REINDEX, REINDEX, REINDEX)),
    CaseConfig("decode_sched20_B64", seed=3, B=64, M=65536, K=512,
               modes=_sched20()),
    CaseConfig("prefill_2048_M65536", seed=4, B=1, M=65536, K=512, Q=2048,
               modes=(FULL,), causal=True),
]


def config(i: int) -> CaseConfig:
    return CONFIGS[i]


def algorithmic_bytes(cfg: CaseConfig) -> dict:
    """Bytes the decode step must move, each once (intermediate scores excluded).

    Per pool entry: 256 B E2M1 latent + 16 B E8M0 scales + HI*DI B E4M3 key.
    Returns a breakdown and the total for one step over all layers.
    """
    B, M, K, D, W, H = cfg.B, cfg.M, cfg.K, cfg.D, cfg.W, cfg.H
    key_row = cfg.HI * cfg.DI
    lat_row = D // 2 + D // 32
    out = dict(scan=0, cand_gather=0, cand_idx=0, attention=0, queries=0)
    for ell, mode in enumerate(cfg.modes):
        if mode in (FULL, REINDEX):
            out["queries"] += B * (key_row + cfg.HI * 4)
            if cfg.P > 0 and mode == REINDEX:
                out["cand_gather"] += B * cfg.P * key_row
                out["cand_idx"] += B * cfg.P * 4
            else:
                out["scan"] += B * M * key_row
        # gathered latent+scales, SWA rows, q (bf16), o (f32), lse, idx
        out["attention"] += B * (K * lat_row + W * D + H * D * 2
                                 + H * D * 4 + H * 4 + K * 4)
    out["total"] = sum(out.values())
    return out
