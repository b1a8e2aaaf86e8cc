"""Seeded synthetic inputs for the CSA2 hot path (host bytes, shared by all sides).

This module only *produces* bytes: normal / uniform draws, the MXFP4 and E4M3
encoders that turn them into the stored formats, and bf16 rounding of queries.
It holds none of the read-side arithmetic (decoding, scoring, selection,
attention); both the HIP path and the CPU checker consume the same bytes.

Random streams: every tensor is drawn from
``numpy.random.default_rng(SeedSequence([seed, stream, *sub]))`` (PCG64), where
``stream`` is a fixed id per tensor kind and ``sub`` is (sequence) for pool
tensors and (layer, sequence) for per-layer tensors, so that any one sequence
can be regenerated on its own and the draws do not depend on batch size or
thread count.

Stream ids
    1  latent, N(0,1) float32 [M][D] before quantisation
    2  planted entries: round(plant_frac*M) entries chosen without replacement;
       their latent rows are multiplied by plant_mult before quantisation
    3  indexer keys, N(0,1) float32 [M][HI][DI] -> E4M3
    10 indexer query, N(0,1) [Q][HI][DI] -> E4M3   (Full / Reindex layers)
    11 indexer head weights, U(0,1) float32 [Q][HI]  (Full / Reindex layers)
    12 attention query, N(0,1)/sqrt(D) [Q][H][D] -> bf16
    13 sliding window, N(0,1) [Q+W-1][D] -> E4M3
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from .configs import CaseConfig, FULL, REINDEX, REUSE

S_LATENT, S_PLANT, S_KEY = 1, 2, 3
S_QIDX, S_W, S_Q, S_SWA = 10, 11, 12, 13


def _rng(*words) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(w) for w in words]))


# ---------------------------------------------------------------------------
# Encoders (write side of the formats; the read side lives elsewhere)
# ---------------------------------------------------------------------------

def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP E4M3 (float8_e4m3fn) bytes, clamped to +-448, RNE."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def encode_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def encode_mxfp4(x: np.ndarray):
    """float32 [..., D] -> (packed E2M1 codes uint8 [..., D/2], E8M0 uint8 [..., D/32]).

    OCP MX rule per block of 32 consecutive elements: shared exponent
    floor(log2(amax)) - 2 (E2M1's largest exponent is 2), elements divided by
    2^shared and rounded to nearest-even on the E2M1 grid, saturating at 6.
    An all-zero block gets scale code 127.  Element 2i goes to the low nibble
    of byte i, element 2i+1 to the high nibble.
    """
    x = np.asarray(x, dtype=np.float32)
    shp = x.shape
    D = shp[-1]
    assert D % 32 == 0
    blk = x.reshape(-1, D // 32, 32)
    amax = np.abs(blk).max(axis=-1)
    _, e = np.frexp(amax)                       # amax = f * 2^e, f in [0.5, 1)
    shared = np.where(amax > 0, e.astype(np.int32) - 1 - 2, 0)
    shared = np.clip(shared, -127, 127)
    scode = (shared + 127).astype(np.uint8)
    y = np.ldexp(blk, -shared[..., None]).astype(np.float64)
    mag = np.abs(y)
    # Round to nearest-even on the E2M1 magnitude grid: step 0.5 below 2,
    # step 1 in [2,4), step 2 from 4, saturate at 6.
    q = np.where(mag < 2.0, np.rint(mag * 2.0) / 2.0,
                 np.where(mag < 4.0, np.rint(mag), 2.0 * np.rint(mag / 2.0)))
    q = np.minimum(q, 6.0)
    code = np.where(q < 2.0, q * 2.0,
                    np.where(q < 4.0, 4.0 + (q - 2.0), 6.0 + (q - 4.0) / 2.0))
    code = code.astype(np.uint8) | (np.signbit(y).astype(np.uint8) << 3)
    code = code.reshape(*shp[:-1], D)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, scode.reshape(*shp[:-1], D // 32)


# ---------------------------------------------------------------------------
# Case containers
# ---------------------------------------------------------------------------

@dataclass
class HostPool:
    latent: np.ndarray   # uint8 [B][M][D/2]
    scale: np.ndarray    # uint8 [B][M][D/32]
    idx_key: np.ndarray  # uint8 [B][M][HI][DI]
    planted: np.ndarray  # int64 [B][n_plant]  (for reference only)


@dataclass
class HostLayer:
    mode: int
    q_idx: Optional[np.ndarray]   # uint8 [B][Q][HI][DI] (None for Reuse)
    w_idx: Optional[np.ndarray]   # float32 [B][Q][HI]
    q: np.ndarray                 # uint16 bf16 bits [B][Q][H][D]
    swa: np.ndarray               # uint8 [B][Q+W-1][D]


@dataclass
class HostCase:
    cfg: CaseConfig
    pool: HostPool
    layers: List[HostLayer]


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _pool_seq(cfg: CaseConfig, b: int, lat, sc, key, planted, chunk=16384):
    M, D = cfg.M, cfg.D
    n_plant = int(round(cfg.plant_frac * M))
    pl = np.sort(_rng(cfg.seed, S_PLANT, b).choice(M, size=n_plant, replace=False)) \
        if n_plant > 0 else np.zeros(0, np.int64)
    planted[b, :n_plant] = pl
    mult = np.ones(M, np.float32)
    mult[pl] = cfg.plant_mult
    g = _rng(cfg.seed, S_LATENT, b)
    for j0 in range(0, M, chunk):
        j1 = min(M, j0 + chunk)
        x = g.standard_normal((j1 - j0, D), dtype=np.float32)
        x *= mult[j0:j1, None]
        lat[b, j0:j1], sc[b, j0:j1] = encode_mxfp4(x)
    g = _rng(cfg.seed, S_KEY, b)
    for j0 in range(0, M, chunk):
        j1 = min(M, j0 + chunk)
        x = g.standard_normal((j1 - j0, cfg.HI, cfg.DI), dtype=np.float32)
        key[b, j0:j1] = encode_e4m3(x)


def make_pool(cfg: CaseConfig) -> HostPool:
    B, M, D = cfg.B, cfg.M, cfg.D
    lat = np.empty((B, M, D // 2), np.uint8)
    sc = np.empty((B, M, D // 32), np.uint8)
    key = np.empty((B, M, cfg.HI, cfg.DI), np.uint8)
    planted = np.zeros((B, int(round(cfg.plant_frac * M))), np.int64)
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(lambda b: _pool_seq(cfg, b, lat, sc, key, planted), range(B)))
    return HostPool(lat, sc, key, planted)


def make_layer(cfg: CaseConfig, ell: int) -> HostLayer:
    B, Q, W, D, H = cfg.B, cfg.Q, cfg.W, cfg.D, cfg.H
    mode = cfg.modes[ell]
    q = np.empty((B, Q, H, D), np.uint16)
    swa = np.empty((B, Q + W - 1, D), np.uint8) if Q + W - 1 > 0 else \
        np.zeros((B, 0, D), np.uint8)
    qi = wi = None
    if mode in (FULL, REINDEX):
        qi = np.empty((B, Q, cfg.HI, cfg.DI), np.uint8)
        wi = np.empty((B, Q, cfg.HI), np.float32)
    for b in range(B):
        if mode in (FULL, REINDEX):
            qi[b] = encode_e4m3(_rng(cfg.seed, S_QIDX, ell, b).standard_normal(
                (Q, cfg.HI, cfg.DI), dtype=np.float32))
            wi[b] = _rng(cfg.seed, S_W, ell, b).random((Q, cfg.HI), dtype=np.float32)
        x = _rng(cfg.seed, S_Q, ell, b).standard_normal((Q, H, D), dtype=np.float32)
        q[b] = encode_bf16(x / np.float32(math.sqrt(D)))
        if swa.shape[1] > 0:
            swa[b] = encode_e4m3(_rng(cfg.seed, S_SWA, ell, b).standard_normal(
                (Q + W - 1, D), dtype=np.float32))
    return HostLayer(mode, qi, wi, q, swa)


def make_case(cfg: CaseConfig) -> HostCase:
    return HostCase(cfg, make_pool(cfg), [make_layer(cfg, l) for l in range(cfg.L)])


def sequence_slice(case: HostCase, b: int) -> HostCase:
    """The same case restricted to one sequence (views, no copies)."""
    p = case.pool
    pool = HostPool(p.latent[b:b + 1], p.scale[b:b + 1], p.idx_key[b:b + 1],
                    p.planted[b:b + 1])
    layers = [HostLayer(L.mode,
                        None if L.q_idx is None else L.q_idx[b:b + 1],
                        None if L.w_idx is None else L.w_idx[b:b + 1],
                        L.q[b:b + 1], L.swa[b:b + 1]) for L in case.layers]
    return HostCase(case.cfg.scaled(B=1), pool, layers)
