"""Write side of the stored formats: encoding new pool entries and window rows (fp64).

TEST INFRASTRUCTURE ONLY: part of the CPU oracle.  Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import this package; the product
path never does.

The pages say that a Full layer generates the KV and index data that later
layers reuse, that the global KV is stored in FP4 (E2M1) and the sliding-window
KV in FP8, and that values are restored at run time ("DeepSeek V4.1-Flash Cuts
KV Cache by 437x ...", paragraphs on the three operating modes, FP4
quantisation and sliding window attention; "DeepSeek V4.1 Flash Architecture
Breakdown", section "How are cache precision and storage arranged?").  They do
not give the encoding rule.  Readings used here:

* FP4 latent: the OCP Microscaling rule per block of 32 consecutive elements.
  The shared exponent is floor(log2(amax)) - 2 (2 is E2M1's largest
  exponent), clamped to the E8M0 range [-127, 127]; every element is divided
  by 2^shared and rounded to the nearest E2M1 value, ties to the even code,
  magnitudes above 6 saturating at 6.  An all-zero block gets scale code 127.
  A negative element keeps its sign, also when it rounds to zero.
* FP8 index keys and window rows: OCP E4M3, clamped to +-448, then rounded to
  the nearest E4M3 value with ties to even (the E4M3 NaN codes are never
  produced).
* A new pool entry is written at the entry number the caller gives (-1 or
  out of range: skipped).  A window of W rows is a ring: token position p
  lives in row p mod W; of T new tokens only the last W can be kept.

Every decision below is taken on exactly representable values (dividing a
float32 by a power of two is exact wherever it matters), so it does not
depend on the precision it is computed in.
"""
from __future__ import annotations

import numpy as np

# E2M1 magnitudes by code (codes 0..7; code | 8 is the negative)
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _round_to_grid(mag: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the nearest grid value for each magnitude (grid ascending),
    ties to the even index; magnitudes beyond the last value take the last."""
    mag = np.asarray(mag, dtype=np.float64)
    i = np.searchsorted(grid, mag, side="left")          # grid[i-1] < mag <= grid[i]
    i = np.clip(i, 1, len(grid) - 1)
    lo, hi = grid[i - 1], grid[i]
    d_lo, d_hi = mag - lo, hi - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (i % 2 == 0))
    out = np.where(pick_hi, i, i - 1)
    return np.where(mag >= grid[-1], len(grid) - 1, out)


def encode_mxfp4_block(x) -> tuple:
    """32 float32 values -> (16 packed E2M1 bytes, E8M0 scale code)."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    assert x.shape == (32,)
    amax = np.max(np.abs(x))
    if amax == 0.0:
        shared = 0
    else:
        _, e = np.frexp(amax)                  # amax = f * 2^e, f in [0.5, 1): floor(log2) = e - 1
        shared = int(np.clip(int(e) - 1 - 2, -127, 127))
    y = x / 2.0 ** shared
    idx = _round_to_grid(np.abs(y), E2M1_MAG)
    codes = idx.astype(np.uint8) | (np.signbit(y).astype(np.uint8) << 3)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    return packed, np.uint8(shared + 127)


def encode_mxfp4_row(x):
    """[D] float32 -> (packed [D/2] uint8, scales [D/32] uint8), block by block."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    packed = np.empty(D // 2, np.uint8)
    scales = np.empty(D // 32, np.uint8)
    for k in range(D // 32):
        packed[16 * k:16 * k + 16], scales[k] = encode_mxfp4_block(x[32 * k:32 * k + 32])
    return packed, scales


def _e4m3_grid() -> np.ndarray:
    """The 127 non-negative finite E4M3 values, ascending: subnormals m * 2^-9,
    then (1 + m/8) * 2^(e-7) for e = 1..15 (e = 15, m = 7 is NaN)."""
    vals = [m * 2.0 ** -9 for m in range(8)]
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals.append((1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


E4M3_GRID = _e4m3_grid()   # index = the code's low 7 bits


def encode_e4m3(x) -> np.ndarray:
    """float32 -> E4M3 bytes: clamp to +-448, nearest value, ties to the even code."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    c = np.clip(x, -448.0, 448.0)
    idx = _round_to_grid(np.abs(c), E4M3_GRID)
    return (idx.astype(np.uint8) | (np.signbit(c).astype(np.uint8) << 7)).astype(np.uint8)


def append_pool(latent, scale, idx_key, x_latent, x_key, slot):
    """New pool entries written in place (copies returned).

    latent [B][M][D/2], scale [B][M][D/32], idx_key [B][M][HI][DI] uint8;
    x_latent [B][T][D], x_key [B][T][HI][DI] float32; slot [B][T] int.
    Entry slot[b][t] of sequence b receives the encoded row t; slots outside
    [0, M) are skipped.  (Two new rows naming the same slot is a caller error.)
    """
    latent, scale, idx_key = latent.copy(), scale.copy(), idx_key.copy()
    B, M = latent.shape[:2]
    T = x_latent.shape[1]
    for b in range(B):
        for t in range(T):
            e = int(slot[b][t])
            if not 0 <= e < M:
                continue
            latent[b, e], scale[b, e] = encode_mxfp4_row(x_latent[b, t])
            idx_key[b, e] = encode_e4m3(x_key[b, t])
    return latent, scale, idx_key


def append_window(ring, x, pos0: int):
    """Window ring [B][W][D] uint8 after tokens pos0 .. pos0+T-1 (rows x [B][T][D]):
    token p lives in row p mod W; of the T new tokens the last W are kept."""
    ring = ring.copy()
    B, W = ring.shape[:2]
    T = x.shape[1]
    for t in range(max(0, T - W), T):
        ring[:, (pos0 + t) % W] = encode_e4m3(x[:, t])
    return ring
