"""Decoding of the stored number formats, written out from their definitions (fp64).

TEST INFRASTRUCTURE ONLY: part of the CPU oracle.  Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import this package; the product
path never does.

The pages fix the formats only by name: the global KV is kept in FP4 with the
E2M1 scheme and the sliding-window KV stays FP8 ("DeepSeek V4.1-Flash Cuts KV
Cache by 437x ...", paragraph on FP4 quantisation; "DeepSeek V4.1 Flash
Architecture Breakdown", section "How are cache precision and storage
arranged?").  The bit layouts below are the OCP 8-bit floating point (E4M3)
and OCP Microscaling (E2M1 element, E8M0 block scale) definitions.  Readings
where the pages are silent: FP8 is the OCP E4M3 variant (bias 7, no infinity,
S.1111.111 is NaN); the FP4 block scale is one E8M0 per 32 consecutive
elements; element 2i sits in the low nibble of byte i.
"""
from __future__ import annotations

import numpy as np


def e4m3_value(b) -> np.ndarray:
    """OCP E4M3 byte -> value: sign, 4 exponent bits (bias 7), 3 mantissa bits.

    Exponent field 0 is subnormal: m * 2^-9.  Otherwise (1 + m/8) * 2^(e-7).
    Bytes 0x7F and 0xFF are NaN; there is no infinity.
    """
    b = np.asarray(b).astype(np.int64)
    s = b >> 7
    e = (b >> 3) & 0xF
    m = b & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where(s == 1, -mag, mag)
    return np.where((b & 0x7F) == 0x7F, np.nan, val)


def e2m1_value(c) -> np.ndarray:
    """OCP E2M1 4-bit code -> value: sign, 2 exponent bits (bias 1), 1 mantissa bit.

    Exponent field 0 is subnormal: m * 0.5.  Otherwise (1 + m/2) * 2^(e-1).
    All 16 codes are finite: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}.
    """
    c = np.asarray(c).astype(np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 0x3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag)


def e8m0_value(x) -> np.ndarray:
    """OCP E8M0 scale byte -> 2^(x-127); 0xFF is NaN."""
    x = np.asarray(x).astype(np.int64)
    return np.where(x == 0xFF, np.nan, np.exp2(x - 127.0))


def bf16_value(u) -> np.ndarray:
    """bf16 bit pattern (uint16) -> value: the top half of an IEEE binary32."""
    u = np.asarray(u).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def unpack_e2m1_codes(packed) -> np.ndarray:
    """uint8 [..., D/2] -> codes [..., D]; element 2i = low nibble of byte i."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequant_latent(packed, scale) -> np.ndarray:
    """FP4 latent rows -> fp64 values.

    c[i] = E2M1(code_i) * E8M0(scale[i // 32]); exact in fp64 for every valid
    code pair (the product has at most two significant bits).
    """
    v = e2m1_value(unpack_e2m1_codes(packed))
    s = e8m0_value(scale)
    return v * np.repeat(s, 32, axis=-1)
