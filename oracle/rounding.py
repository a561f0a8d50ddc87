"""Rounding of fp64 values to the storage formats, round-to-nearest-even.

Weights are drawn in fp64 and rounded once, directly, to their storage format
(no double rounding through fp32).  The pages name BF16 and FP8 checkpoints
([P2] hardware requirements list BF16, FP8 and NVFP4 variants); the fp8 format
here is OCP E4M3FN (3 mantissa bits, bias 7, largest finite 448, no infinity),
with saturation at +-448.

Pins (tests/test_oracle_rounding.py): torch's CPU casts fp32 -> bfloat16 and
fp32 -> float8_e4m3fn on every value where they apply, and exact rational
arithmetic (``fractions``) for fp64 inputs that fp32 cannot hold; for E2M1,
brute force over the 15 representable values (nearest, ties to the even
code) and the format's own examples of the MX block scale.
"""
from __future__ import annotations

import numpy as np


def _round_sig(x, sig_bits: int, min_quantum_exp: int):
    """Round to ``sig_bits`` significant bits, RNE, quantum at least 2^min_q."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # |x| in [2^(e-1), 2^e)
    q = np.maximum(e - sig_bits, min_quantum_exp)
    return np.ldexp(np.rint(np.ldexp(x, -q)), q)


def round_bf16(x):
    """fp64 -> nearest bfloat16 value (8 significant bits), returned as fp64."""
    out = _round_sig(x, 8, -133)
    big = np.ldexp(1.0, 128)
    return np.where(np.abs(out) >= big, np.copysign(np.inf, out), out)


def round_fp32(x):
    """fp64 -> nearest fp32 value, returned as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


E4M3_MAX = 448.0


def round_e4m3(x):
    """fp64 -> nearest E4M3FN value (4 significant bits), saturating."""
    out = _round_sig(x, 4, -9)
    return np.clip(out, -E4M3_MAX, E4M3_MAX)


E2M1_MAX = 6.0


def round_e2m1(x):
    """fp64 -> nearest E2M1 value (2 significant bits, smallest step 0.5:
    0, 0.5, 1, 1.5, 2, 3, 4, 6), ties to even, saturating at +-6."""
    out = _round_sig(x, 2, -1)
    return np.clip(out, -E2M1_MAX, E2M1_MAX)


def mx_scale_exp(amax):
    """Shared exponent of an MXFP4 block with largest magnitude amax (OCP
    Microscaling Formats v1.0): floor(log2 amax) minus 2, the exponent of the
    largest E2M1 power of two, clamped to [-126, 127] (E8M0 reaches -127;
    stopping at -126 keeps the scale a normal fp32 number); 0 for an all-zero
    block."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))     # amax in [2^(e-1), 2^e)
    return np.where(amax > 0, np.clip(e - 1 - 2, -126, 127), 0).astype(np.int64)


def quantize_mxfp4(w):
    """Rows w[n][K] (K a multiple of 32) -> (dequantised values, block
    exponents [n][K/32]): each 32-element block shares the scale 2^e and its
    elements are round_e2m1(w / 2^e)."""
    w = np.asarray(w, dtype=np.float64)
    n, K = w.shape
    blk = w.reshape(n, K // 32, 32)
    e = mx_scale_exp(np.max(np.abs(blk), axis=2))
    q = round_e2m1(np.ldexp(blk, -e[:, :, None]))
    return np.ldexp(q, e[:, :, None]).reshape(n, K), e


def bf16_bits(v):
    """uint16 bit patterns of values that are exactly bfloat16."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_from_bits(b):
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_from_bits(b):
    """Decode E4M3FN bytes (0x7F / 0xFF are NaN)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    ex = (b >> 3) & 0xF
    m = b & 0x7
    val = np.where(ex == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp((8 + m).astype(np.float64), ex - 10))
    val = np.where((b & 0x7F) == 0x7F, np.nan, val)
    return s * val


def e4m3_bits(v):
    """Encode values that are exactly E4M3FN into bytes."""
    v = np.asarray(v, dtype=np.float64)
    s = (np.signbit(v)).astype(np.int64) << 7
    a = np.abs(v)
    _, e = np.frexp(np.where(a == 0, 1.0, a))
    ex = e - 1 + 7                         # biased exponent for normals
    sub = a < np.ldexp(1.0, -6)
    m_norm = np.ldexp(a, -(e - 1) + 3) - 8  # 3 fraction bits
    m_sub = np.ldexp(a, 9)
    code = np.where(sub, m_sub, (ex << 3) + m_norm)
    return (s + code.astype(np.int64)).astype(np.uint8)
