"""Pins of the oracle's rounding to bf16 / fp32 / E4M3FN.

torch's CPU casts are the library routine; exact rational arithmetic checks
the fp64 inputs that fp32 cannot hold (single rounding, no detour via fp32).
"""
from fractions import Fraction

import numpy as np
import torch

from oracle.rounding import (round_bf16, round_e4m3, round_fp32, bf16_bits,
                             bf16_from_bits, e4m3_bits, e4m3_from_bits, E4M3_MAX)


def _fp32_samples(n, seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    return f[np.isfinite(f)]


def test_bf16_matches_torch_cast_on_fp32_inputs():
    f = _fp32_samples(1 << 20, 1)
    # add exact ties: bf16 value + half an ulp
    base = _fp32_samples(1 << 16, 2)
    b = torch.from_numpy(base).to(torch.bfloat16).to(torch.float32).numpy()
    ties = (b.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    f = np.concatenate([f, ties[np.isfinite(ties)]])
    ref = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_bf16(f.astype(np.float64))
    both_inf = np.isinf(ref) & np.isinf(got) & (np.sign(ref) == np.sign(got))
    assert np.all((got == ref) | both_inf)


def test_bf16_single_rounding_from_fp64():
    rng = np.random.default_rng(3)
    lo = torch.from_numpy(_fp32_samples(4000, 4)).to(torch.bfloat16).to(torch.float64).numpy()
    lo = lo[(np.abs(lo) > 1e-30) & (np.abs(lo) < 1e30)]
    for x0 in lo[:2000]:
        b1 = Fraction(float(x0))
        bits = int(bf16_bits(np.array([x0]))[0])
        b2 = Fraction(float(bf16_from_bits(np.array([bits + 1]))[0]))
        mid = (b1 + b2) / 2
        for sgn in (+1, -1):
            # just off the midpoint by far less than an fp32 ulp
            x = float(mid + sgn * abs(b2 - b1) * Fraction(1, 2**40))
            xf = Fraction(x)
            want = b2 if abs(xf - b2) < abs(xf - b1) else b1
            got = Fraction(float(round_bf16(np.array([x]))[0]))
            assert got == want


def test_fp32_rounding_matches_numpy_cast():
    x = np.random.default_rng(5).standard_normal(10000) * 1e3
    assert np.array_equal(round_fp32(x), x.astype(np.float32).astype(np.float64))


def test_e4m3_matches_torch_cast_within_range():
    all_codes = np.arange(256, dtype=np.uint8)
    vals = e4m3_from_bits(all_codes)
    finite = vals[np.isfinite(vals)]
    assert finite.max() == E4M3_MAX
    # every finite value, midpoints between neighbours, and random values
    s = np.sort(np.unique(finite))
    mids = (s[1:] + s[:-1]) / 2
    rnd = np.random.default_rng(6).uniform(-E4M3_MAX, E4M3_MAX, 200000)
    x = np.concatenate([s, mids, rnd, np.random.default_rng(7).uniform(-0.02, 0.02, 100000)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = round_e4m3(x.astype(np.float64))
    assert np.array_equal(got, ref)
    # codes round-trip
    assert np.array_equal(e4m3_from_bits(e4m3_bits(finite)), finite)
    assert np.array_equal(
        e4m3_bits(finite),
        torch.from_numpy(finite.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_e4m3_saturates():
    assert round_e4m3(np.array([449.0, 470.0, 1e6, -1e6])).tolist() == [448.0, 448.0, 448.0, -448.0]
