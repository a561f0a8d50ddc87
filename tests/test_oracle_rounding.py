"""Pins of the oracle's rounding to bf16 / fp32 / E4M3FN.

torch's CPU casts are the library routine; exact rational arithmetic checks
the fp64 inputs that fp32 cannot hold (single rounding, no detour via fp32).
"""
from fractions import Fraction

import numpy as np
import torch

from oracle import rounding
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


def test_e2m1_nearest_by_brute_force():
    # E2M1 (OCP Microscaling Formats v1.0): codes 0..7 are 0, 0.5, 1, 1.5, 2,
    # 3, 4, 6; round to nearest, ties to the even code, saturate at +-6
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    rng = np.random.default_rng(5)
    mids = (grid[1:] + grid[:-1]) / 2
    xs = np.concatenate([rng.uniform(-9, 9, 4000), mids, -mids, grid, -grid, [6.5, 7.0, 1e9, -7.99]])
    for x in xs:
        a = abs(x)
        d = np.abs(grid - min(a, 6.0))
        best = np.flatnonzero(d == d.min())
        code = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
        want = np.copysign(grid[code], x)
        got = float(rounding.round_e2m1(np.array([x]))[0])
        assert got == want or (got == 0 and want == 0), (x, got, want)


def test_mx_block_scale_and_quantize():
    # the shared exponent puts the block's largest magnitude in [4, 8) before
    # rounding; examples: max 6 -> 2^0, max 8 -> 2^1, max 0.08 -> 2^-6
    assert list(rounding.mx_scale_exp(np.array([6.0, 7.9, 8.0, 0.08, 0.0]))) == [0, 0, 1, -6, 0]
    rng = np.random.default_rng(6)
    w = rng.normal(0, 0.02, (16, 128))
    w[3, :32] = 0.0                                   # an all-zero block
    v, e = rounding.quantize_mxfp4(w)
    assert e.shape == (16, 4) and e[3, 0] == 0 and np.all(v[3, :32] == 0)
    blk = w.reshape(16, 4, 32)
    amax = np.abs(blk).max(axis=2)
    nz = amax > 0
    r = amax[nz] / np.ldexp(1.0, e[nz])
    assert np.all((r >= 4) & (r < 8))
    q = np.ldexp(v.reshape(16, 4, 32), -e[:, :, None])
    grid = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}
    assert set(np.abs(q).ravel().tolist()) <= grid
    # error at most half the local step (the grid step is 0.5 below 2, 1
    # below 4, 2 above), except saturated elements, which become +-6
    x = np.ldexp(blk, -e[:, :, None])
    step = np.where(np.abs(x) < 2, 0.5, np.where(np.abs(x) < 4, 1.0, 2.0))
    sat = np.abs(x) > 6
    assert np.all(np.abs(q - x)[~sat] <= step[~sat] / 2 + 1e-12)
    assert np.all(np.abs(q[sat]) == 6)
