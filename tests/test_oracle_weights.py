"""Pins of the synthetic weight generator (Philox + Box-Muller, N(0, 0.02^2)).

Checks against the normal law (Kolmogorov-Smirnov), the chi-square(2) law of
each Box-Muller pair's squared radius, pair independence, and the storage
formats' invariants.
"""
import numpy as np
from scipy import stats

import synth_inputs
from oracle import weights
from oracle.rounding import bf16_bits, bf16_from_bits, e4m3_bits, e4m3_from_bits, quantize_mxfp4


def test_normal_law_and_box_muller_pairs():
    z = weights.normal_draws(0, 5, np.arange(400000))
    assert stats.kstest(z, "norm").pvalue > 1e-3
    z0, z1 = z[0::2], z[1::2]
    r2 = z0 ** 2 + z1 ** 2
    assert stats.kstest(r2, stats.chi2(2).cdf).pvalue > 1e-3
    assert abs(np.corrcoef(z0, z1)[0, 1]) < 0.01
    assert abs(np.corrcoef(z0 ** 2, z1 ** 2)[0, 1]) < 0.01
    # different tensors / seeds give different streams
    z2 = weights.normal_draws(0, 6, np.arange(1000))
    z3 = weights.normal_draws(1, 5, np.arange(1000))
    assert np.mean(z2 == z[:1000]) < 0.01 and np.mean(z3 == z[:1000]) < 0.01


def test_tensor_ids_are_distinct():
    cfg = synth_inputs.workload("tiny")
    ids = [weights.tensor_id(cfg, "embed"), weights.tensor_id(cfg, "lm")]
    for l in range(cfg["L"]):
        for n in weights.LAYER_TENSORS:
            ids.append(weights.tensor_id(cfg, n, l))
        for e in range(cfg["E"]):
            for n in ("wg", "wu", "wd"):
                ids.append(weights.tensor_id(cfg, n, l, e))
        for n in ("sg", "su", "sd"):
            ids.append(weights.tensor_id(cfg, n, l))
    assert len(ids) == len(set(ids))


def test_storage_formats():
    cfg = synth_inputs.workload("tiny", wdtype="bf16")
    v, s = weights.stored_rows(cfg, "wq", 0, rows=np.arange(8))
    assert s is None
    raw = weights.raw_rows(cfg, "wq", 0, rows=np.arange(8))
    assert np.array_equal(bf16_from_bits(bf16_bits(v)), v)
    ulp = np.ldexp(1.0, np.frexp(np.abs(raw))[1] - 8)
    assert np.all(np.abs(v - raw) <= ulp / 2)
    assert abs(np.std(raw) - 0.02) < 0.002

    cfg8 = synth_inputs.workload("tiny", wdtype="fp8")
    v8, s8 = weights.stored_rows(cfg8, "wg", 1, 3, rows=np.arange(16))
    q = v8 / s8[:, None]
    assert np.array_equal(e4m3_from_bits(e4m3_bits(q)), q)
    assert np.all(np.abs(q) <= 448)
    assert np.all(np.abs(q).max(axis=1) >= 416)   # row max lands near the top
    assert np.array_equal(bf16_from_bits(bf16_bits(s8)), s8)
    # non-attention, non-expert tensors stay bf16 in fp8 models
    assert weights.storage(cfg8, "wr") == "bf16" and weights.storage(cfg8, "lm") == "bf16"

    cfg4 = synth_inputs.workload("tiny", wdtype="mxfp4")
    v4, e4 = weights.stored_rows(cfg4, "wd", 1, 2, rows=np.arange(8))
    raw4 = weights.raw_rows(cfg4, "wd", 1, 2, rows=np.arange(8))
    assert e4.shape == (8, cfg4["fe"] // 32)
    v_ref, e_ref = quantize_mxfp4(raw4)
    assert np.array_equal(v4, v_ref) and np.array_equal(e4, e_ref)
    assert weights.storage(cfg4, "wg") == "mxfp4" and weights.storage(cfg4, "wq") == "fp8"
    assert weights.storage(cfg4, "sg") == "bf16" and weights.storage(cfg4, "lm") == "bf16"
