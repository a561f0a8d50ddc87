"""The oracle's C weight generator (oracle/csrc/wgen.c) against its numpy
definition (oracle/weights.py, itself pinned by test_oracle_weights.py and
test_oracle_philox.py): stored values, fp8 row scales and MXFP4 block
exponents bit-identical on more than 10^6 elements of every storage format,
including row subsets, rows at the end of large tensors (counters above
2^32 / 4) and ragged row lengths."""
import numpy as np
import pytest

import synth_inputs
from oracle import weights
from oracle.weights import _c_generator, raw_rows, stored_rows_c

pytestmark = pytest.mark.skipif(_c_generator() is None, reason="oracle/libwgen.so not built")


def _numpy_stored(cfg, name, layer, expert, rows):
    # the numpy path of stored_rows, whatever the C generator's availability
    from oracle.rounding import round_bf16, round_e4m3, round_fp32, quantize_mxfp4, E4M3_MAX
    w = raw_rows(cfg, name, layer, expert, rows)
    fmt = weights.storage(cfg, name)
    if fmt == "f32":
        return round_fp32(w), None
    if fmt == "bf16":
        return round_bf16(w), None
    if fmt == "mxfp4":
        return quantize_mxfp4(w)
    s = round_bf16(np.max(np.abs(w), axis=1) / E4M3_MAX)
    return round_e4m3(w / s[:, None]) * s[:, None], s


@pytest.mark.parametrize("wd,name,layer,expert,rows", [
    ("bf16", "wg", 3, 17, np.arange(400)),
    ("bf16", "lm", None, None, np.array([0, 1, 5, 262143, 131071, 77777])),   # n up to 7.4e8
    ("bf16", "embed", None, None, np.arange(262144 - 300, 262144)),
    ("fp8", "wq", 29, None, np.arange(0, 2048, 5)),
    ("fp8", "wd", 7, 127, np.arange(300)),
    ("mxfp4", "wu", 11, 64, np.arange(350)),
    ("mxfp4", "wd", 0, 3, np.arange(2816 - 300, 2816)),
    ("f32", "wg", 1, 2, np.arange(512)),
])
def test_c_generator_equals_numpy_definition(wd, name, layer, expert, rows):
    cfg = synth_inputs.workload("step_bf16", wdtype=wd, weight_seed=0x0123456789ABCDEF)
    got, gaux = stored_rows_c(cfg, name, layer, expert, rows)
    ref, raux = _numpy_stored(cfg, name, layer, expert, rows)
    assert got.shape == ref.shape
    if wd == "f32":
        # fp32 rounding of fp64 draws whose last bits may differ between two
        # libm implementations: a flip needs a draw within an ulp of a
        # rounding boundary (probability about 2^-29 per value)
        assert np.mean(got != ref) < 1e-5
    else:
        assert np.array_equal(got, ref)
    if raux is not None:
        assert np.array_equal(gaux, raux)


def test_c_generator_raw_values_and_total_count():
    cfg = synth_inputs.workload("step_bf16", weight_seed=3)
    n = 0
    for e in range(4):
        got, _ = stored_rows_c(cfg, "wg", 2, e, np.arange(704), fmt="raw")
        ref = raw_rows(cfg, "wg", 2, e, np.arange(704))
        assert np.allclose(got, ref, rtol=1e-13, atol=0)
        n += got.size
    assert n > 10 ** 6
