"""The row-wise layer check used by the full-width GPU tests
(tests/oracle_rows.py), exercised on the CPU with data of the oracle's own
forward: from a full forward's traced layer inputs and K/V, check_layer must
reproduce every checked row (canvas rows with no mask, prefill rows with the
causal mask) to rounding, and must reject a planted error in a key, a value
or a layer output; the threaded sampler must equal the plain one."""
import numpy as np
import pytest

import synth_inputs
from oracle import loop, model
from oracle import sampler as osamp
from oracle.weights import Weights
from tests.oracle_rows import check_layer, sample_threaded


def _setup():
    w = synth_inputs.workload("tiny", fs=128, P0=40)
    W = Weights(w)
    req = loop.Request(w)
    pre = synth_inputs.prefix_ids(w["V"], w["P0"], 4)
    tr_p = []
    pos_p = np.arange(w["P0"])
    _, kv_p, fin_p = model.forward(w, W, pre, pos_p, req.cache, causal=True, head=False, trace=tr_p)
    req.append(kv_p, pre)
    x = loop.init_canvas(w, 3, 0, 0)
    tr_c = []
    pos_c = w["P0"] + np.arange(w["C"])
    _, kv_c, fin_c = model.forward(w, W, x, pos_c, req.cache, causal=False, head=False, trace=tr_c)
    return w, req, tr_p, kv_p, fin_p, tr_c, kv_c, fin_c


def _items(w, l, req, tr_p, kv_p, fin_p, tr_c, kv_c, fin_c, rows, ppos):
    L, P0 = w["L"], w["P0"]
    K = np.concatenate([req.cache[l][0], kv_c[l][0]], axis=1)
    V = np.concatenate([req.cache[l][1], kv_c[l][1]], axis=1)
    cpos = P0 + rows
    return [
        dict(name="canvas", h_in=tr_c[l]["h_in"][rows],
             h_out=(tr_c[l + 1]["h_in"] if l + 1 < L else fin_c)[rows], pos=cpos, K=K, V=V, causal=False,
             ids=tr_c[l]["ids"][rows], k_got=K[:, cpos].transpose(1, 0, 2), v_got=V[:, cpos].transpose(1, 0, 2)),
        dict(name="prefill", h_in=tr_p[l]["h_in"][ppos],
             h_out=(tr_p[l + 1]["h_in"] if l + 1 < L else fin_p)[ppos], pos=ppos, K=K[:, :P0], V=V[:, :P0],
             causal=True, ids=tr_p[l]["ids"][ppos], k_got=K[:, ppos].transpose(1, 0, 2),
             v_got=V[:, ppos].transpose(1, 0, 2)),
    ]


def test_check_layer_reproduces_the_oracle_forward_and_rejects_errors():
    w, req, *rest = _setup()
    rows = np.array([0, 7, 100, 255])
    ppos = np.array([0, 1, 20, 39])
    for l in range(w["L"]):
        res = check_layer(w, l, _items(w, l, req, *rest, rows, ppos), 1e-12)
        assert all(r["adopted"] == 0 for r in res)
    for key in ("k_got", "v_got", "h_out"):
        for which in (0, 1):
            items = _items(w, 1, req, *rest, rows, ppos)
            items[which][key] = items[which][key].copy()
            items[which][key][1] *= 1.001
            with pytest.raises(AssertionError):
                check_layer(w, 1, items, 1e-6)


def test_sample_threaded_equals_plain_sampler():
    w = synth_inputs.workload("tiny")
    z = np.random.default_rng(5).standard_normal((w["C"], w["V"])) * 3
    a = osamp.sample(w, z, 7, 3, 1, 2)
    b = sample_threaded(w, z, 7, 3, 1, 2)
    for k in ("H", "a", "pmax", "margin", "lock", "x_next"):
        assert np.array_equal(a[k], b[k]), k
    assert abs(a["Hbar"] - b["Hbar"]) <= 1e-12 * a["Hbar"]


def test_activation_quantiser_model_rows():
    # the test-side model of the E4M3 activation quantiser: every value is an
    # E4M3 code times the row scale max|bf16 row| / 448 (fp32), the largest
    # magnitude maps to the code 448, and a zero row stays zero
    from oracle.rounding import round_bf16, round_e4m3
    from tests.oracle_rows import e4m3_rows
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 2816)) * np.array([1e-3, 1.0, 10.0, 1e4, 0.5])[:, None]
    x[4] = 0.0
    q = e4m3_rows(x)
    amax = np.abs(round_bf16(x)).max(axis=1)
    for i in range(4):
        s = np.float64(np.float32(amax[i]) / np.float32(448))
        codes = q[i] / s
        assert np.array_equal(round_e4m3(codes), codes)
        assert np.abs(codes).max() == 448.0
        assert 0.01 < np.linalg.norm(q[i] - x[i]) / np.linalg.norm(x[i]) < 0.05
    assert not q[4].any()
