"""Pins of the oracle sampler and stop rule.

Closed forms: uniform logits give H = ln V; a two-level distribution (one
logit a, V-1 logits 0) has p1 = e^a / (e^a + V - 1) and
H = -p1 ln p1 - (1 - p1) ln((1 - p1)/(V - 1)).  The stop truth table follows
the rule on the canvas page: mean entropy < 0.005 and the same argmax at every
position in two consecutive passes, cap 48.
"""
import math

import numpy as np

import synth_inputs
from oracle import sampler


def test_uniform_logits_give_ln_v():
    for V, want in [(4096, 8.317766166719343), (262144, 12.476649250079015)]:
        assert want == math.log(V) or abs(want - math.log(V)) < 1e-15
        z = np.full((2, V), 3.25, dtype=np.float32)
        H, a, pmax, margin = sampler.row_stats(z)
        assert np.allclose(H, math.log(V), rtol=0, atol=1e-12)
        assert np.all(a == 0)                      # all tied: lowest id
        assert np.allclose(pmax, 1.0 / V) and np.allclose(margin, 0.0)


def test_two_level_closed_form():
    V = 4096
    for av in (0.5, 5.0, 12.0, 30.0):
        z = np.zeros((1, V)); z[0, 777] = av
        H, a, pmax, margin = sampler.row_stats(z)
        p1 = math.exp(av) / (math.exp(av) + V - 1)
        q = (1 - p1) / (V - 1)
        want = -p1 * math.log(p1) - (1 - p1) * math.log(q)
        assert abs(H[0] - want) <= 1e-13 + 1e-12 * want
        assert a[0] == 777 and abs(pmax[0] - p1) < 1e-14 and abs(margin[0] - (p1 - q)) < 1e-14


def test_bounds_and_pmax_identity():
    z = np.random.default_rng(0).standard_normal((64, 4096)) * np.linspace(0.1, 20, 64)[:, None]
    H, a, pmax, _ = sampler.row_stats(z)
    assert np.all(H >= -1e-12) and np.all(H <= math.log(4096) + 1e-12)
    S = np.exp(z - z.max(axis=1, keepdims=True)).sum(axis=1)
    assert np.allclose(pmax, 1.0 / S, rtol=1e-14)
    assert np.array_equal(a, np.argmax(z, axis=1))


def test_argmax_ties_lowest_id():
    z = np.zeros((1, 100)); z[0, [17, 42, 99]] = 5.0
    assert sampler.row_stats(z)[1][0] == 17


def test_stop_truth_table():
    cfg = synth_inputs.workload("tiny")
    a = np.arange(256)
    b = a.copy(); b[100] += 1
    rule = lambda t, H, x, y: sampler.stop_rule(t, H, x, y, cfg["stop_H"], cfg["max_steps"])
    assert rule(1, 0.0, a, None) is False          # pass 1 never stops
    assert rule(2, 0.001, a, a) is True            # both conditions
    assert rule(2, 0.001, b, a) is False           # one position differs
    assert rule(5, 0.005, a, a) is False           # threshold is strict
    assert rule(5, 0.0049999, a, a) is True
    assert rule(7, 0.3, a, a) is False             # stable but uncertain
    assert rule(48, 7.0, b, a) is True             # cap
    assert rule(47, 7.0, b, a) is False


def test_lock_and_renoise():
    cfg = synth_inputs.workload("tiny")
    V = cfg["V"]
    z = np.zeros((256, V))
    z[:128, 5] = 30.0            # confident rows -> lock to id 5
    z[128:, 5] = 1.0             # flat rows -> re-noise
    out = sampler.sample(cfg, z, seed=3, step=4, block=1, req=0)
    assert np.all(out["lock"][:128]) and not np.any(out["lock"][128:])
    assert np.all(out["x_next"][:128] == 5)
    from oracle import philox
    noise = philox.token_draw(3, np.arange(256), 4, 1, 0, V)
    assert np.array_equal(out["x_next"][128:], noise[128:])
    # lock threshold is strict: p_max exactly 0.9 does not lock
    zz = np.zeros((1, 10)); zz[0, 0] = math.log(0.9 * 9 / 0.1)
    H, a, pmax, _ = sampler.row_stats(zz)
    assert abs(pmax[0] - 0.9) < 1e-15


def test_entropy_bound_lock_rule():
    # two-level rows whose closed-form entropy lies just above, at about, and
    # just below the bound: kept exactly where H <= bound; the rest re-noised
    V, bound = 4096, 0.1

    def H2(a):
        p1 = math.exp(a) / (math.exp(a) + V - 1)
        return -p1 * math.log(p1) - (1 - p1) * math.log((1 - p1) / (V - 1))
    lo, hi = 0.0, 60.0                             # H2 falls monotonically in a
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        lo, hi = (mid, hi) if H2(mid) > bound else (lo, mid)
    gaps = [hi - 0.05, hi - 0.001, hi + 0.001, hi + 0.05, 1.0, 40.0]
    z = np.zeros((len(gaps), V))
    z[np.arange(len(gaps)), 777] = gaps
    want = np.array([H2(a) <= bound for a in gaps])
    assert list(want) == [False, False, True, True, False, True]
    w = synth_inputs.workload("tiny", lock_rule="entropy", entropy_bound=bound)
    out = sampler.sample(w, z, seed=3, step=2, block=1, req=5)
    assert np.array_equal(out["lock"], want)
    assert np.allclose(out["H"], [H2(a) for a in gaps], rtol=1e-10, atol=1e-14)
    noise = sampler.philox.token_draw(3, np.arange(len(gaps)), 2, 1, 5, V)
    assert np.array_equal(out["x_next"], np.where(want, 777, noise))
    # the default rule on the same rows: max probability against 0.9
    ref = sampler.sample(synth_inputs.workload("tiny"), z, seed=3, step=2, block=1, req=5)
    assert np.array_equal(ref["lock"], ref["pmax"] > 0.9) and not np.array_equal(ref["lock"], want)
