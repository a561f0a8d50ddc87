"""Pins of the oracle forward pieces: attention, RMSNorm, RoPE, MoE."""
import itertools

import numpy as np

import synth_inputs
from oracle import model
from oracle.weights import Weights


def _loops_attention(q, K, V, causal_from=None):
    """Explicit scalar loops: the textbook definition, one query at a time."""
    n, Hq, dh = q.shape
    Hkv, m, _ = K.shape
    out = np.zeros((n, Hq, dh))
    for i in range(n):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            keys = range(m) if causal_from is None else range(causal_from + i + 1)
            s = {j: sum(q[i, h, c] * K[g, j, c] for c in range(dh)) / np.sqrt(dh) for j in keys}
            mx = max(s.values())
            w = {j: np.exp(v - mx) for j, v in s.items()}
            tot = sum(w.values())
            for c in range(dh):
                out[i, h, c] = sum(w[j] * V[g, j, c] for j in keys) / tot
    return out


def test_attention_canvas_and_causal_match_loops():
    rng = np.random.default_rng(0)
    P, C, dh, Hq, Hkv = 3, 4, 4, 4, 2
    q = rng.standard_normal((C, Hq, dh))
    K = rng.standard_normal((Hkv, P + C, dh))
    V = rng.standard_normal((Hkv, P + C, dh))
    got = model.attention(q, K, V)
    assert np.allclose(got, _loops_attention(q, K, V), atol=1e-13)
    allowed = np.concatenate([np.ones((C, P), bool), np.tril(np.ones((C, C), bool))], axis=1)
    got_c = model.attention(q, K, V, allowed)
    assert np.allclose(got_c, _loops_attention(q, K, V, causal_from=P), atol=1e-13)
    # GQA: query heads 0,1 read kv head 0; changing kv head 1 leaves them alone
    K2 = K.copy(); K2[1] += rng.standard_normal(K2[1].shape)
    assert np.array_equal(model.attention(q, K2, V)[:, :2], got[:, :2])
    assert not np.allclose(model.attention(q, K2, V)[:, 2:], got[:, 2:])


def test_rmsnorm_unit_rms_and_scale_invariance():
    x = np.random.default_rng(1).standard_normal((5, 64)) * 3
    y = model.rmsnorm(x, 0.0)
    assert np.allclose(np.sqrt(np.mean(y ** 2, axis=1)), 1.0, atol=1e-14)
    assert np.allclose(model.rmsnorm(7.5 * x, 0.0), y, atol=1e-14)
    assert np.allclose(model.rmsnorm(x, 1e-6), y, atol=1e-6)


def test_rope_norm_and_relative_position():
    rng = np.random.default_rng(2)
    dh = 16
    q = rng.standard_normal((1, 1, dh))
    k = rng.standard_normal((1, 1, dh))
    for p in (0, 5, 1000):
        assert np.isclose(np.linalg.norm(model.rope(q, [p], 1e4)), np.linalg.norm(q), rtol=1e-14)
    assert np.array_equal(model.rope(q, [0], 1e4), q)
    dots = []
    for m, n in [(10, 7), (110, 107), (3, 0)]:
        dots.append(np.sum(model.rope(q, [m], 1e4) * model.rope(k, [n], 1e4)))
    assert np.allclose(dots, dots[0], atol=1e-12)
    far = np.sum(model.rope(q, [20], 1e4) * model.rope(k, [7], 1e4))
    assert not np.isclose(far, dots[0])
    # first pair rotates by exactly the position (frequency 1), in the plane
    # spanned by dims 0 and dh/2
    e = np.zeros((1, 1, dh)); e[0, 0, 0] = 1.0
    r = model.rope(e, [0.3], 1e4)[0, 0]
    assert np.isclose(r[0], np.cos(0.3)) and np.isclose(r[dh // 2], np.sin(0.3))


def _small_cfg(**kw):
    cfg = synth_inputs.workload("tiny", L=1, d=32, Hq=2, Hkv=1, dh=16, E=4, k=2,
                                fe=24, fs=0, V=64)
    cfg.update(kw)
    return cfg


def test_topk_route_ties_and_gates():
    r = np.array([[1.0, 3.0, 3.0, 0.5], [2.0, 2.0, 2.0, 2.0], [-1, 4, 0, 4]])
    ids, g = model.topk_route(r, 2)
    assert ids.tolist() == [[1, 2], [0, 1], [1, 3]]
    assert np.allclose(g.sum(axis=1), 1.0, atol=1e-15)
    rng = np.random.default_rng(3)
    r = rng.standard_normal((50, 16))
    ids, g = model.topk_route(r, 5)
    ref = np.argsort(-r, axis=1, kind="stable")[:, :5]
    assert np.array_equal(ids, ref)
    assert np.allclose(g.sum(axis=1), 1.0, atol=1e-14)
    assert np.all(np.diff(g, axis=1) <= 0)


def test_moe_special_cases():
    rng = np.random.default_rng(4)
    u = rng.standard_normal((6, 32))
    # E = k: every expert, gates = full softmax of router logits
    cfg = _small_cfg(E=3, k=3)
    W = Weights(cfg)
    out, r, _, _ = model.moe(cfg, W, 0, u)
    p = np.exp(r - r.max(axis=1, keepdims=True)); p /= p.sum(axis=1, keepdims=True)
    ref = sum(p[:, [e]] * model.swiglu(u, W.get("wg", 0, e), W.get("wu", 0, e), W.get("wd", 0, e))
              for e in range(3))
    assert np.allclose(out, ref, atol=1e-15)
    # E = k = 1: a plain SwiGLU FFN, written out element by element
    cfg1 = _small_cfg(E=1, k=1)
    W1 = Weights(cfg1)
    out1, _, _, g1 = model.moe(cfg1, W1, 0, u)
    assert np.all(g1 == 1.0)
    Wg, Wu, Wd = W1.get("wg", 0, 0), W1.get("wu", 0, 0), W1.get("wd", 0, 0)
    for t in range(2):
        hid = [(lambda a: a / (1 + np.exp(-a)))(Wg[j] @ u[t]) * (Wu[j] @ u[t]) for j in range(Wg.shape[0])]
        ref_t = [sum(Wd[o, j] * hid[j] for j in range(len(hid))) for o in range(Wd.shape[0])]
        assert np.allclose(out1[t], ref_t, atol=1e-15)
    # shared FFN is added with weight 1
    cfgs = _small_cfg(fs=8)
    Ws = Weights(cfgs)
    o_s, _, _, _ = model.moe(cfgs, Ws, 0, u)
    o_n, _, _, _ = model.moe(_small_cfg(), Weights(_small_cfg()), 0, u)
    assert np.allclose(o_s - o_n, model.swiglu(u, Ws.get("sg", 0), Ws.get("su", 0), Ws.get("sd", 0)), atol=1e-15)


def test_moe_token_permutation_equivariance():
    cfg = _small_cfg()
    W = Weights(cfg)
    u = np.random.default_rng(5).standard_normal((10, 32))
    perm = np.random.default_rng(6).permutation(10)
    a, _, ia, _ = model.moe(cfg, W, 0, u)
    b, _, ib, _ = model.moe(cfg, W, 0, u[perm])
    assert np.allclose(a[perm], b, atol=1e-15)
    assert np.array_equal(ia[perm], ib)


def test_canvas_forward_is_permutation_equivariant_without_rope():
    # no mask and no positions: the canvas is a set; causal prefill is not
    cfg = _small_cfg(theta=0.0)
    W = Weights(cfg)
    ids = np.array([3, 9, 1, 40, 7])
    perm = np.array([4, 2, 0, 1, 3])
    cache = model.empty_cache(cfg)
    za, _, _ = model.forward(cfg, W, ids, np.arange(5), cache)
    zb, _, _ = model.forward(cfg, W, ids[perm], np.arange(5), cache)
    assert np.allclose(za[perm], zb, atol=1e-12)
    ca, _, _ = model.forward(cfg, W, ids, np.arange(5), cache, causal=True)
    cb, _, _ = model.forward(cfg, W, ids[perm], np.arange(5), cache, causal=True)
    assert not np.allclose(ca[perm], cb)


def test_forced_routing_with_own_choice_is_identity():
    cfg = _small_cfg(fs=8)
    W = Weights(cfg)
    u = np.random.default_rng(8).standard_normal((9, 32))
    a, r, ids, g = model.moe(cfg, W, 0, u)
    b, r2, ids2, g2 = model.moe(cfg, W, 0, u, forced_ids=ids[:, ::-1])
    assert np.array_equal(ids2, ids[:, ::-1]) and np.allclose(a, b, atol=1e-15)
    c, _, _, _ = model.moe(cfg, W, 0, u, forced_ids=(ids + 1) % cfg["E"])
    assert not np.allclose(a, c)
