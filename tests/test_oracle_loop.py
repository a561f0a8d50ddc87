"""Pins of the oracle loop: adaptive stop, cap, commit and resume."""
import time

import numpy as np

import synth_inputs
from oracle import loop, model, philox
from oracle.weights import Weights


def _copy_model(cfg, s):
    """Layer outputs vanish (Wo = 0, expert down = 0), LM head = s * embedding.

    Then the logits of position i are s * RMSNorm(E[x_i]) . E^T, whose argmax
    is x_i itself by a wide margin: every position locks at pass 1 and the
    argmax repeats at pass 2.
    """
    W = Weights(cfg)
    for l in range(cfg["L"]):
        W.set("wo", np.zeros_like(W.get("wo", l)), l)
        for e in range(cfg["E"]):
            W.set("wd", np.zeros_like(W.get("wd", l, e)), l, e)
    W.set("lm", s * W.get("embed"))
    return W


def test_copy_model_stops_at_pass_two_and_commits_initial_canvas():
    cfg = synth_inputs.workload("tiny")
    W = _copy_model(cfg, 8.0)
    prefix = synth_inputs.prefix_ids(cfg["V"], cfg["P0"], cfg["prefix_seed"])
    req, blocks = loop.generate(cfg, W, prefix, 1, cfg["gen_seed"], keep=True)
    b = blocks[0]
    x1 = loop.init_canvas(cfg, cfg["gen_seed"], 0, 0)
    assert b["steps"] == 2
    assert np.array_equal(b["ids"], x1)
    p1, p2 = b["passes"]
    assert p1["lock"].all() and p1["Hbar"] < 0.005 and not p1["stop"]
    assert p2["stop"] and np.array_equal(p2["a"], p1["a"])
    assert req.P == cfg["P0"] + cfg["C"]


def test_random_weights_never_lock_and_stop_at_cap():
    cfg = synth_inputs.workload("tiny")
    W = Weights(cfg)
    prefix = synth_inputs.prefix_ids(cfg["V"], cfg["P0"], cfg["prefix_seed"])
    t0 = time.time()
    req, blocks = loop.generate(cfg, W, prefix, 1, cfg["gen_seed"], keep=True)
    b = blocks[0]
    assert b["steps"] == 48 and len(b["passes"]) == 48
    for t, p in enumerate(b["passes"], start=1):
        assert not p["lock"].any()
        assert p["stop"] == (t == 48)
        want_x = philox.token_draw(cfg["gen_seed"], np.arange(256), t - 1, 0, 0, cfg["V"])
        assert np.array_equal(p["x"], want_x)
        assert abs(p["Hbar"] - np.log(cfg["V"])) < 0.1
    assert np.array_equal(b["ids"], b["passes"][-1]["a"])


def _block_causal_reference(cfg, W, prefix, blocks):
    """One forward over prefix + blocks with a block-causal mask."""
    ids = np.concatenate([prefix] + list(blocks))
    n, P0, C = len(ids), len(prefix), cfg["C"]
    blk = np.full(n, -1)
    for b in range(len(blocks)):
        blk[P0 + b * C: P0 + (b + 1) * C] = b
    allowed = np.zeros((n, n), bool)
    for i in range(n):
        for j in range(n):
            if blk[i] < 0:
                allowed[i, j] = j <= i and blk[j] < 0
            else:
                allowed[i, j] = blk[j] <= blk[i]
    h = W.get("embed")[ids]
    empty = model.empty_cache(cfg)
    kv = []
    for l in range(cfg["L"]):
        K0, V0 = empty[l]
        h, k, v, _ = model.layer(cfg, W, l, h, np.arange(n), K0, V0, allowed)
        kv.append((k, v))
    return kv


def test_incremental_commit_equals_block_causal_forward_and_prefix_is_immutable():
    cfg = synth_inputs.workload("tiny", L=2, d=64, Hq=4, Hkv=2, dh=16, E=4, k=2,
                                fe=32, V=256, C=8, P0=5)
    W = Weights(cfg)
    prefix = synth_inputs.prefix_ids(cfg["V"], cfg["P0"], 4)
    b0 = np.arange(8) * 3 % 256
    b1 = (np.arange(8) * 7 + 1) % 256
    req = loop.Request(cfg)
    loop.prefill(cfg, W, req, prefix)
    snap = [(K.copy(), V.copy()) for K, V in req.cache]
    loop.commit(cfg, W, req, b0)
    for (K, V), (K0, V0) in zip(req.cache, snap):
        assert np.array_equal(K[:, :5], K0) and np.array_equal(V[:, :5], V0)
    snap = [(K.copy(), V.copy()) for K, V in req.cache]
    loop.commit(cfg, W, req, b1)
    for (K, V), (K0, V0) in zip(req.cache, snap):
        assert np.array_equal(K[:, :13], K0) and np.array_equal(V[:, :13], V0)
    ref = _block_causal_reference(cfg, W, prefix, [b0, b1])
    for (K, V), (Kr, Vr) in zip(req.cache, ref):
        assert np.allclose(K, Kr, atol=1e-12) and np.allclose(V, Vr, atol=1e-12)


def test_resume_from_saved_state_reproduces_next_block():
    cfg = synth_inputs.workload("tiny", L=1, d=64, Hq=2, Hkv=1, dh=32, E=4, k=2,
                                fe=32, V=512, P0=16, max_steps=3)
    W = Weights(cfg)
    prefix = synth_inputs.prefix_ids(cfg["V"], cfg["P0"], 5)
    req, blocks = loop.generate(cfg, W, prefix, 2, seed=9)
    req2 = loop.Request(cfg)
    loop.prefill(cfg, W, req2, prefix)
    first = loop.run_block(cfg, W, req2, 0, 9)
    saved = req2.copy()
    again = loop.run_block(cfg, W, saved, 1, 9)
    assert np.array_equal(first["ids"], blocks[0]["ids"])
    assert np.array_equal(again["ids"], blocks[1]["ids"])
    assert saved.ids == req.ids
