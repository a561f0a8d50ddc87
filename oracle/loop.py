"""Prefill, denoise loop and block commit, in fp64.

Follows the pages' four steps ([P3] ① to ④; [P4] "architecture"):
① the prompt is encoded causally into a reusable KV cache;
② a 256-token canvas is filled with uniform random ids;
③ passes denoise the canvas until the adaptive stop (or the cap of 48);
④ the converged block is committed to the KV cache and the next canvas is
   conditioned on it; committed blocks are never rewritten.
Readings: the committed ids are the argmax of the stopping pass (also when the
cap fires); the committed block's K/V are those of a canvas-mode pass over the
committed ids at positions P..P+255 (bidirectional inside the block, over the
whole cache), appended at [P, P+256); P grows by 256.  Requests are
independent (own cache, own Philox stream keyed by request index).

Pins (tests/test_oracle_loop.py): the copy model (layer outputs zeroed, LM
head = s * embedding) stops at exactly pass 2 and commits its initial canvas;
random weights never lock and stop at exactly pass 48 with a pure-Philox
canvas; incremental commits equal one block-causal forward; the committed
prefix is never modified; resuming from a saved state reproduces the rest.
"""
from __future__ import annotations

import numpy as np

from . import model, philox, sampler


class Request:
    """KV cache and committed ids of one request."""

    def __init__(self, cfg, req=0):
        self.cfg = cfg
        self.req = req
        self.cache = model.empty_cache(cfg)
        self.ids = []

    @property
    def P(self):
        return self.cache[0][0].shape[1]

    def append(self, new_kv, ids):
        self.cache = [(np.concatenate([K, k], axis=1), np.concatenate([V, v], axis=1))
                      for (K, V), (k, v) in zip(self.cache, new_kv)]
        self.ids.extend(int(i) for i in ids)

    def copy(self):
        r = Request(self.cfg, self.req)
        r.cache = [(K.copy(), V.copy()) for K, V in self.cache]
        r.ids = list(self.ids)
        return r


def prefill(cfg, W, req, ids, forced_routing=None):
    """Causal forward over prompt ids at positions P.. ; appends their K/V."""
    pos = req.P + np.arange(len(ids))
    _, new_kv, _ = model.forward(cfg, W, ids, pos, req.cache, causal=True, head=False,
                                 forced_routing=forced_routing)
    req.append(new_kv, ids)


def init_canvas(cfg, seed, block, req_idx):
    return philox.token_draw(seed, np.arange(cfg["C"]), 0, block, req_idx, cfg["V"])


def denoise_pass(cfg, W, req, x, t, block, seed, trace=None, forced_routing=None):
    """Pass t over canvas x: logits, sampler outputs and this pass's K/V."""
    pos = req.P + np.arange(cfg["C"])
    z, new_kv, _ = model.forward(cfg, W, x, pos, req.cache, causal=False, trace=trace,
                                 forced_routing=forced_routing)
    out = sampler.sample(cfg, z, seed, t, block, req.req)
    out["z"] = z
    out["kv"] = new_kv
    return out


def commit(cfg, W, req, ids, forced_routing=None):
    """Append the K/V of a canvas-mode pass over the committed ids."""
    pos = req.P + np.arange(len(ids))
    _, new_kv, _ = model.forward(cfg, W, ids, pos, req.cache, causal=False, head=False,
                                 forced_routing=forced_routing)
    req.append(new_kv, ids)


def run_block(cfg, W, req, block, seed, keep=False):
    """Denoise one block to the adaptive stop and commit it.

    Returns dict(ids, steps, passes) where passes (if keep) lists per-pass
    sampler outputs with the canvas fed to that pass.
    """
    x = init_canvas(cfg, seed, block, req.req)
    a_prev = None
    passes = []
    for t in range(1, cfg["max_steps"] + 1):
        out = denoise_pass(cfg, W, req, x, t, block, seed)
        out["x"] = x
        stop = sampler.stop_rule(t, out["Hbar"], out["a"], a_prev, cfg["stop_H"], cfg["max_steps"])
        out["stop"] = stop
        if keep:
            passes.append(out)
        if stop:
            committed = out["a"].astype(np.int64)
            commit(cfg, W, req, committed)
            return dict(ids=committed, steps=t, passes=passes)
        a_prev = out["a"]
        x = out["x_next"]
    raise AssertionError("unreachable: the cap always stops")


def generate(cfg, W, prefix, n_blocks, seed, req_idx=0, keep=False):
    req = Request(cfg, req_idx)
    prefill(cfg, W, req, prefix)
    blocks = [run_block(cfg, W, req, b, seed, keep) for b in range(n_blocks)]
    return req, blocks
