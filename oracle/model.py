"""Forward pass of the MoE decoder over a canvas, in fp64.

What the pages fix:
* The canvas forward is bidirectional: every canvas token attends every other
  canvas token ([P4] "how text diffusion works", last paragraphs; [P5]
  developer value, "bi-directional attention").
* The prompt is encoded left to right with causal attention into a reusable
  KV cache, and each canvas attends that committed history ([P3] step ①;
  [P4] "architecture", the two attention modes and block autoregressive
  diffusion).
* The backbone is a mixture-of-experts decoder ([P1] §2.2 table; [P4] "what it
  is"; [P5] intro) with a diffusion head on top ([P5] intro).
What the pages leave open takes the plainest pre-norm decoder reading:
RMSNorm with unit gain and eps 1e-6 before attention, before the MoE and before
the head; rotate-half rotary embedding with base 10^4 at absolute positions
(keys cached after rotation); attention scale 1/sqrt(dh), no soft-cap, no
window; grouped-query attention with query head h reading KV head
h // (Hq/Hkv); router logits u.Wr^T, top-k with ties to the lower expert id,
gates = softmax over the k selected logits; SwiGLU experts
Wd (silu(Wg u) * (Wu u)); an optional shared SwiGLU FFN added with weight 1;
an untied LM head.

Pins (tests/test_oracle_model.py): attention against explicit scalar loops
(canvas and causal, GQA); RMSNorm output RMS = 1 and scale invariance; RoPE
norm preservation and relative-position dependence; MoE special cases (E=k is
a full-softmax mixture, E=k=1 is one SwiGLU FFN), gates summing to 1, top-k
against a full sort, token-permutation equivariance; block-causal equivalence
of incremental commits.
"""
from __future__ import annotations

import numpy as np


def rmsnorm(x, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope_angles(positions, dh, theta):
    """angle[p][i] = position_p * theta^(-2i/dh), i < dh/2."""
    i = np.arange(dh // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / dh)
    return np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]


def rope(x, positions, theta):
    """Rotate-half rotary embedding of x[n][H][dh] at the given positions."""
    if theta == 0:
        return np.array(x, dtype=np.float64)
    dh = x.shape[-1]
    ang = rope_angles(positions, dh, theta)[:, None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., : dh // 2], x[..., dh // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention(q, K, V, allowed=None):
    """o[n][Hq][dh] = softmax(q K^T / sqrt(dh)) V per head, GQA.

    q: [n][Hq][dh]; K, V: [Hkv][m][dh]; allowed: optional bool [n][m] mask
    (True = may attend).  No mask means every query sees every key.
    """
    n, Hq, dh = q.shape
    Hkv = K.shape[0]
    grp = Hq // Hkv
    out = np.empty((n, Hq, dh))
    for h in range(Hq):
        g = h // grp
        s = q[:, h, :] @ K[g].T / np.sqrt(dh)
        if allowed is not None:
            s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ V[g]
    return out


def silu(a):
    return a / (1.0 + np.exp(-a))


def swiglu(u, Wg, Wu, Wd):
    return (silu(u @ Wg.T) * (u @ Wu.T)) @ Wd.T


def topk_route(r, k):
    """Top-k expert ids per row (ties -> lower id) and softmax gates over them."""
    n, E = r.shape
    ids = np.empty((n, k), dtype=np.int64)
    for t in range(n):
        order = sorted(range(E), key=lambda e: (-r[t, e], e))
        ids[t] = order[:k]
    sel = np.take_along_axis(r, ids, axis=1)
    g = np.exp(sel - sel.max(axis=1, keepdims=True))
    g /= g.sum(axis=1, keepdims=True)
    return ids, g


def moe(cfg, W, layer, u, forced_ids=None):
    """MoE FFN output for normed rows u[n][d]: routed experts + shared FFN.

    forced_ids (optional [n][k]) replaces the top-k choice; the gates are still
    the softmax of this oracle's router logits over those experts.  Used only
    to follow another implementation's routing where a top-k decision was a
    near-tie (lockstep comparison).
    """
    r = u @ W.get("wr", layer).T
    if forced_ids is None:
        ids, gates = topk_route(r, cfg["k"])
    else:
        ids = np.asarray(forced_ids, dtype=np.int64)
        sel = np.take_along_axis(r, ids, axis=1)
        gates = np.exp(sel - sel.max(axis=1, keepdims=True))
        gates /= gates.sum(axis=1, keepdims=True)
    out = np.zeros_like(u)
    for e in range(cfg["E"]):
        rows, slot = np.nonzero(ids == e)
        if rows.size == 0:
            continue
        y = swiglu(u[rows], W.get("wg", layer, e), W.get("wu", layer, e), W.get("wd", layer, e))
        out[rows] += gates[rows, slot][:, None] * y
    if cfg["fs"] > 0:
        out += swiglu(u, W.get("sg", layer), W.get("su", layer), W.get("sd", layer))
    return out, r, ids, gates


def layer(cfg, W, l, h, positions, K_prev, V_prev, allowed=None, forced_ids=None):
    """One decoder layer over rows h[n][d].

    K_prev, V_prev: [Hkv][m][dh] cached keys/values this layer attends in
    front of the new rows.  Returns (h_out, k_new, v_new, trace); k_new and
    v_new are [Hkv][n][dh] (keys after rotation).
    """
    n = h.shape[0]
    Hq, Hkv, dh = cfg["Hq"], cfg["Hkv"], cfg["dh"]
    u = rmsnorm(h, cfg["eps"])
    q = (u @ W.get("wq", l).T).reshape(n, Hq, dh)
    k = (u @ W.get("wk", l).T).reshape(n, Hkv, dh)
    v = (u @ W.get("wv", l).T).reshape(n, Hkv, dh)
    q = rope(q, positions, cfg["theta"])
    k = rope(k, positions, cfg["theta"])
    k_new = k.transpose(1, 0, 2)
    v_new = v.transpose(1, 0, 2)
    K = np.concatenate([K_prev, k_new], axis=1)
    V = np.concatenate([V_prev, v_new], axis=1)
    o = attention(q, K, V, allowed).reshape(n, Hq * dh)
    h = h + o @ W.get("wo", l).T
    u2 = rmsnorm(h, cfg["eps"])
    f, r, ids, gates = moe(cfg, W, l, u2, forced_ids)
    h = h + f
    return h, k_new, v_new, dict(router=r, ids=ids, gates=gates)


def empty_cache(cfg):
    Hkv, dh = cfg["Hkv"], cfg["dh"]
    return [(np.zeros((Hkv, 0, dh)), np.zeros((Hkv, 0, dh))) for _ in range(cfg["L"])]


def forward(cfg, W, ids, positions, cache, causal=False, head=True, trace=None, forced_routing=None):
    """Forward of token ids at the given positions over a KV cache.

    cache: per-layer (K, V) [Hkv][m][dh] of the committed history.
    causal=False: the canvas mode (no mask).  causal=True: token i also sees
    new tokens j <= i (prefill).  Returns (logits or None, new per-layer
    (k, v), final hidden rows).  ``trace`` (a list) receives each layer's input.
    ``forced_routing`` (optional, per layer [n][k] or None) follows given
    top-k choices (see moe).
    """
    h = W.rows("embed", np.asarray(ids))
    n = h.shape[0]
    new_kv = []
    for l in range(cfg["L"]):
        K_prev, V_prev = cache[l]
        allowed = None
        if causal:
            m = K_prev.shape[1]
            allowed = np.concatenate([np.ones((n, m), bool), np.tril(np.ones((n, n), bool))], axis=1)
        if trace is not None:
            trace.append(dict(h_in=h.copy()))
        fr = None if forced_routing is None else forced_routing[l]
        h, k_new, v_new, tr = layer(cfg, W, l, h, positions, K_prev, V_prev, allowed, fr)
        if trace is not None:
            trace[-1].update(tr)
        new_kv.append((k_new, v_new))
    logits = lm_head(cfg, W, h) if head else None
    return logits, new_kv, h


def lm_head(cfg, W, h, vocab_rows=None):
    """Logits z = RMSNorm(h) W_lm^T (optionally only some vocabulary rows)."""
    u = rmsnorm(h, cfg["eps"])
    Wl = W.get("lm") if vocab_rows is None else W.rows("lm", vocab_rows)
    return u @ Wl.T
