"""Vocabulary-wide sampler, lock / re-noise rule and adaptive stop, in fp64.

What the pages fix ([P3] step ③ and FAQ 3; [P4] "how text diffusion works";
[P1] §2.1 table; [P5] "how text diffusion works"):
* each pass predicts every canvas position at once; confident positions are
  kept (locked) and used as context, uncertain ones are re-noised and chosen
  again in a later pass;
* the canvas starts as token ids drawn uniformly from the whole vocabulary,
  not as mask tokens ([P3] step ② and pitfall 2);
* the loop stops when the canvas mean entropy is below 0.005 and the
  highest-probability token at every position is the same in two consecutive
  passes; 48 passes per block is the recommended cap.
Readings where the pages are silent: entropy in nats; argmax ties go to the
lowest id; lock when max probability > 0.9 (strict), re-evaluated at every
pass (a locked position takes this pass's argmax, it is not frozen);
re-noise draws a fresh uniform id from Philox keyed by (seed; position, pass,
block, request); stability compares this pass's argmax with the previous
pass's at all positions, so the earliest stop is pass 2; both stop conditions
are strict and tested at the same pass; pass 48 always stops.
Entropy-bound variant ([P3] A/B guide: the serving example selects an
entropy-bound sampler with bound 0.1 and says no more): the same keep or
re-noise choice per position, made on the entropy: keep the argmax when
H <= bound (nats, inclusive), else re-noise.

Pins (tests/test_oracle_sampler.py): uniform logits give H = ln V exactly;
two-level distributions against their closed form; H in [0, ln V];
p_max = 1/sum(exp(z - max)); argmax ties; the stop truth table; entropy-bound
decisions on two-level rows whose closed-form entropy straddles the bound.
"""
from __future__ import annotations

import numpy as np

from . import philox


def row_stats(z):
    """Per row of logits z[n][V]: entropy H (nats), argmax a, max prob, top-2
    probability margin.  Rows are processed in chunks to bound memory."""
    z = np.asarray(z)
    n = z.shape[0]
    H = np.empty(n); pmax = np.empty(n); margin = np.empty(n)
    a = np.empty(n, dtype=np.int64)
    for r0 in range(0, n, 16):
        zz = np.asarray(z[r0:r0 + 16], dtype=np.float64)
        zmax = zz.max(axis=1, keepdims=True)
        e = np.exp(zz - zmax)
        p = e / e.sum(axis=1, keepdims=True)
        plogp = np.where(p > 0, p * np.log(np.where(p > 0, p, 1.0)), 0.0)
        H[r0:r0 + 16] = -plogp.sum(axis=1)
        a[r0:r0 + 16] = np.argmax(zz, axis=1)          # first (lowest) index of the max
        top = np.partition(p, p.shape[1] - 2, axis=1)[:, -2:] if p.shape[1] > 1 else np.concatenate([p, 0 * p], 1)
        pmax[r0:r0 + 16] = top.max(axis=1)
        margin[r0:r0 + 16] = top.max(axis=1) - top.min(axis=1)
    return H, a, pmax, margin


def sample(cfg, z, seed, step, block, req, pos=None):
    """One sampler pass over canvas logits z[C][V] after pass ``step``.

    ``pos`` (optional) gives the canvas positions of the rows of z when z
    holds only some of them (default: rows 0..C-1); every quantity except
    Hbar is per position, and Hbar is then the mean over the given rows.
    Returns dict(H, a, pmax, margin, lock, x_next, Hbar).
    """
    H, a, pmax, margin = row_stats(z)
    if cfg.get("lock_rule", "maxprob") == "entropy":
        lock = H <= cfg["entropy_bound"]
    else:
        lock = pmax > cfg["lock"]
    pos = np.arange(z.shape[0]) if pos is None else np.asarray(pos)
    noise = philox.token_draw(seed, pos, step, block, req, z.shape[1])
    x_next = np.where(lock, a, noise)
    return dict(H=H, a=a, pmax=pmax, margin=margin, lock=lock,
                x_next=x_next.astype(np.int64), Hbar=float(H.mean()))


def stop_rule(t, Hbar, a_t, a_prev, stop_H, max_steps):
    """Adaptive stop after pass t (1-based)."""
    if t >= max_steps:
        return True
    if t < 2 or a_prev is None:
        return False
    return bool(Hbar < stop_H and np.array_equal(np.asarray(a_t), np.asarray(a_prev)))
