"""Shared helpers of the GPU parity tests (no method arithmetic here)."""
import sys

import numpy as np
import torch


def announce(name, **kw):
    """Print the case before any GPU work so a fault still names it."""
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)
    sys.stdout.flush()


def rel_l2_rows(got, ref):
    """Per-row ||got - ref|| / ||ref||, the tolerance metric for hidden states
    and logits."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm((got - ref).reshape(got.shape[0], -1), axis=1)
    den = np.linalg.norm(ref.reshape(ref.shape[0], -1), axis=1)
    return num / np.maximum(den, 1e-300)


def to_np(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2, "mxfp4": 6e-2}


def check_routing(gpu_ids, oracle_trace, k, band):
    """Lockstep check of routing decisions.

    oracle_trace: the oracle's per-layer trace of a run that followed the GPU's
    routing (forced ids).  A GPU top-k set must equal the oracle's own top-k of
    its router logits, or every expert the GPU chose must lie within
    band * rms(logits) of the oracle's k-th largest logit (a near-tie that
    rounding may decide either way).  Returns the number of such adoptions.
    """
    adopted = 0
    for l, tr in enumerate(oracle_trace):
        r = tr["router"]
        g = np.asarray(gpu_ids[l][: r.shape[0]], dtype=np.int64)
        kth = np.sort(r, axis=1)[:, ::-1][:, k - 1]
        rms = np.sqrt(np.mean(r ** 2, axis=1))
        own = np.argsort(-r, axis=1, kind="stable")[:, :k]
        for t in range(r.shape[0]):
            if set(g[t]) == set(own[t]):
                continue
            chosen = r[t, g[t]]
            assert np.all(chosen >= kth[t] - band * rms[t]), (l, t, chosen, kth[t])
            adopted += 1
    return adopted
