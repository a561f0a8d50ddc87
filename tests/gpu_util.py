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


TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}
