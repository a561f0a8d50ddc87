"""Seeded synthetic inputs shared by the HIP path's callers and the oracle.

This module holds workload shapes and seeded input generators only.  It holds
none of the method's arithmetic: no Philox, no weight generator, no sampler.
Random numbers that the method itself draws (canvas initialisation, re-noise)
and the synthetic weights are produced on each side by its own implementation
of Philox4x32-10; only the data handed in from outside (prompt token ids and
the sampler-only logits) comes from here, through numpy's PCG64 generator.

Workloads (shapes follow the DiffusionGemma pages: 256-token canvas, step cap
48, stop threshold 0.005 nats, MoE backbone of the 26B-A4B family):

* ``tiny``      2 layers, d=256, 4/2 heads of 64, 8 experts top-2 (hidden 512),
                vocab 4096, fp32, prefix 128 tokens, one block.
* ``sampler``   sampler only: fp32 logits 256 x 262144, row sigma ~ U[0.5, 8].
* ``step_bf16`` 30 layers, d=2816, 16/8 heads of 128, 128 experts top-8
                (hidden 704) plus a shared FFN (hidden 2112), vocab 262144,
                bf16, prefix 4096 tokens, one denoise step.
* ``gen_bf16``  the ``step_bf16`` model generating 4 blocks of 256 tokens.
* ``batch_fp8`` the ``step_bf16`` model with fp8 e4m3 attention and expert
                weights, 32 requests of 4096-token prefixes.
* ``step_mxfp4`` the ``step_bf16`` step with MXFP4 experts and fp8 attention.
* ``batch_mxfp4`` the ``batch_fp8`` batch with MXFP4 experts.
"""
from __future__ import annotations

import copy

import numpy as np

CANVAS = 256          # canvas length (tokens per block)
MAX_STEPS = 48        # recommended per-block step cap
LOCK_THRESHOLD = 0.9  # lock a position when its max probability exceeds this
STOP_ENTROPY = 0.005  # adaptive stop: mean canvas entropy below this (nats)

_COMMON = dict(C=CANVAS, max_steps=MAX_STEPS, lock=LOCK_THRESHOLD,
               stop_H=STOP_ENTROPY, eps=1e-6, theta=10000.0,
               weight_seed=0, gen_seed=1, prefix_seed=2)

WORKLOADS = {
    "tiny": dict(_COMMON, L=2, d=256, Hq=4, Hkv=2, dh=64, E=8, k=2, fe=512,
                 fs=0, V=4096, wdtype="f32", P0=128, R=1, blocks=1),
    "sampler": dict(_COMMON, T=256, V=262144, logits_seed=1),
    "step_bf16": dict(_COMMON, L=30, d=2816, Hq=16, Hkv=8, dh=128, E=128, k=8,
                      fe=704, fs=2112, V=262144, wdtype="bf16", P0=4096, R=1,
                      blocks=1),
    "gen_bf16": dict(_COMMON, L=30, d=2816, Hq=16, Hkv=8, dh=128, E=128, k=8,
                     fe=704, fs=2112, V=262144, wdtype="bf16", P0=4096, R=1,
                     blocks=4),
    "batch_fp8": dict(_COMMON, L=30, d=2816, Hq=16, Hkv=8, dh=128, E=128, k=8,
                      fe=704, fs=2112, V=262144, wdtype="fp8", P0=4096, R=32,
                      blocks=1),
    "step_mxfp4": dict(_COMMON, L=30, d=2816, Hq=16, Hkv=8, dh=128, E=128, k=8,
                       fe=704, fs=2112, V=262144, wdtype="mxfp4", P0=4096, R=1,
                       blocks=1),
    "batch_mxfp4": dict(_COMMON, L=30, d=2816, Hq=16, Hkv=8, dh=128, E=128, k=8,
                        fe=704, fs=2112, V=262144, wdtype="mxfp4", P0=4096, R=32,
                        blocks=1),
}


def workload(name: str, **overrides) -> dict:
    """A copy of a named workload with optional overrides."""
    w = copy.deepcopy(WORKLOADS[name])
    w.update(overrides)
    w["name"] = name
    return w


def prefix_ids(V: int, n: int, seed: int, req: int = 0) -> np.ndarray:
    """Prompt token ids: n ids uniform over [0, V), one stream per request."""
    rng = np.random.Generator(np.random.PCG64([seed, req]))
    return rng.integers(0, V, size=n, dtype=np.int64).astype(np.int32)


def sampler_logits(T: int, V: int, seed: int) -> np.ndarray:
    """fp32 logits [T][V]; row r is N(0, sigma_r) with sigma_r ~ U[0.5, 8]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    sigma = rng.uniform(0.5, 8.0, size=T)
    out = np.empty((T, V), dtype=np.float32)
    for r in range(T):
        out[r] = (rng.standard_normal(V) * sigma[r]).astype(np.float32)
    return out
