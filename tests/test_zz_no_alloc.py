"""The allocation-free sampler entry point (cd_sample_step_noalloc, the
partials in the library's fixed per-GPU buffer) against cd_sample_step with
a caller workspace, through the C ABI, on two calls in a row (the second
smaller, with a previous argmax, so stale partials of the first would show)
and on a request beyond the fixed buffer (refused, nothing written)."""
import numpy as np
import pytest
import torch

import synth_inputs
from block_text_diffusion_amd import binding as B
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu


def _bufs(rows, C, dev):
    return dict(tok=torch.full((rows,), -7, dtype=torch.int32, device=dev),
                am=torch.full((rows,), -7, dtype=torch.int32, device=dev),
                lk=torch.full((rows,), 9, dtype=torch.uint8, device=dev),
                H=torch.full((rows,), -1.0, dtype=torch.float64, device=dev),
                pm=torch.full((rows,), -1.0, dtype=torch.float64, device=dev),
                info=torch.zeros(rows // C * B.STEP_INFO_BYTES, dtype=torch.uint8, device=dev))


def _call(noalloc, cfg, z, rows, prev, seed, step, block, req0, b, dev):
    if noalloc:
        B.cd_sample_step_noalloc(cfg, z, rows, prev, seed, step, block, req0, b["tok"], b["am"], b["lk"], b["H"],
                                 b["pm"], b["info"])
    else:
        ws = torch.empty(B.cd_sample_workspace_bytes(rows, cfg.vocab), dtype=torch.uint8, device=dev)
        B.cd_sample_step(cfg, z, rows, prev, seed, step, block, req0, b["tok"], b["am"], b["lk"], b["H"],
                         b["pm"], b["info"], ws)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in b.items()}


def test_noalloc_sampler_equals_workspace_sampler():
    dev = torch.device("cuda")
    cases = [(512, 262144, None, 3, 1, 0, 0), (256, 32768, "prev", 5, 4, 2, 7)]
    for rows, V, prev, seed, step, block, req0 in cases:
        announce("noalloc_sampler", rows=rows, V=V)
        w = synth_inputs.workload("tiny", V=V)
        cfg = B.make_config(w)
        z = torch.from_numpy(synth_inputs.sampler_logits(rows, V, seed)).to(dev)
        pv = None
        if prev:
            pv = torch.from_numpy(np.random.default_rng(0).integers(0, V, rows).astype(np.int32)).to(dev)
            pv[:128] = z[:128].argmax(dim=1).to(torch.int32)
        got = _call(True, cfg, z, rows, pv, seed, step, block, req0, _bufs(rows, w["C"], dev), dev)
        ref = _call(False, cfg, z, rows, pv, seed, step, block, req0, _bufs(rows, w["C"], dev), dev)
        for k in ("tok", "am", "lk", "H", "pm", "info"):
            assert torch.equal(got[k], ref[k]), (rows, V, k)
        assert (got["am"] >= 0).all() and (got["H"] >= 0).all()


def test_noalloc_sampler_refuses_beyond_its_buffer():
    dev = torch.device("cuda")
    w = synth_inputs.workload("tiny", V=262144)
    cfg = B.make_config(w)
    rows = 2304                                      # 2304 x 32 chunks > 65536 partials
    announce("noalloc_sampler_capacity", rows=rows)
    z = torch.zeros(1, dtype=torch.float32, device=dev)
    b = _bufs(256, w["C"], dev)
    with pytest.raises(B.CDError) as e:
        B.cd_sample_step_noalloc(cfg, z, rows, None, 1, 1, 0, 0, b["tok"], b["am"], b["lk"], b["H"], b["pm"],
                                 b["info"])
    assert e.value.code == B.CD_ERR_CAPACITY
    torch.cuda.synchronize()
    assert (b["tok"] == -7).all()
