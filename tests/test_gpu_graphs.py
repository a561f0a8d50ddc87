"""Graph replay of denoise passes (cd_set_graphs) against the same passes
launched one by one, through the C ABI.

Two contexts run the same prefills, canvas starts and passes, one with graph
replay (the default) and one with it switched off; after every pass the
logits, canvases, argmax, lock bits, entropies, step records and the K/V
cache must be bit-identical.  Between passes the program does eager work of
its own (a torch reduction and a synchronising step-record read), the graph
of a configuration is replayed several times, a commit moves a request's
context length (a new graph), and a slot without a canvas rides along (its
active mask is part of the graph's key)."""
import numpy as np
import pytest
import torch

import synth_inputs
from block_text_diffusion_amd import binding as B
from block_text_diffusion_amd.engine import Engine
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu


def small(wdtype, **kw):
    base = dict(wdtype=wdtype, dh=128, Hq=4, Hkv=2, E=16, k=4, fe=256, fs=128, V=4096, P0=100)
    base.update(kw)
    return synth_inputs.workload("tiny", **base)


@pytest.mark.parametrize("wdtype", ["f32", "bf16"])
def test_graph_replay_equals_launches_one_by_one(wdtype):
    w = small(wdtype, C=128, max_steps=48)
    C = w["C"]
    announce("graphs", wdtype=wdtype)
    engs = []
    for graphs in (True, False):
        eng = Engine(w, max_requests=2, max_ctx=w["P0"] + 3 * C, max_prefill=w["P0"])
        B.cd_set_graphs(eng.ctx, graphs)
        B.cd_synth_weights(eng.ctx, w["weight_seed"])
        for r, n in enumerate((w["P0"], 37)):
            B.cd_prefill(eng.ctx, r, torch.from_numpy(synth_inputs.prefix_ids(w["V"], n, 7, r)).cuda())
            B.cd_init_canvas(eng.ctx, r, 11, 0)
        engs.append(eng)

    def snap(eng, n_req):
        torch.cuda.synchronize()
        return dict(z=eng.logits(n_req).clone(), x=eng.canvas().clone(), a=eng.argmax().clone(),
                    K=eng.kcache().clone(), V=eng.vcache().clone(),
                    H=eng.view(B.CD_BUF_ENTROPY, torch.float64, (2, C)).clone(),
                    L=eng.view(B.CD_BUF_LOCK, torch.uint8, (2, C)).clone())

    def compare(tag, n_req):
        s0, s1 = snap(engs[0], n_req), snap(engs[1], n_req)
        for key in s0:
            assert torch.equal(s0[key], s1[key]), (tag, key)
        i0, i1 = engs[0].step_info(n_req), engs[1].step_info(n_req)
        for a, b in zip(i0, i1):
            assert (a.step, a.n_locked, a.stable, a.stop, a.canvas_is_argmax, a.mean_entropy) == \
                   (b.step, b.n_locked, b.stable, b.stop, b.canvas_is_argmax, b.mean_entropy), tag

    scratch = torch.randn(1 << 20, device="cuda")
    for t in range(4):                       # one graph, replayed with eager work between the passes
        for eng in engs:
            B.cd_denoise_step(eng.ctx, 2, eng.info)
        float(scratch.sum())                 # the program's own work on the same stream
        compare(f"pass {t + 1}", 2)
    # a commit moves request 0's context length: a new graph for the next passes
    ids = [torch.empty(C, dtype=torch.int32, device="cuda") for _ in engs]
    for eng, out in zip(engs, ids):
        B.cd_commit_block(eng.ctx, 0, out)
        B.cd_init_canvas(eng.ctx, 0, 11, 1)
    assert torch.equal(ids[0], ids[1])
    for t in range(3):
        for eng in engs:
            B.cd_denoise_step(eng.ctx, 2, eng.info)
        compare(f"block 1 pass {t + 1}", 2)
    # request 1 commits and stays without a canvas: it rides along (another
    # active mask, another graph); then back to the first graph's key is not
    # possible (request 0 advanced), so replay the new one twice
    for eng, out in zip(engs, ids):
        B.cd_commit_block(eng.ctx, 1, out)
    assert torch.equal(ids[0], ids[1])
    for t in range(2):
        for eng in engs:
            B.cd_denoise_step(eng.ctx, 2, eng.info)
        compare(f"ride-along pass {t + 1}", 2)
    # switching graphs off on the first context releases them; passes continue
    B.cd_set_graphs(engs[0].ctx, False)
    for eng in engs:
        B.cd_denoise_step(eng.ctx, 2, eng.info)
    compare("after switching off", 2)
    for eng in engs:
        eng.close()
