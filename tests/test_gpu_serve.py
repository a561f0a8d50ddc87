"""The batched retire/admit loop (cd_serve) and idle slots riding along in a
pass, through the C ABI, against the oracle.

* a queue of three requests with 1, 3 and 1 blocks and prompts of different
  lengths on two slots: a finished request hands its slot to the next queued
  one, and once the queue is empty the request in slot 1 moves down to the
  idle slot 0 for its last block.  The step cap of 2 makes every block stop at pass
  2, so the pass counts are known and each committed block is pass 2's argmax
  of the oracle run of that request on its own, with its Philox streams keyed
  by its queue index (a wrong key changes the re-noised canvas that pass 2
  sees and with it the argmax nearly everywhere).  Positions whose oracle top
  two logits lie within 1e-4 are excluded (fp32 reduction order may swap
  them); the rest must match exactly.
* cd_denoise_step with an idle slot: its canvas, committed length and
  sampler outputs stay as they were and its record is all zero.
* cd_move_request in the middle of a block: the moved request continues,
  commits and starts its next block in the new slot and still matches the
  oracle run of its own request index.
* a loop that fails (non-finite logits) releases every slot."""
import numpy as np
import pytest
import torch

import synth_inputs
from block_text_diffusion_amd import binding as B
from block_text_diffusion_amd.engine import Engine
from oracle import loop
from oracle.weights import Weights
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu


def test_serve_queue_matches_oracle_per_request():
    w = synth_inputs.workload("tiny", max_steps=2)
    C = w["C"]
    lens, n_blocks, seeds = [40, 64, 17], [1, 3, 1], [5, 6, 7]
    announce("serve_queue", lens=lens, blocks=n_blocks, slots=2)
    prefs = [synth_inputs.prefix_ids(w["V"], n, 31, q) for q, n in enumerate(lens)]
    eng = Engine(w, max_requests=2, max_ctx=64 + 3 * C, max_prefill=64)
    B.cd_synth_weights(eng.ctx, w["weight_seed"])
    out = torch.full((sum(n_blocks) * C,), -1, dtype=torch.int32, device="cuda")
    steps = B.cd_serve(eng.ctx, [torch.from_numpy(p).cuda() for p in prefs], n_blocks, seeds, 2, out)
    torch.cuda.synchronize()
    assert steps == [[2], [2, 2, 2], [2]]
    assert [B.cd_get_length(eng.ctx, r) for r in range(2)] == [0, 0]
    got = out.cpu().numpy().astype(np.int64)
    eng.close()
    W = Weights(w)
    off = 0
    for q in range(3):
        req = loop.Request(w, q)
        loop.prefill(w, W, req, prefs[q])
        for b in range(n_blocks[q]):
            x = loop.init_canvas(w, seeds[q], b, q)
            for t in (1, 2):
                ref = loop.denoise_pass(w, W, req, x, t, b, seeds[q])
                x = ref["x_next"]
            ids = got[off:off + C]
            srt = np.sort(ref["z"], axis=1)
            clear = srt[:, -1] - srt[:, -2] > 1e-4
            assert clear.mean() > 0.9
            assert np.array_equal(ids[clear], ref["a"][clear]), (q, b)
            loop.commit(w, W, req, ids)
            off += C


def test_idle_slot_rides_along_unchanged():
    w = synth_inputs.workload("tiny")
    C = w["C"]
    announce("serve_idle_slot")
    eng = Engine(w, max_requests=2, max_ctx=64 + 2 * C, max_prefill=w["P0"])
    B.cd_synth_weights(eng.ctx, w["weight_seed"])
    for r in range(2):
        B.cd_prefill(eng.ctx, r, torch.from_numpy(synth_inputs.prefix_ids(w["V"], 50 + r, 3, r)).cuda())
    B.cd_init_canvas(eng.ctx, 0, 9, 0)
    B.cd_denoise_step(eng.ctx, 1, eng.info)
    B.cd_commit_block(eng.ctx, 0, torch.empty(C, dtype=torch.int32, device="cuda"))
    B.cd_init_canvas(eng.ctx, 1, 9, 0)
    torch.cuda.synchronize()
    before = [t.clone() for t in (eng.canvas()[0], eng.argmax()[0])]
    P0 = B.cd_get_length(eng.ctx, 0)
    assert P0 == 50 + C
    B.cd_denoise_step(eng.ctx, 2, eng.info)          # slot 0 idle, slot 1 active
    info = eng.step_info(2)
    assert (info[0].step, info[0].stop, info[0].n_locked, info[0].mean_entropy) == (0, 0, 0, 0.0)
    assert info[1].step == 1
    assert torch.equal(eng.canvas()[0], before[0]) and torch.equal(eng.argmax()[0], before[1])
    assert B.cd_get_length(eng.ctx, 0) == P0
    # slot 1's pass equals the same pass with slot 1 alone (fp32 to 1e-5)
    z_batch = eng.logits(2)[C:].clone()
    eng.close()
    eng = Engine(w, max_requests=2, max_ctx=64 + 2 * C, max_prefill=w["P0"])
    B.cd_synth_weights(eng.ctx, w["weight_seed"])
    B.cd_prefill(eng.ctx, 1, torch.from_numpy(synth_inputs.prefix_ids(w["V"], 51, 3, 1)).cuda())
    B.cd_init_canvas(eng.ctx, 1, 9, 0)
    B.cd_denoise_step(eng.ctx, 2, eng.info)          # slot 0 idle with nothing committed
    z_alone = eng.logits(2)[C:].clone()
    eng.close()
    err = ((z_batch - z_alone).norm(dim=1) / z_alone.norm(dim=1)).max().item()
    assert err <= 1e-5


def test_move_mid_block_matches_oracle():
    # request 1 runs pass 1 in slot 1 (slot 0 idle), moves to slot 0, runs
    # pass 2 there, commits and starts its second block through the public
    # calls: every draw stays keyed by request index 1
    w = synth_inputs.workload("tiny")
    C, seed = w["C"], 4
    announce("serve_move_mid_block")
    pre = synth_inputs.prefix_ids(w["V"], 70, 8, 1)
    eng = Engine(w, max_requests=2, max_ctx=70 + 2 * C, max_prefill=w["P0"])
    B.cd_synth_weights(eng.ctx, w["weight_seed"])
    B.cd_prefill(eng.ctx, 1, torch.from_numpy(pre).cuda())
    B.cd_init_canvas(eng.ctx, 1, seed, 0)
    B.cd_denoise_step(eng.ctx, 2, eng.info)
    with pytest.raises(B.CDError) as e:
        B.cd_move_request(eng.ctx, 0, 1)                 # slot 1 is not free
    assert e.value.code == B.CD_ERR_BAD_STATE
    B.cd_move_request(eng.ctx, 1, 0)
    assert [B.cd_get_length(eng.ctx, r) for r in range(2)] == [70, 0]
    B.cd_denoise_step(eng.ctx, 1, eng.info)
    assert eng.step_info(1)[0].step == 2
    got = []
    ids = torch.empty(C, dtype=torch.int32, device="cuda")
    B.cd_commit_block(eng.ctx, 0, ids)
    got.append(ids.cpu().numpy().astype(np.int64))
    B.cd_init_canvas(eng.ctx, 0, seed, 1)
    for _ in range(2):
        B.cd_denoise_step(eng.ctx, 1, eng.info)
    assert eng.step_info(1)[0].step == 2
    B.cd_commit_block(eng.ctx, 0, ids)
    got.append(ids.cpu().numpy().astype(np.int64))
    assert B.cd_get_length(eng.ctx, 0) == 70 + 2 * C
    eng.close()
    W = Weights(w)
    req = loop.Request(w, 1)
    loop.prefill(w, W, req, pre)
    for b in range(2):
        x = loop.init_canvas(w, seed, b, 1)
        for t in (1, 2):
            ref = loop.denoise_pass(w, W, req, x, t, b, seed)
            x = ref["x_next"]
        srt = np.sort(ref["z"], axis=1)
        clear = srt[:, -1] - srt[:, -2] > 1e-4
        assert clear.mean() > 0.9
        assert np.array_equal(got[b][clear], ref["a"][clear]), b
        loop.commit(w, W, req, got[b])


def test_serve_failure_releases_slots():
    # NaN LM-head weights make every logit NaN: the sampler flags it, the
    # loop stops with CD_ERR_NUMERIC, and every slot is released
    w = synth_inputs.workload("tiny")
    C = w["C"]
    announce("serve_failure_path")
    eng = Engine(w, max_requests=2, max_ctx=64 + C, max_prefill=64)
    B.cd_synth_weights(eng.ctx, w["weight_seed"])
    B.cd_set_weight(eng.ctx, B.CD_W_LM, 0, 0, torch.full((w["V"], w["d"]), float("nan"), device="cuda"))
    prefs = [torch.from_numpy(synth_inputs.prefix_ids(w["V"], 30 + q, 2, q)).cuda() for q in range(3)]
    out = torch.empty(3 * C, dtype=torch.int32, device="cuda")
    with pytest.raises(B.CDError) as e:
        B.cd_serve(eng.ctx, prefs, [1, 1, 1], [1, 2, 3], 2, out)
    assert e.value.code == B.CD_ERR_NUMERIC
    assert [B.cd_get_length(eng.ctx, r) for r in range(2)] == [0, 0]
    B.cd_init_canvas(eng.ctx, 0, 1, 0)                 # no canvas was left active
    eng.close()
