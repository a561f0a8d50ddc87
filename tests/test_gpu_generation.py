"""Parity of the four-block generation on the realistic-width bf16 model
(the explainer's official benchmark shape: a 4,096-token prompt, 1,024
generated tokens as four 256-token blocks; steps ① to ④ per block), in the
launch configuration bench.py times for ``gen_bf16``.

test_generation_lockstep runs the whole generation and checks, against the
oracle:
* every canvas start (bit-exact Philox with the block index);
* every pass of block 0 and the first and last pass of blocks 1-3:
  layers 0 and 29 at 16 canvas rows from the GPU's own layer inputs and K/V
  cache (which holds the committed blocks), the LM head on sampled
  vocabulary rows, and the sampler on the GPU's full 256 x 262144 logits
  (argmax, lock bits, entropies, the next canvas);
* the stop: random weights never lock (max probability about 4e-4), so
  every block stops at exactly pass 48;
* every commit: the committed ids are the stopping pass's argmax, and the
  committed keys/values (recomputed from those ids, since the canvas at the
  cap differs from them) at layers 0 and 29 for 16 rows;
* the committed prefix is never written again (bit-identical cache below P
  after every later block).
test_generation_commit_every_layer checks the commit of block 0 and of block
3 at every layer (the committed block's keys/values and each layer's output
at 16 rows).  Tolerance bf16 2e-2 (per-row relative L2); routing follows the
near-tie rule with at most 4% of the checked decisions adopted."""
import numpy as np
import pytest
import torch

import synth_inputs
from block_text_diffusion_amd import binding as B
from block_text_diffusion_amd.engine import Engine
from oracle import model, philox
from oracle.weights import Weights
from tests.gpu_util import TOL, announce, rel_l2_rows, to_np
from tests.oracle_rows import Summary, check_layer
from tests.test_gpu_full_width import ADOPT_CAP, CANVAS_ROWS, check_sampler

pytestmark = pytest.mark.gpu


class Gen:
    """The GPU side: engine, prefill, and per-pass / per-commit downloads."""

    def __init__(self, w):
        self.w = w
        L, C, d, k, P0 = w["L"], w["C"], w["d"], w["k"], w["P0"]
        self.eng = Engine(w, max_ctx=P0 + w["blocks"] * C)
        B.cd_synth_weights(self.eng.ctx, w["weight_seed"])
        self.prefix = synth_inputs.prefix_ids(w["V"], P0, w["prefix_seed"])
        B.cd_prefill(self.eng.ctx, 0, torch.from_numpy(self.prefix).cuda())
        self.th = torch.zeros(L, C, d, dtype=torch.float32, device="cuda")
        self.tid = torch.zeros(L, C, k, dtype=torch.int32, device="cuda")
        self.tg = torch.zeros(L, C, k, dtype=torch.float32, device="cuda")
        self.rows = torch.from_numpy(CANVAS_ROWS).cuda()

    def trace(self, on):
        if on:
            B.cd_set_trace(self.eng.ctx, self.th, self.tid, self.tg)
        else:
            B.cd_set_trace(self.eng.ctx)

    def rows_of_forward(self, layers, P):
        """Traced inputs, routing and K/V of the last forward (positions
        P..P+C-1) for the checked rows at the given layers."""
        w, eng = self.w, self.eng
        C, d = w["C"], w["d"]
        out = {}
        hid = to_np(eng.view(B.CD_BUF_HIDDEN, torch.float32, (C, d))[self.rows])
        for l in layers:
            out[l] = dict(h=to_np(self.th[l, self.rows]),
                          h_next=to_np(self.th[l + 1, self.rows]) if l + 1 < w["L"] else hid,
                          ids=to_np(self.tid[l, self.rows]),
                          K=to_np(eng.kcache()[0, l, :, :P + C, :]).astype(np.float64),
                          V=to_np(eng.vcache()[0, l, :, :, :P + C]).astype(np.float64).transpose(0, 2, 1))
        return out, hid

    def close(self):
        self.eng.close()


def layer_items(fw, l, P, C):
    g = fw[l]
    pos = P + CANVAS_ROWS
    return [dict(name="canvas", h_in=g["h"], h_out=g["h_next"], pos=pos, K=g["K"], V=g["V"], causal=False,
                 ids=g["ids"], k_got=g["K"][:, pos].transpose(1, 0, 2), v_got=g["V"][:, pos].transpose(1, 0, 2))]


def test_generation_lockstep():
    w = synth_inputs.workload("gen_bf16")
    tol = TOL[w["wdtype"]]
    L, C, V, P0, nb, seed = w["L"], w["C"], w["V"], w["P0"], w["blocks"], w["gen_seed"]
    announce("generation_lockstep", workload="gen_bf16", blocks=nb, P0=P0)
    g = Gen(w)
    eng = g.eng
    Wc = Weights(w)                      # layers 0 and L-1 cached over all passes
    S = Summary("gen_bf16 lockstep")
    vrows = np.sort(np.random.default_rng(2).choice(V, size=64, replace=False))
    layers = (0, L - 1)
    prefix_kv = None
    for b in range(nb):
        P = P0 + b * C
        assert B.cd_get_length(eng.ctx, 0) == P
        B.cd_init_canvas(eng.ctx, 0, seed, b)
        x = eng.canvas()[0].cpu().numpy()
        assert np.array_equal(x, philox.token_draw(seed, np.arange(C), 0, b, 0, V)), b
        t = 0
        while True:
            t += 1
            checked = b == 0 or t in (1, w["max_steps"])
            g.trace(checked)
            B.cd_denoise_step(eng.ctx, 1, eng.info)
            info = eng.step_info()[0]
            assert info.step == t and info.nonfinite == 0
            if checked:
                g.trace(False)
                fw, hid = g.rows_of_forward(layers, P)
                for l in layers:
                    S.add_layer(check_layer(w, l, layer_items(fw, l, P, C), tol, W=Wc), "pass_")
                zr = model.lm_head(w, Wc, hid, vocab_rows=vrows)
                z = eng.logits().cpu().numpy()
                S.add("pass_lm_head", rel_l2_rows(z[CANVAS_ROWS][:, vrows], zr).max())
                assert S.err["pass_lm_head"] <= tol
                am = eng.argmax()[0].cpu().numpy()
                lock = to_np(eng.view(B.CD_BUF_LOCK, torch.uint8, (1, C))[0]).astype(bool)
                xn = eng.canvas()[0].cpu().numpy()
                H = to_np(eng.view(B.CD_BUF_ENTROPY, torch.float64, (1, C))[0])
                ref = check_sampler(w, z, am, lock, xn, H, info.mean_entropy, seed, t, b, 0)
                assert not ref["lock"].any() and ref["pmax"].max() < 0.01
                assert np.array_equal(xn, philox.token_draw(seed, np.arange(C), t, b, 0, V))
                print(f"block {b} pass {t}: max errors {S.err}", flush=True)
            if info.stop:
                break
        assert t == w["max_steps"], (b, t)               # random weights: the cap
        a_last = eng.argmax()[0].cpu().numpy()
        ids = torch.empty(C, dtype=torch.int32, device="cuda")
        g.trace(True)
        B.cd_commit_block(eng.ctx, 0, ids)
        g.trace(False)
        committed = ids.cpu().numpy()
        assert np.array_equal(committed, a_last)
        assert B.cd_get_length(eng.ctx, 0) == P + C
        fw, _ = g.rows_of_forward(layers, P)
        for l in layers:
            S.add_layer(check_layer(w, l, layer_items(fw, l, P, C), tol, W=Wc), "commit_")
        # the committed prefix below P is bit-identical after this block
        if prefix_kv is not None:
            Pp = prefix_kv[0].shape[-2]
            assert torch.equal(eng.kcache()[0, :, :, :Pp, :], prefix_kv[0]), b
            assert torch.equal(eng.vcache()[0, :, :, :, :Pp], prefix_kv[1]), b
        prefix_kv = (eng.kcache()[0, :, :, :P + C, :].clone(), eng.vcache()[0, :, :, :, :P + C].clone())
    g.close()
    S.report(ADOPT_CAP[w["wdtype"]])


@pytest.mark.parametrize("block", [0, 3])
def test_generation_commit_every_layer(block):
    w = synth_inputs.workload("gen_bf16")
    tol = TOL[w["wdtype"]]
    L, C, P0, seed = w["L"], w["C"], w["P0"], w["gen_seed"]
    announce("generation_commit_every_layer", workload="gen_bf16", block=block)
    g = Gen(w)
    eng = g.eng
    ids = torch.empty(C, dtype=torch.int32, device="cuda")
    for b in range(block + 1):
        B.cd_init_canvas(eng.ctx, 0, seed, b)
        while True:
            B.cd_denoise_step(eng.ctx, 1, eng.info)
            if eng.step_info()[0].stop:
                break
        a_last = eng.argmax()[0].cpu().numpy()
        g.trace(b == block)
        B.cd_commit_block(eng.ctx, 0, ids)
        g.trace(False)
    assert np.array_equal(ids.cpu().numpy(), a_last)
    P = P0 + block * C
    fw, _ = g.rows_of_forward(range(L), P)
    g.close()
    S = Summary(f"gen_bf16 commit of block {block}")
    for l in range(L):
        res = check_layer(w, l, layer_items(fw, l, P, C), tol)
        S.add_layer(res)
        print(f"layer {l}: {[{k2: float(f'{v:.2e}') for k2, v in r.items()} for r in res]}", flush=True)
    S.report(ADOPT_CAP[w["wdtype"]])
