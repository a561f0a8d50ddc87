"""Parity at the realistic width (30 layers, d=2816, 128 experts top-8 plus a
shared FFN, vocabulary 262144, bf16, 4096-token prefix), in the launch
configuration bench.py times.  The oracle cannot run the whole step in a test,
so it checks what it can compute one item at a time:

* the canvas start ids (bit-exact Philox);
* layer-0 prefill keys at sampled prompt positions (they depend only on the
  token);
* one denoise pass, layer by layer: from the GPU's traced input of layer l
  and the GPU's K/V cache, the oracle recomputes the canvas K/V and the
  layer's output for sampled canvas rows and compares it with the GPU's input
  of layer l+1 (the final residual for the last layer), following the GPU's
  routing under the near-tie rule;
* the LM head on sampled vocabulary rows from the GPU's final residual;
* the sampler on the GPU's own logits (all 256 x 262144).
The same step with MXFP4 experts and fp8 attention (``step_mxfp4``) is
checked the same way.  Tolerance: bf16 2e-2, MXFP4 6e-2 (per-row relative
L2)."""
import numpy as np
import pytest
import torch

import synth_inputs
from block_text_diffusion_amd import binding as B
from block_text_diffusion_amd.engine import Engine
from oracle import loop, model, philox, sampler as osamp
from oracle.weights import Weights
from tests.gpu_util import TOL, announce, rel_l2_rows, to_np
from tests.oracle_rows import layer_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["step_bf16", "step_mxfp4"])
def test_step_full_width_sampled_parity(name):
    w = synth_inputs.workload(name)
    tol = TOL[w["wdtype"]]
    announce("full_width_step", workload=name, L=w["L"], d=w["d"], E=w["E"], V=w["V"], P0=w["P0"])
    L, C, d, k, P0, V = w["L"], w["C"], w["d"], w["k"], w["P0"], w["V"]
    eng = Engine(w, max_ctx=P0 + C)
    B.cd_synth_weights(eng.ctx, w["weight_seed"])
    prefix = synth_inputs.prefix_ids(V, P0, w["prefix_seed"])
    B.cd_prefill(eng.ctx, 0, torch.from_numpy(prefix).cuda())
    seed = w["gen_seed"]
    B.cd_init_canvas(eng.ctx, 0, seed, 0)
    x = eng.canvas()[0].cpu().numpy()
    assert np.array_equal(x, philox.token_draw(seed, np.arange(C), 0, 0, 0, V))

    check_layers = [0, L - 1]
    th = torch.zeros(L, C, d, dtype=torch.float32, device="cuda")
    tid = torch.zeros(L, C, k, dtype=torch.int32, device="cuda")
    tg = torch.zeros(L, C, k, dtype=torch.float32, device="cuda")
    B.cd_set_trace(eng.ctx, th, tid, tg)
    B.cd_denoise_step(eng.ctx, 1, eng.info)
    info = eng.step_info()[0]
    B.cd_set_trace(eng.ctx)
    hs = {l: to_np(th[l]) for l in check_layers + [l + 1 for l in check_layers if l + 1 < L]}
    ids = {l: to_np(tid[l]) for l in check_layers}
    hfinal = to_np(eng.view(B.CD_BUF_HIDDEN, torch.float32, (C, d)))
    kc = {l: to_np(eng.kcache()[0, l, :, :P0 + C, :]) for l in check_layers}
    vc = {l: to_np(eng.vcache()[0, l, :, :, :P0 + C]).transpose(0, 2, 1) for l in check_layers}
    z = eng.logits().cpu().numpy()
    am = eng.argmax()[0].cpu().numpy()
    lock = to_np(eng.view(B.CD_BUF_LOCK, torch.uint8, (1, C))[0]).astype(bool)
    xn = eng.canvas()[0].cpu().numpy()
    H = to_np(eng.view(B.CD_BUF_ENTROPY, torch.float64, (1, C))[0])
    eng.close()

    # layer-0 prefill keys at sampled prompt positions
    W0 = Weights(w)
    ppos = np.array([0, 1, 777, 2048, P0 - 1])
    u0 = model.rmsnorm(W0.rows("embed", prefix[ppos]), w["eps"])
    k0 = model.rope((u0 @ W0.get("wk", 0).T).reshape(len(ppos), w["Hkv"], w["dh"]), ppos, w["theta"])
    got = kc[0][:, ppos, :].transpose(1, 0, 2)
    assert rel_l2_rows(got.reshape(len(ppos), -1), k0.reshape(len(ppos), -1)).max() <= tol

    # layers, from the GPU's own inputs
    pos = P0 + np.arange(C)
    rows = np.array([5, 137])
    adopted = 0
    for l in check_layers:
        W = Weights(w)
        h_out, kr, vr, ad = layer_rows(w, W, l, hs[l], rows, kc[l], vc[l], pos, ids[l][rows], tol)
        adopted += ad
        got_k = kc[l][:, P0 + rows, :].transpose(1, 0, 2)
        got_v = vc[l][:, P0 + rows, :].transpose(1, 0, 2)
        assert rel_l2_rows(got_k.reshape(len(rows), -1), kr.reshape(len(rows), -1)).max() <= tol, l
        assert rel_l2_rows(got_v.reshape(len(rows), -1), vr.reshape(len(rows), -1)).max() <= tol, l
        nxt = hs[l + 1] if l + 1 < L else hfinal
        assert rel_l2_rows(nxt[rows], h_out).max() <= tol, l
        del W
    print(f"routing decisions adopted from near-ties: {adopted}")

    # LM head on sampled vocabulary rows
    vrows = np.random.default_rng(0).choice(V, size=512, replace=False)
    vrows.sort()
    zref = model.lm_head(w, W0, hfinal, vocab_rows=vrows)
    assert rel_l2_rows(z[:, vrows], zref).max() <= tol

    # sampler on the GPU's own logits
    ref = osamp.sample(w, z, seed, 1, 0, 0)
    decided = ref["margin"] > 1e-3
    assert np.array_equal(am[decided], ref["a"][decided])
    ok = np.abs(ref["pmax"] - w["lock"]) > 1e-3
    assert np.array_equal(lock[ok], ref["lock"][ok])
    same = lock == ref["lock"]
    assert np.array_equal(xn[same & ~lock], ref["x_next"][same & ~lock])
    assert np.all(np.abs(H - ref["H"]) <= 1e-5 + 1e-5 * ref["H"])
    assert abs(info.mean_entropy - ref["Hbar"]) <= 1e-6 * ref["Hbar"]
    assert info.step == 1 and info.stop == 0
