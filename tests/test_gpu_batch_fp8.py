"""Parity of the 32-request fp8 batch at the realistic width (30 layers,
d=2816, 128 experts top-8 plus a shared FFN, vocabulary 262144, fp8 e4m3
attention and expert weights with per-row bf16 scales, 4096-token prefix per
request), one denoise pass over all 32 canvases in the launch configuration
bench.py times.  The oracle checks what it can compute item by item:

* every request's canvas start ids (bit-exact Philox, request index in the
  counter) for three requests;
* for the first and last request, sampled canvas rows through layers 0 and 29
  from the GPU's own layer inputs and K/V cache, following the GPU's routing
  under the near-tie rule;
* the LM head on sampled vocabulary rows of the last request;
* the sampler on the last request's GPU logits (its own Philox stream).
The same batch with MXFP4 experts (``batch_mxfp4``: 512 rows per expert, so
the expert GEMMs run the LDS-staged kernel's MXFP4 path at K = 2816 and 704)
is checked the same way.  Tolerance: fp8 and MXFP4 6e-2 (per-row relative
L2)."""
import numpy as np
import pytest
import torch

import synth_inputs
from block_text_diffusion_amd import binding as B
from block_text_diffusion_amd.engine import Engine
from oracle import model, philox, sampler as osamp
from oracle.weights import Weights
from tests.gpu_util import TOL, announce, rel_l2_rows, to_np
from tests.oracle_rows import layer_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["batch_fp8", "batch_mxfp4"])
def test_batch_full_width_sampled_parity(name):
    w = synth_inputs.workload(name)
    tol = TOL[w["wdtype"]]
    L, C, d, k, P0, V, R = w["L"], w["C"], w["d"], w["k"], w["P0"], w["V"], w["R"]
    announce("batch", workload=name, R=R, L=L, d=d, E=w["E"], V=V, P0=P0)
    eng = Engine(w, max_ctx=P0 + C)
    B.cd_synth_weights(eng.ctx, w["weight_seed"])
    for r in range(R):
        pre = synth_inputs.prefix_ids(V, P0, w["prefix_seed"], r)
        B.cd_prefill(eng.ctx, r, torch.from_numpy(pre).cuda())
    seed = w["gen_seed"]
    for r in range(R):
        B.cd_init_canvas(eng.ctx, r, seed, 0)
    canvas0 = eng.canvas().cpu().numpy()
    for r in (0, 17, R - 1):
        assert np.array_equal(canvas0[r], philox.token_draw(seed, np.arange(C), 0, 0, r, V)), r

    T = R * C
    th = torch.zeros(L, T, d, dtype=torch.float32, device="cuda")
    tid = torch.zeros(L, T, k, dtype=torch.int32, device="cuda")
    tg = torch.zeros(L, T, k, dtype=torch.float32, device="cuda")
    B.cd_set_trace(eng.ctx, th, tid, tg)
    B.cd_denoise_step(eng.ctx, R, eng.info)
    infos = eng.step_info(R)
    B.cd_set_trace(eng.ctx)
    assert all(i.step == 1 and i.stop == 0 and i.nonfinite == 0 for i in infos)

    check_req, check_layers = (0, R - 1), (0, L - 1)
    hid = eng.view(B.CD_BUF_HIDDEN, torch.float32, (T, d))
    got = {}
    for r in check_req:
        sl = slice(r * C, (r + 1) * C)
        for l in check_layers:
            got[r, l] = dict(
                h_in=to_np(th[l, sl]),
                h_out=to_np(th[l + 1, sl]) if l + 1 < L else to_np(hid[sl]),
                ids=to_np(tid[l, sl]),
                K=to_np(eng.kcache()[r, l, :, :P0 + C, :]),
                V=to_np(eng.vcache()[r, l, :, :, :P0 + C]).transpose(0, 2, 1))
    rl = R - 1
    z = eng.logits(R)[rl * C:(rl + 1) * C].cpu().numpy()
    hfinal = to_np(hid[rl * C:(rl + 1) * C])
    am = eng.argmax()[rl].cpu().numpy()
    lock = to_np(eng.view(B.CD_BUF_LOCK, torch.uint8, (R, C))[rl]).astype(bool)
    xn = eng.canvas()[rl].cpu().numpy()
    H = to_np(eng.view(B.CD_BUF_ENTROPY, torch.float64, (R, C))[rl])
    del th, tid, tg
    eng.close()

    # sampled canvas rows of two requests through the first and last layer
    pos = P0 + np.arange(C)
    rows = np.array([3, 200])
    adopted = 0
    for l in check_layers:
        W = Weights(w)
        for r in check_req:
            gl = got[r, l]
            h_out, kr, vr, ad = layer_rows(w, W, l, gl["h_in"], rows, gl["K"], gl["V"], pos, gl["ids"][rows], tol)
            adopted += ad
            gk = gl["K"][:, P0 + rows, :].transpose(1, 0, 2)
            gv = gl["V"][:, P0 + rows, :].transpose(1, 0, 2)
            assert rel_l2_rows(gk.reshape(len(rows), -1), kr.reshape(len(rows), -1)).max() <= tol, (r, l)
            assert rel_l2_rows(gv.reshape(len(rows), -1), vr.reshape(len(rows), -1)).max() <= tol, (r, l)
            assert rel_l2_rows(gl["h_out"][rows], h_out).max() <= tol, (r, l)
        del W
    print(f"routing decisions adopted from near-ties: {adopted}")

    # LM head (bf16) on sampled vocabulary rows of the last request
    W0 = Weights(w)
    vrows = np.sort(np.random.default_rng(1).choice(V, size=256, replace=False))
    zref = model.lm_head(w, W0, hfinal, vocab_rows=vrows)
    assert rel_l2_rows(z[:, vrows], zref).max() <= tol

    # sampler on the last request's own logits and Philox stream
    ref = osamp.sample(w, z, seed, 1, 0, rl)
    decided = ref["margin"] > 1e-3
    assert np.array_equal(am[decided], ref["a"][decided])
    ok = np.abs(ref["pmax"] - w["lock"]) > 1e-3
    assert np.array_equal(lock[ok], ref["lock"][ok])
    same = lock == ref["lock"]
    assert np.array_equal(xn[same & ~lock], ref["x_next"][same & ~lock])
    assert np.all(np.abs(H - ref["H"]) <= 1e-5 + 1e-5 * ref["H"])
    assert abs(infos[rl].mean_entropy - ref["Hbar"]) <= 1e-6 * ref["Hbar"]
