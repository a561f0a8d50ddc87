"""Parity of the 32-request fp8 batch at the realistic width (30 layers,
d=2816, 128 experts top-8 plus a shared FFN, vocabulary 262144, fp8 e4m3
attention and expert weights with per-row bf16 scales, 4096-token prefix per
request), one denoise pass over all 32 canvases in the launch configuration
bench.py times.  The oracle checks what it can compute row by row:

* the canvas start ids of three requests (bit-exact Philox, request index
  in the counter);
* for the first and the last request, 16 canvas rows each (two in every
  32-row tile of the request's canvas) at every layer, from the GPU's own
  layer inputs and K/V cache: the rows' keys/values and the layer output,
  following the GPU's routing under the near-tie rule (at most 4% adopted);
* the LM head on sampled vocabulary rows of the last request;
* the sampler on the last request's GPU logits (its own Philox stream).
The same batch with MXFP4 experts (``batch_mxfp4``: 512 rows per expert, so
the expert GEMMs run MXFP4 weights on the block-scaled fp4 x fp8 MFMA at
K = 2816 and 704) is checked the same way.  Tolerance: fp8 and MXFP4 6e-2
(per-row relative L2).  At this batch the QKV projection and the routed
experts quantise their activation rows to E4M3 (reading R18), which the
oracle does not emulate; the same rows are therefore also taken along the
GPU's arithmetic (bf16 activation rows, the per-row E4M3 quantiser, bf16
intermediate rows, tests/oracle_rows.check_layer_w8a8): keys and values at
every layer within 6e-3, the layer output at the first and last layer within
2e-2.  The largest errors are printed as one "[parity]" line."""
import numpy as np
import pytest
import torch

import synth_inputs
from block_text_diffusion_amd import binding as B
from block_text_diffusion_amd.engine import Engine
from oracle import model, philox
from oracle.weights import Weights
from tests.gpu_util import TOL, announce, rel_l2_rows, to_np
from tests.oracle_rows import Summary, check_layer, check_layer_w8a8
from tests.test_gpu_full_width import (ADOPT_CAP, CANVAS_ROWS, W8A8_MOE_MEDIAN, W8A8_TOL_H, W8A8_TOL_KV,
                                       W8A8_TOL_MOE, check_sampler)

pytestmark = pytest.mark.gpu

ROWS = {0: CANVAS_ROWS, 31: np.array([0, 31, 33, 62, 64, 95, 97, 127, 128, 159, 161, 191, 192, 223, 224, 255])}


@pytest.mark.parametrize("name", ["batch_fp8", "batch_mxfp4"])
def test_batch_full_width_every_layer(name):
    w = synth_inputs.workload(name)
    tol = TOL[w["wdtype"]]
    L, C, d, k, P0, V, R = w["L"], w["C"], w["d"], w["k"], w["P0"], w["V"], w["R"]
    assert R == 32
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
    thm = torch.zeros(L, T, d, dtype=torch.float32, device="cuda")
    tid = torch.zeros(L, T, k, dtype=torch.int32, device="cuda")
    tg = torch.zeros(L, T, k, dtype=torch.float32, device="cuda")
    B.cd_set_trace(eng.ctx, th, tid, tg, thm)
    B.cd_denoise_step(eng.ctx, R, eng.info)
    infos = eng.step_info(R)
    B.cd_set_trace(eng.ctx)
    assert all(i.step == 1 and i.stop == 0 and i.nonfinite == 0 for i in infos)

    hid = eng.view(B.CD_BUF_HIDDEN, torch.float32, (T, d))
    got = {}
    for r, rows in ROWS.items():
        gr = torch.from_numpy(r * C + rows).cuda()
        got[r] = dict(h=to_np(th[:, gr]), hm=to_np(thm[:, gr]), fin=to_np(hid[gr]), ids=to_np(tid[:, gr]),
                      K=eng.kcache()[r, :, :, :P0 + C, :].cpu(), V=eng.vcache()[r, :, :, :, :P0 + C].cpu())
    rl = R - 1
    z = eng.logits(R)[rl * C:(rl + 1) * C].cpu().numpy()
    hfinal = to_np(hid[rl * C:(rl + 1) * C])
    am = eng.argmax()[rl].cpu().numpy()
    lock = to_np(eng.view(B.CD_BUF_LOCK, torch.uint8, (R, C))[rl]).astype(bool)
    xn = eng.canvas()[rl].cpu().numpy()
    H = to_np(eng.view(B.CD_BUF_ENTROPY, torch.float64, (R, C))[rl])
    del th, thm, tid, tg, hid
    eng.close()
    del eng

    S = Summary(name)
    moe_rows = []
    for l in range(L):
        items = []
        for r, rows in ROWS.items():
            g = got[r]
            K = g["K"][l].float().numpy().astype(np.float64)
            Vv = g["V"][l].float().numpy().astype(np.float64).transpose(0, 2, 1)
            pos = P0 + rows
            items.append(dict(name=f"req{r}", h_in=g["h"][l], h_out=g["h"][l + 1] if l + 1 < L else g["fin"],
                              h_mid=g["hm"][l], pos=pos, K=K, V=Vv, causal=False, ids=g["ids"][l],
                              k_got=K[:, pos].transpose(1, 0, 2), v_got=Vv[:, pos].transpose(1, 0, 2)))
        res = check_layer(w, l, items, tol)
        S.add_layer(res)
        # the QKV GEMM (fp8 attention weights) runs W8A8 at 8192 rows, and the
        # routed experts (fp8 or MXFP4 weights) on E4M3 activations: the same
        # rows along the GPU's arithmetic
        m8 = check_layer_w8a8(w, l, items, W8A8_TOL_KV, W8A8_TOL_H if l in (0, L - 1) else None,
                              experts=True, tol_moe=W8A8_TOL_MOE)
        moe_rows.append(m8.pop("moe_rows", np.zeros(0)))
        for key, val in m8.items():
            S.add(key, val)
        print(f"layer {l}: {[{k2: float(f'{v:.2e}') for k2, v in r_.items()} for r_ in res]} "
              f"w8a8 model: {({k2: float(f'{v:.2e}') for k2, v in m8.items()})}", flush=True)

    # LM head (bf16) on sampled vocabulary rows of the last request
    vrows = np.sort(np.random.default_rng(1).choice(V, size=256, replace=False))
    zref = model.lm_head(w, Weights(w, cache=False), hfinal, vocab_rows=vrows)
    S.add("lm_head", rel_l2_rows(z[:, vrows], zref).max())
    assert S.err["lm_head"] <= tol
    check_sampler(w, z, am, lock, xn, H, infos[rl].mean_entropy, seed, 1, 0, rl)
    med = float(np.median(np.concatenate(moe_rows)))
    S.add("moe8_median", med)
    assert med <= W8A8_MOE_MEDIAN, ("w8a8 moe median", med)
    S.report(ADOPT_CAP[w["wdtype"]])
