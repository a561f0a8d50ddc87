"""Parity at the realistic width (30 layers, d=2816, 128 experts top-8 plus a
shared FFN, vocabulary 262144, bf16, 4096-token prefix), in the launch
configuration bench.py times.  The oracle cannot run the whole step in a
test, so it checks what it can compute row by row, at every layer:

* the canvas start ids (bit-exact Philox);
* the causal prefill, layer by layer, at 8 prompt positions spread over the
  prompt: from the GPU's traced input of layer l and the GPU's K/V cache, the
  oracle recomputes those rows' keys/values and the layer output (causal
  attention over the cache) and compares them with the cache and the GPU's
  input of layer l+1 (the prefill's final residual after the last layer);
* one denoise pass, layer by layer, at 16 canvas rows (two in every 32-row
  tile, both 128-row halves): the rows' keys/values in the cache and the
  layer output (attention over the whole cache, no mask);
* routing: the GPU's top-k set equals the oracle's own, or lies within the
  near-tie band (then the oracle follows it); at most 4% of the checked
  decisions may be such adoptions;
* the LM head on 512 sampled vocabulary rows from the GPU's final residual;
* the sampler on the GPU's own logits (all 256 x 262144).
The same step with MXFP4 experts and fp8 attention (``step_mxfp4``) is
checked the same way.  Tolerance: bf16 2e-2, MXFP4 6e-2 (per-row relative
L2).  Its 4096-row prefill runs the QKV projection W8A8 and the MXFP4
experts on the block-scaled fp4 x fp8 MFMA (activation rows quantised to
E4M3, reading R18), which the oracle does not emulate, so the
prompt rows are also taken along the GPU's arithmetic (check_layer_w8a8):
keys and values within 6e-3 at every layer, the layer output within 2e-2 at
the first and last layer.  The largest errors are printed as one "[parity]"
line."""
import numpy as np
import pytest
import torch

import synth_inputs
from block_text_diffusion_amd import binding as B
from block_text_diffusion_amd.engine import Engine
from oracle import model, philox
from oracle.weights import Weights
from tests.gpu_util import TOL, announce, rel_l2_rows, to_np
from tests.oracle_rows import Summary, check_layer, check_layer_w8a8, sample_threaded

pytestmark = pytest.mark.gpu

# largest share of checked routing decisions the GPU may take from the
# near-tie band (its top-k set differs from the oracle's own)
ADOPT_CAP = {"f32": 0.01, "bf16": 0.04, "fp8": 0.04, "mxfp4": 0.04}
# the GPU arithmetic modelled in the test (check_layer_w8a8): what is left is
# the bf16 rounding of the outputs and fp32 accumulation
W8A8_TOL_KV, W8A8_TOL_H = 6e-3, 2e-2
# the MoE block modelled from the GPU's own input rows (the traced residual
# after the attention block): per row within 3e-2 (a few E4M3 steps of
# single elements of the down projection's input, moved by fp32 rounding
# upstream), median over the checked rows within 2e-3 (the bf16 rounding of
# the expert outputs and fp32 summation order)
W8A8_TOL_MOE, W8A8_MOE_MEDIAN = 3e-2, 2e-3
CANVAS_ROWS = np.array([2, 29, 35, 60, 66, 93, 101, 126, 130, 157, 163, 190, 197, 222, 229, 254])
PREFILL_POS = np.array([0, 1, 777, 2047, 2048, 3001, 4094, 4095])


def check_sampler(w, z, am, lock, xn, H, Hbar, seed, step, block, req):
    ref = sample_threaded(w, z, seed, step, block, req)
    decided = ref["margin"] > 1e-3
    assert np.array_equal(am[decided], ref["a"][decided])
    ok = np.abs(ref["pmax"] - w["lock"]) > 1e-3
    assert np.array_equal(lock[ok], ref["lock"][ok])
    same = lock == ref["lock"]
    assert np.array_equal(xn[same & ~lock], ref["x_next"][same & ~lock])
    assert np.all(np.abs(H - ref["H"]) <= 1e-5 + 1e-5 * ref["H"])
    assert abs(Hbar - ref["Hbar"]) <= 1e-6 * ref["Hbar"]
    return ref


@pytest.mark.parametrize("name", ["step_bf16", "step_mxfp4"])
def test_step_full_width_every_layer(name):
    w = synth_inputs.workload(name)
    tol = TOL[w["wdtype"]]
    announce("full_width_step", workload=name, L=w["L"], d=w["d"], E=w["E"], V=w["V"], P0=w["P0"])
    L, C, d, k, P0, V = w["L"], w["C"], w["d"], w["k"], w["P0"], w["V"]
    eng = Engine(w, max_ctx=P0 + C)
    B.cd_synth_weights(eng.ctx, w["weight_seed"])
    prefix = synth_inputs.prefix_ids(V, P0, w["prefix_seed"])
    th = torch.zeros(L * P0 * d, dtype=torch.float32, device="cuda")
    thm = torch.zeros(L * P0 * d, dtype=torch.float32, device="cuda")
    tid = torch.zeros(L * P0 * k, dtype=torch.int32, device="cuda")
    tg = torch.zeros(L * P0 * k, dtype=torch.float32, device="cuda")
    B.cd_set_trace(eng.ctx, th, tid, tg, thm)
    B.cd_prefill(eng.ctx, 0, torch.from_numpy(prefix).cuda())
    torch.cuda.synchronize()
    pp = torch.from_numpy(PREFILL_POS).cuda()
    p_h = to_np(th.view(L, P0, d)[:, pp])
    p_hm = to_np(thm.view(L, P0, d)[:, pp])
    p_ids = to_np(tid.view(L, P0, k)[:, pp])
    p_fin = to_np(eng.view(B.CD_BUF_HIDDEN, torch.float32, (P0, d))[pp])
    seed = w["gen_seed"]
    B.cd_init_canvas(eng.ctx, 0, seed, 0)
    x = eng.canvas()[0].cpu().numpy()
    assert np.array_equal(x, philox.token_draw(seed, np.arange(C), 0, 0, 0, V))
    B.cd_denoise_step(eng.ctx, 1, eng.info)
    info = eng.step_info()[0]
    B.cd_set_trace(eng.ctx)
    assert info.step == 1 and info.stop == 0
    cr = torch.from_numpy(CANVAS_ROWS).cuda()
    c_h = to_np(th[:L * C * d].view(L, C, d)[:, cr])
    c_ids = to_np(tid[:L * C * k].view(L, C, k)[:, cr])
    hfinal = to_np(eng.view(B.CD_BUF_HIDDEN, torch.float32, (C, d)))
    Kc = eng.kcache()[0, :, :, :P0 + C, :].cpu()
    Vc = eng.vcache()[0, :, :, :, :P0 + C].cpu()
    z = eng.logits().cpu().numpy()
    am = eng.argmax()[0].cpu().numpy()
    lock = to_np(eng.view(B.CD_BUF_LOCK, torch.uint8, (1, C))[0]).astype(bool)
    xn = eng.canvas()[0].cpu().numpy()
    H = to_np(eng.view(B.CD_BUF_ENTROPY, torch.float64, (1, C))[0])
    del th, tid, tg
    eng.close()
    del eng

    S = Summary(name)
    cpos = P0 + CANVAS_ROWS
    moe_rows = []
    for l in range(L):
        K = Kc[l].float().numpy().astype(np.float64)                     # [Hkv][P0+C][dh]
        Vv = Vc[l].float().numpy().astype(np.float64).transpose(0, 2, 1)
        items = [
            dict(name="canvas", h_in=c_h[l], h_out=c_h[l + 1] if l + 1 < L else hfinal[CANVAS_ROWS], pos=cpos,
                 K=K, V=Vv, causal=False, ids=c_ids[l], k_got=K[:, cpos].transpose(1, 0, 2),
                 v_got=Vv[:, cpos].transpose(1, 0, 2)),
            dict(name="prefill", h_in=p_h[l], h_out=p_h[l + 1] if l + 1 < L else p_fin, h_mid=p_hm[l],
                 pos=PREFILL_POS,
                 K=K[:, :P0], V=Vv[:, :P0], causal=True, ids=p_ids[l],
                 k_got=K[:, PREFILL_POS].transpose(1, 0, 2), v_got=Vv[:, PREFILL_POS].transpose(1, 0, 2)),
        ]
        res = check_layer(w, l, items, tol)
        S.add_layer(res[:1], "canvas_")
        S.add_layer(res[1:], "prefill_")
        m8 = {}
        if w["wdtype"] in ("fp8", "mxfp4"):
            # the 4096-row prefill runs the QKV GEMM of the fp8 attention weights
            # W8A8 and the routed experts on E4M3 activations (fp8 or MXFP4
            # weights): its rows along the GPU's arithmetic
            m8 = check_layer_w8a8(w, l, items[1:], W8A8_TOL_KV, W8A8_TOL_H if l in (0, L - 1) else None,
                                  experts=True, tol_moe=W8A8_TOL_MOE)
            moe_rows.append(m8.pop("moe_rows", np.zeros(0)))
            for key, val in m8.items():
                S.add("prefill_" + key, val)
        print(f"layer {l}: {[{k2: float(f'{v:.2e}') for k2, v in r.items()} for r in res]} "
              f"w8a8 model: {({k2: float(f'{v:.2e}') for k2, v in m8.items()})}", flush=True)

    # LM head on sampled vocabulary rows
    vrows = np.sort(np.random.default_rng(0).choice(V, size=512, replace=False))
    zref = model.lm_head(w, Weights(w, cache=False), hfinal, vocab_rows=vrows)
    S.add("lm_head", rel_l2_rows(z[:, vrows], zref).max())
    assert S.err["lm_head"] <= tol
    check_sampler(w, z, am, lock, xn, H, info.mean_entropy, seed, 1, 0, 0)
    if moe_rows:
        med = float(np.median(np.concatenate(moe_rows)))
        S.add("prefill_moe8_median", med)
        assert med <= W8A8_MOE_MEDIAN, ("w8a8 moe median", med)
    S.report(ADOPT_CAP[w["wdtype"]])
