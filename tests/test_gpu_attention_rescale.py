"""The attention softmax takes each row's scores relative to a reference that
moves only when a score exceeds it by more than 2^attn_rescale_log2 (lazy
rescaling; O and the row sum always share the reference, so the result is the
softmax up to rounding).  These cases make the reference move:

* sharp scores: query and key weights of the tiny fp32 model scaled by 8
  (scores 64x larger, about 9 powers of two per standard deviation), default
  threshold; the test checks that in layer 0 some rows' second key block
  beats their first by more than 2^8, so the first key split must move its
  reference mid-row;
* the tiny fp32 model and the small bf16 model with a threshold of 2^-20:
  every growth of a row maximum rescales O.

Prefill (causal) K/V and one canvas pass (per-layer hidden states, logits)
are compared with the oracle.  Tolerances: bf16 2e-2 and fp32 1e-5 per-row
relative L2, except the sharp fp32 case: the softmax turns an absolute score
error e into a relative weight error e, and scores 64x larger carry 64x the
absolute fp32 rounding of the score products, so that case allows 64e-5."""
import numpy as np
import pytest
import torch

import synth_inputs
from block_text_diffusion_amd import binding as B
from block_text_diffusion_amd.engine import Engine
from oracle import loop, model
from oracle import weights as ow
from oracle.weights import Weights
from tests.gpu_util import TOL, announce, check_routing, rel_l2_rows, to_np

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


def _scale_qk(eng, W, w, s):
    for l in range(w["L"]):
        for kind, name in ((B.CD_W_Q, "wq"), (B.CD_W_K, "wk")):
            shape = ow.tensor_shape(w, name)
            x = eng.weight(kind, l, 0, shape)
            B.cd_set_weight(eng.ctx, kind, l, 0, (x * s).contiguous())
            W.set(name, W.get(name, l) * s, l)


def _layer0_jumps(w, W, h0, pos, K_prev):
    """Rows (query, head) of layer 0 whose largest scaled score over keys
    64..127 exceeds the one over keys 0..63 by more than 8 (base 2)."""
    dh, Hq, Hkv = w["dh"], w["Hq"], w["Hkv"]
    u = model.rmsnorm(h0, w["eps"])
    n = u.shape[0]
    q = model.rope((u @ W.get("wq", 0).T).reshape(n, Hq, dh), pos, w["theta"])
    k = model.rope((u @ W.get("wk", 0).T).reshape(n, Hkv, dh), pos, w["theta"])
    K = np.concatenate([K_prev, k.transpose(1, 0, 2)], axis=1)
    jumps = 0
    for h in range(Hq):
        sc = q[:, h, :] @ K[h // (Hq // Hkv)].T * (LOG2E / np.sqrt(dh))
        jumps += int(np.sum(sc[:, 64:128].max(axis=1) - sc[:, :64].max(axis=1) > 8.0))
    return jumps


def _prefill_and_pass(w, qk_scale, tol, want_jumps=False):
    L, C, k = w["L"], w["C"], w["k"]
    eng = Engine(w)
    B.cd_synth_weights(eng.ctx, w["weight_seed"])
    W = Weights(w)
    if qk_scale != 1:
        _scale_qk(eng, W, w, qk_scale)
    T = max(C, w["P0"])
    th = torch.zeros(L, T, w["d"], dtype=torch.float32, device="cuda")
    tid = torch.zeros(L, T, k, dtype=torch.int32, device="cuda")
    tg = torch.zeros(L, T, k, dtype=torch.float32, device="cuda")
    B.cd_set_trace(eng.ctx, th, tid, tg)

    def gpu_routing(n):
        torch.cuda.synchronize()
        flat = tid.view(-1)[: L * n * k].view(L, n, k)
        return [to_np(flat[i]) for i in range(L)]

    pre = synth_inputs.prefix_ids(w["V"], w["P0"], 5)
    B.cd_prefill(eng.ctx, 0, torch.from_numpy(pre).cuda())
    gid = gpu_routing(len(pre))
    req = loop.Request(w)
    tr = []
    _, kv, _ = model.forward(w, W, pre, np.arange(len(pre)), req.cache, causal=True, head=False, trace=tr,
                             forced_routing=gid)
    check_routing(gid, tr, k, tol)
    req.append(kv, pre)
    for l in range(L):
        Kg = to_np(eng.kcache()[0, l, :, : w["P0"], :])
        Vg = to_np(eng.vcache()[0, l, :, :, : w["P0"]]).transpose(0, 2, 1)
        Ko, Vo = req.cache[l][0], req.cache[l][1]
        assert rel_l2_rows(Kg.reshape(-1, w["dh"]), Ko.reshape(-1, w["dh"])).max() <= tol, ("K", l)
        assert rel_l2_rows(Vg.reshape(-1, w["dh"]), Vo.reshape(-1, w["dh"])).max() <= tol, ("V", l)

    seed = 31
    B.cd_init_canvas(eng.ctx, 0, seed, 0)
    x = loop.init_canvas(w, seed, 0, 0)
    B.cd_denoise_step(eng.ctx, 1, eng.info)
    gid = gpu_routing(C)
    tr = []
    ref = loop.denoise_pass(w, W, req, x, 1, 0, seed, trace=tr, forced_routing=gid)
    check_routing(gid, tr, k, tol)
    hs = th.view(-1)[: L * C * w["d"]].view(L, C, w["d"])   # the trace of an n-row forward is [L][n][d]
    errs = [rel_l2_rows(to_np(hs[l]), tr[l]["h_in"]).max() for l in range(L)]
    ez = rel_l2_rows(to_np(eng.logits()), ref["z"]).max()
    print(f"max rel err per layer {['%.2e' % e for e in errs]}, logits {ez:.2e}")
    assert max(errs) <= tol and ez <= tol, (errs, ez)
    if want_jumps:
        jumps = _layer0_jumps(w, W, tr[0]["h_in"], w["P0"] + np.arange(C), req.cache[0][0])
        print(f"layer-0 rows whose reference must move by more than 2^8: {jumps}")
        assert jumps > 0
    eng.close()


def test_sharp_scores_move_the_reference_fp32():
    w = synth_inputs.workload("tiny")
    announce("attn_rescale_sharp_f32", scale=8)
    _prefill_and_pass(w, 8.0, 64 * TOL["f32"], want_jumps=True)


def test_tiny_threshold_fp32():
    w = synth_inputs.workload("tiny", attn_rescale_log2=2.0 ** -20)
    announce("attn_rescale_tiny_threshold_f32")
    _prefill_and_pass(w, 1.0, TOL["f32"])


def test_tiny_threshold_bf16():
    w = synth_inputs.workload("tiny", wdtype="bf16", dh=128, Hq=4, Hkv=2, E=16, k=4, fe=256, fs=128, P0=100,
                              C=200, attn_rescale_log2=2.0 ** -20)
    announce("attn_rescale_tiny_threshold_bf16")
    _prefill_and_pass(w, 1.0, TOL["bf16"])
