"""End-to-end parity of the HIP path with the oracle on the tiny fp32 model
(2 layers, d=256, 4/2 heads, 8 experts top-2, vocab 4096, prefix 128): prefill
KV, canvas start, per-layer hidden states and routing, logits, sampler
decisions at every pass of the loop, the stop at the cap, and the commit.
Tolerance 1e-5 (per-row relative L2) for fp32."""
import numpy as np
import pytest
import torch

import synth_inputs
from block_text_diffusion_amd import binding as B
from block_text_diffusion_amd.engine import Engine
from oracle import loop, model
from oracle.weights import Weights
from tests.gpu_util import announce, rel_l2_rows, to_np

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _kv(eng, l, P0, P1):
    K = to_np(eng.kcache()[0, l, :, P0:P1, :])                       # [Hkv][n][dh]
    V = to_np(eng.vcache()[0, l, :, :, P0:P1]).transpose(0, 2, 1)    # [Hkv][n][dh]
    return K, V


def _cmp_kv(eng, req_o, w, P0, P1, tol):
    for l in range(w["L"]):
        K, V = _kv(eng, l, P0, P1)
        Ko, Vo = req_o.cache[l][0][:, P0:P1], req_o.cache[l][1][:, P0:P1]
        assert rel_l2_rows(K.reshape(-1, w["dh"]), Ko.reshape(-1, w["dh"])).max() <= tol, l
        assert rel_l2_rows(V.reshape(-1, w["dh"]), Vo.reshape(-1, w["dh"])).max() <= tol, l


def _route_checks(tr_ids, ref_tr, w, tol):
    for l in range(w["L"]):
        r = ref_tr[l]["router"]
        srt = np.sort(r, axis=1)[:, ::-1]
        gap = srt[:, w["k"] - 1] - srt[:, w["k"]]
        rms = np.sqrt(np.mean(r ** 2, axis=1))
        decided = gap > tol * 10 * rms
        got = np.sort(tr_ids[l], axis=1)
        want = np.sort(ref_tr[l]["ids"], axis=1)
        assert np.array_equal(got[decided], want[decided]), l
        assert decided.mean() > 0.9


def test_tiny_prefill_loop_commit_matches_oracle():
    w = synth_inputs.workload("tiny")
    announce("tiny_e2e", **{k: w[k] for k in ("L", "d", "E", "V", "P0")})
    L, d, k, C = w["L"], w["d"], w["k"], w["C"]
    eng = Engine(w)
    B.cd_synth_weights(eng.ctx, w["weight_seed"])
    prefix = synth_inputs.prefix_ids(w["V"], w["P0"], w["prefix_seed"])
    B.cd_prefill(eng.ctx, 0, torch.from_numpy(prefix).cuda())
    W = Weights(w)
    req = loop.Request(w)
    loop.prefill(w, W, req, prefix)
    torch.cuda.synchronize()
    _cmp_kv(eng, req, w, 0, w["P0"], TOL)
    kv_prefix = [tuple(x.copy() for x in _kv(eng, l, 0, w["P0"])) for l in range(L)]

    seed = w["gen_seed"]
    B.cd_init_canvas(eng.ctx, 0, seed, 0)
    x = loop.init_canvas(w, seed, 0, 0)
    assert np.array_equal(eng.canvas()[0].cpu().numpy(), x)

    th = torch.zeros(L, C, d, dtype=torch.float32, device="cuda")
    tid = torch.zeros(L, C, k, dtype=torch.int32, device="cuda")
    tg = torch.zeros(L, C, k, dtype=torch.float32, device="cuda")
    B.cd_set_trace(eng.ctx, th, tid, tg)
    a_prev = None
    for t in range(1, w["max_steps"] + 1):
        tr = [] if t == 1 else None
        ref = loop.denoise_pass(w, W, req, x, t, 0, seed, trace=tr)
        B.cd_denoise_step(eng.ctx, 1, eng.info)
        info = eng.step_info()[0]
        z = to_np(eng.logits())
        assert rel_l2_rows(z, ref["z"]).max() <= TOL, t
        if t == 1:
            for l in range(L):
                assert rel_l2_rows(to_np(th[l]), tr[l]["h_in"]).max() <= TOL, l
            _route_checks(to_np(tid), tr, w, TOL)
            B.cd_set_trace(eng.ctx)
        a = eng.argmax()[0].cpu().numpy()
        decided = ref["margin"] > 1e-3
        assert np.array_equal(a[decided], ref["a"][decided])
        srt = np.sort(ref["z"], axis=1)
        assert np.array_equal(a[srt[:, -1] - srt[:, -2] > 1e-4], ref["a"][srt[:, -1] - srt[:, -2] > 1e-4])
        assert info.n_locked == 0 and not ref["lock"].any()
        assert info.step == t
        assert abs(info.mean_entropy - ref["Hbar"]) <= 1e-6 * ref["Hbar"]
        stop = ref["Hbar"] < w["stop_H"] and a_prev is not None and np.array_equal(ref["a"], a_prev)
        assert info.stop == int(stop or t == w["max_steps"])
        x_gpu = eng.canvas()[0].cpu().numpy()
        assert np.array_equal(x_gpu, ref["x_next"])          # all re-noised: pure Philox
        a_prev = ref["a"]
        x = x_gpu
        if info.stop:
            break
    assert t == 48

    out = torch.empty(C, dtype=torch.int32, device="cuda")
    B.cd_commit_block(eng.ctx, 0, out)
    committed = out.cpu().numpy()
    assert np.array_equal(committed, eng.argmax()[0].cpu().numpy())
    loop.commit(w, W, req, committed.astype(np.int64))       # the oracle adopts the GPU's ids
    torch.cuda.synchronize()
    assert B.cd_get_length(eng.ctx, 0) == w["P0"] + C
    _cmp_kv(eng, req, w, w["P0"], w["P0"] + C, TOL)
    for l in range(L):
        Kp, Vp = _kv(eng, l, 0, w["P0"])
        assert np.array_equal(Kp, kv_prefix[l][0]) and np.array_equal(Vp, kv_prefix[l][1])
    eng.close()


def _copy_model_gpu(eng, w, s):
    d, fe, qd = w["d"], w["fe"], w["Hq"] * w["dh"]
    for l in range(w["L"]):
        B.cd_set_weight(eng.ctx, B.CD_W_O, l, 0, torch.zeros(d, qd, device="cuda"))
        for e in range(w["E"]):
            B.cd_set_weight(eng.ctx, B.CD_W_DOWN, l, e, torch.zeros(d, fe, device="cuda"))
    E = eng.weight(B.CD_W_EMBED, 0, 0, (w["V"], d))
    B.cd_set_weight(eng.ctx, B.CD_W_LM, 0, 0, E * s)


def _copy_model_oracle(w, s):
    W = Weights(w)
    for l in range(w["L"]):
        W.set("wo", np.zeros_like(W.get("wo", l)), l)
        for e in range(w["E"]):
            W.set("wd", np.zeros_like(W.get("wd", l, e)), l, e)
    W.set("lm", s * W.get("embed"))
    return W


def test_tiny_copy_model_stops_at_pass_two_via_generate():
    w = synth_inputs.workload("tiny")
    announce("tiny_copy_model_generate")
    eng = Engine(w)
    B.cd_synth_weights(eng.ctx, w["weight_seed"])
    _copy_model_gpu(eng, w, 8.0)
    prefix = torch.from_numpy(synth_inputs.prefix_ids(w["V"], w["P0"], w["prefix_seed"])).cuda()
    out = torch.empty(w["C"], dtype=torch.int32, device="cuda")
    steps = B.cd_generate(eng.ctx, 0, prefix, 1, w["gen_seed"], out)
    assert steps == [2]
    assert np.array_equal(out.cpu().numpy(), loop.init_canvas(w, w["gen_seed"], 0, 0))
    assert B.cd_get_length(eng.ctx, 0) == w["P0"] + w["C"]
    eng.close()


@pytest.mark.parametrize("rule,s", [("maxprob", 2.1), ("entropy", 2.65)])
def test_tiny_mixed_lock_decisions_match_oracle(rule, s):
    # copy-model scales chosen so that about half the positions lock at
    # pass 1 under each rule (max prob > 0.9, or entropy <= 0.1 nats)
    w = synth_inputs.workload("tiny", lock_rule=rule, entropy_bound=0.1)
    announce("tiny_mixed_lock", rule=rule, s=s)
    eng = Engine(w)
    B.cd_synth_weights(eng.ctx, w["weight_seed"])
    _copy_model_gpu(eng, w, s)
    W = _copy_model_oracle(w, s)
    prefix = synth_inputs.prefix_ids(w["V"], w["P0"], w["prefix_seed"])
    B.cd_prefill(eng.ctx, 0, torch.from_numpy(prefix).cuda())
    req = loop.Request(w)
    loop.prefill(w, W, req, prefix)
    seed = w["gen_seed"]
    B.cd_init_canvas(eng.ctx, 0, seed, 0)
    x = loop.init_canvas(w, seed, 0, 0)
    for t in (1, 2, 3):
        ref = loop.denoise_pass(w, W, req, x, t, 0, seed)
        B.cd_denoise_step(eng.ctx, 1, eng.info)
        info = eng.step_info()[0]
        assert rel_l2_rows(to_np(eng.logits()), ref["z"]).max() <= TOL
        lock = to_np(eng.view(B.CD_BUF_LOCK, torch.uint8, (1, w["C"]))[0]).astype(bool)
        ok = (np.abs(ref["pmax"] - w["lock"]) > 1e-3 if rule == "maxprob"
              else np.abs(ref["H"] - w["entropy_bound"]) > 1e-3)
        assert np.array_equal(lock[ok], ref["lock"][ok])
        if t == 1:
            assert 20 < ref["lock"].sum() < 236
        same = lock == ref["lock"]
        xg = eng.canvas()[0].cpu().numpy()
        assert np.array_equal(xg[same], ref["x_next"][same])
        assert info.n_locked == int(lock.sum())
        x = xg                                   # lockstep: the oracle follows the GPU canvas
    eng.close()
