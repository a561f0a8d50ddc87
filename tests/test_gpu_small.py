"""End-to-end parity on small bf16 / fp8 / MXFP4-expert models that use every kernel path of
the realistic-width step (head_dim 128, grouped-query pairs, top-k routing
over 16 experts, a shared FFN, bf16 activations) with ragged sizes: a
100-token prefix, a second request with a 37-token prefix denoised in the
same pass, a 200-token canvas.  Tolerances: bf16 2e-2, fp8 and MXFP4 6e-2 (per-row
relative L2 of hidden states, K/V and logits)."""
import numpy as np
import pytest
import torch

import synth_inputs
from block_text_diffusion_amd import binding as B
from block_text_diffusion_amd.engine import Engine
from oracle import loop
from oracle.weights import Weights
from tests.gpu_util import TOL, announce, check_routing, rel_l2_rows, to_np

pytestmark = pytest.mark.gpu


def small(wdtype, **kw):
    base = dict(wdtype=wdtype, dh=128, Hq=4, Hkv=2, E=16, k=4, fe=256, fs=128, V=4096, P0=100)
    base.update(kw)
    return synth_inputs.workload("tiny", **base)


def _cmp_kv(eng, req_o, w, r, P0, P1, tol):
    for l in range(w["L"]):
        K = to_np(eng.kcache()[r, l, :, P0:P1, :])
        V = to_np(eng.vcache()[r, l, :, :, P0:P1]).transpose(0, 2, 1)
        Ko, Vo = req_o.cache[l][0][:, P0:P1], req_o.cache[l][1][:, P0:P1]
        assert rel_l2_rows(K.reshape(-1, w["dh"]), Ko.reshape(-1, w["dh"])).max() <= tol, ("K", l)
        assert rel_l2_rows(V.reshape(-1, w["dh"]), Vo.reshape(-1, w["dh"])).max() <= tol, ("V", l)


@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "mxfp4"])
def test_small_two_requests_step_and_commit(wdtype):
    w = small(wdtype, C=200)
    tol = TOL[wdtype]
    announce("small_e2e", wdtype=wdtype, C=w["C"])
    C, L, k = w["C"], w["L"], w["k"]
    eng = Engine(w, max_requests=2, max_ctx=w["P0"] + 2 * C, max_prefill=w["P0"])
    B.cd_synth_weights(eng.ctx, w["weight_seed"])
    W = Weights(w)
    rows = 2 * C
    th = torch.zeros(L, rows, w["d"], dtype=torch.float32, device="cuda")
    tid = torch.zeros(L, rows, k, dtype=torch.int32, device="cuda")
    tg = torch.zeros(L, rows, k, dtype=torch.float32, device="cuda")
    B.cd_set_trace(eng.ctx, th, tid, tg)

    def gpu_routing(n):
        # the trace of a forward over n rows is packed as [L][n][k]
        torch.cuda.synchronize()
        flat = tid.view(-1)[: L * n * k].view(L, n, k)
        return [to_np(flat[l]) for l in range(L)]

    prefixes = [synth_inputs.prefix_ids(w["V"], w["P0"], 7, 0), synth_inputs.prefix_ids(w["V"], 37, 7, 1)]
    reqs = []
    adopted = 0
    for r, pre in enumerate(prefixes):
        B.cd_prefill(eng.ctx, r, torch.from_numpy(pre).cuda())
        gid = gpu_routing(len(pre))
        ro = loop.Request(w, r)
        tr = []
        pos = np.arange(len(pre))
        from oracle import model
        _, kv, _ = model.forward(w, W, pre, pos, ro.cache, causal=True, head=False, trace=tr, forced_routing=gid)
        adopted += check_routing(gid, tr, k, tol)
        ro.append(kv, pre)
        reqs.append(ro)
    for r, pre in enumerate(prefixes):
        _cmp_kv(eng, reqs[r], w, r, 0, len(pre), tol)
    seed = 99
    xs = []
    for r in range(2):
        B.cd_init_canvas(eng.ctx, r, seed, 0)
        xs.append(loop.init_canvas(w, seed, 0, r))
    for t in (1, 2):
        B.cd_denoise_step(eng.ctx, 2, eng.info)
        infos = eng.step_info(2)
        z = to_np(eng.logits(2))
        gid_all = gpu_routing(rows)
        hs = [to_np(th[l]) for l in range(L)]
        for r in range(2):
            tr = []
            gid = [g[r * C:(r + 1) * C] for g in gid_all]
            ref = loop.denoise_pass(w, W, reqs[r], xs[r], t, 0, seed, trace=tr, forced_routing=gid)
            adopted += check_routing(gid, tr, k, tol)
            zr = z[r * C:(r + 1) * C]
            assert rel_l2_rows(zr, ref["z"]).max() <= tol, (r, t)
            for l in range(L):
                assert rel_l2_rows(hs[l][r * C:(r + 1) * C], tr[l]["h_in"]).max() <= tol, (r, l)
            assert infos[r].step == t and infos[r].n_locked == 0
            assert abs(infos[r].mean_entropy - ref["Hbar"]) <= 1e-3 * ref["Hbar"]
            xg = eng.canvas()[r].cpu().numpy()
            assert np.array_equal(xg, ref["x_next"])
            xs[r] = xg
    for r in range(2):
        out = torch.empty(C, dtype=torch.int32, device="cuda")
        P_before = B.cd_get_length(eng.ctx, r)
        B.cd_commit_block(eng.ctx, r, out)
        gid = gpu_routing(C)
        ids = out.cpu().numpy().astype(np.int64)
        tr = []
        pos = P_before + np.arange(C)
        from oracle import model
        _, kv, _ = model.forward(w, W, ids, pos, reqs[r].cache, causal=False, head=False, trace=tr,
                                 forced_routing=gid)
        adopted += check_routing(gid, tr, k, tol)
        reqs[r].append(kv, ids)
        assert B.cd_get_length(eng.ctx, r) == P_before + C
        _cmp_kv(eng, reqs[r], w, r, P_before, P_before + C, tol)
    print(f"routing decisions adopted from near-ties: {adopted}")
    eng.close()


def test_small_f32_generate_two_blocks_conditions_on_history():
    # fp32 keeps router and argmax decisions clear of rounding, so the whole
    # two-block generation can be compared without lockstep adoption
    w = small("f32", max_steps=3)
    announce("small_generate_two_blocks_f32")
    C = w["C"]
    eng = Engine(w, max_ctx=w["P0"] + 2 * C)
    B.cd_synth_weights(eng.ctx, w["weight_seed"])
    pre = synth_inputs.prefix_ids(w["V"], w["P0"], 3)
    out = torch.empty(2 * C, dtype=torch.int32, device="cuda")
    steps = B.cd_generate(eng.ctx, 0, torch.from_numpy(pre).cuda(), 2, 5, out)
    assert steps == [3, 3]
    assert B.cd_get_length(eng.ctx, 0) == w["P0"] + 2 * C
    W = Weights(w)
    req = loop.Request(w)
    loop.prefill(w, W, req, pre)
    got = out.cpu().numpy()
    for b in range(2):
        x = loop.init_canvas(w, 5, b, 0)
        for t in (1, 2, 3):
            ref = loop.denoise_pass(w, W, req, x, t, b, 5)
            x = ref["x_next"]
        srt = np.sort(ref["z"], axis=1)
        clear = srt[:, -1] - srt[:, -2] > 1e-4
        assert clear.mean() > 0.9
        assert np.array_equal(got[b * C:(b + 1) * C][clear], ref["a"][clear])
        loop.commit(w, W, req, got[b * C:(b + 1) * C].astype(np.int64))
    _cmp_kv(eng, req, w, 0, 0, w["P0"] + 2 * C, TOL["f32"])
    eng.close()
