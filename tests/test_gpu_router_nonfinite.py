"""Non-finite router logits (tiny fp32 model: 2 layers, 8 experts top-2).

A NaN router logit must neither pick an expert id outside [0, E) nor pick one
expert twice for a token (either would send rows to a wrong or duplicated
expert tile), and it must not vanish: the row's gates turn NaN, the logits
follow, and the loop reports CD_ERR_NUMERIC.  Layer 0's router gets NaN
weight rows for experts 0..3 (those logits are NaN for every token, the other
four stay finite); layer 1 then sees NaN hidden rows, so all of its logits are
NaN.  Expected: layer 0 picks two distinct experts among 4..7, layer 1 the
two lowest ids (NaN ranks as -inf, ties go to the lower id), every traced gate
is NaN, and cd_generate fails with CD_ERR_NUMERIC."""
import numpy as np
import pytest
import torch

import synth_inputs
from block_text_diffusion_amd import binding as B
from block_text_diffusion_amd.engine import Engine
from tests.gpu_util import announce, to_np

pytestmark = pytest.mark.gpu


def test_nan_router_logits_keep_ids_valid_and_fail_loudly():
    w = synth_inputs.workload("tiny")
    L, d, E, k, C = w["L"], w["d"], w["E"], w["k"], w["C"]
    announce("router_nonfinite", L=L, E=E, k=k)
    eng = Engine(w)
    B.cd_synth_weights(eng.ctx, w["weight_seed"])
    router = torch.empty(E, d, dtype=torch.float32, device="cuda")
    B.cd_get_weight(eng.ctx, B.CD_W_ROUTER, 0, 0, router)
    router[: E // 2] = float("nan")
    B.cd_set_weight(eng.ctx, B.CD_W_ROUTER, 0, 0, router)

    tid = torch.full((L, C, k), -1, dtype=torch.int32, device="cuda")
    tg = torch.zeros(L, C, k, dtype=torch.float32, device="cuda")
    B.cd_set_trace(eng.ctx, None, tid, tg)
    prefix = torch.from_numpy(synth_inputs.prefix_ids(w["V"], w["P0"], w["prefix_seed"])).cuda()
    out = torch.empty(C, dtype=torch.int32, device="cuda")
    with pytest.raises(B.CDError) as e:
        B.cd_generate(eng.ctx, 0, prefix, 1, w["gen_seed"], out)
    assert e.value.code == B.CD_ERR_NUMERIC
    torch.cuda.synchronize()
    B.cd_set_trace(eng.ctx)

    # the trace holds the last forward: the first canvas pass over C rows
    ids, gates = to_np(tid), to_np(tg)
    assert ((ids >= 0) & (ids < E)).all()
    for l in range(L):
        s = np.sort(ids[l], axis=1)
        assert (s[:, 1:] != s[:, :-1]).all(), l               # k distinct experts per token
    assert (ids[0] >= E // 2).all()                            # only the finite logits win
    assert (np.sort(ids[1], axis=1) == np.arange(k)).all()     # all NaN: lowest ids
    assert np.isnan(gates).all()
    eng.close()
