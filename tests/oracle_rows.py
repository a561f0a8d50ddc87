"""Oracle recomputation of single rows of a full-width forward, for the
sampled parity tests (test code composing oracle functions; the full-size
forward is too large for the oracle to run whole)."""
import numpy as np

from oracle import model


def layer_rows(w, W, l, h_in, rows, K_all, V_all, pos, gpu_ids, tol):
    """Oracle output of layer l for the given canvas rows, attending the GPU's
    keys/values of the whole context; returns (h_out rows, k rows, v rows,
    adopted routing decisions)."""
    Hq, Hkv, dh = w["Hq"], w["Hkv"], w["dh"]
    u = model.rmsnorm(h_in[rows], w["eps"])
    q = model.rope((u @ W.get("wq", l).T).reshape(len(rows), Hq, dh), pos[rows], w["theta"])
    k = model.rope((u @ W.get("wk", l).T).reshape(len(rows), Hkv, dh), pos[rows], w["theta"])
    v = (u @ W.get("wv", l).T).reshape(len(rows), Hkv, dh)
    o = model.attention(q, K_all, V_all).reshape(len(rows), Hq * dh)
    h = h_in[rows] + o @ W.get("wo", l).T
    u2 = model.rmsnorm(h, w["eps"])
    r = u2 @ W.get("wr", l).T
    own = np.argsort(-r, axis=1, kind="stable")[:, :w["k"]]
    kth = np.sort(r, axis=1)[:, ::-1][:, w["k"] - 1]
    rms = np.sqrt(np.mean(r ** 2, axis=1))
    adopted = 0
    for t in range(len(rows)):
        if set(gpu_ids[t]) != set(own[t]):
            assert np.all(r[t, gpu_ids[t]] >= kth[t] - tol * rms[t]), (l, rows[t])
            adopted += 1
    f, _, _, _ = model.moe(w, W, l, u2, forced_ids=gpu_ids)
    return h + f, k, v, adopted
