"""Oracle recomputation of single rows of a full-width forward, for the
sampled parity tests (test code composing oracle functions; the full-size
forward is too large for the oracle to run whole).

A layer is checked from the GPU's own traced input rows of that layer and
the GPU's K/V cache of that layer: the oracle computes the rows' keys and
values, their attention over the cache (no mask for canvas rows; keys at or
before the row's position for prefill rows), the output projection and the
MoE block, following the GPU's routing where a top-k decision is a near-tie
(rule R23), and the result is compared with the GPU's input of the next
layer.  Each layer's weights are generated once for all rows checked in it.
"""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

from oracle import model
from oracle import sampler as osamp
from oracle.rounding import round_bf16, round_e4m3
from oracle.weights import Weights
from tests.gpu_util import rel_l2_rows


def _n_threads():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return 4


def sample_threaded(w, z, seed, step, block, req):
    """The oracle sampler over all rows of z[C][V], rows split over threads
    (each chunk with its canvas positions); Hbar over all rows."""
    n = z.shape[0]
    nt = _n_threads()
    bounds = np.linspace(0, n, nt + 1).astype(int)
    chunks = [(bounds[i], bounds[i + 1]) for i in range(nt) if bounds[i + 1] > bounds[i]]
    with ThreadPoolExecutor(len(chunks)) as ex:
        parts = list(ex.map(lambda c: osamp.sample(w, z[c[0]:c[1]], seed, step, block, req,
                                                   pos=np.arange(c[0], c[1])), chunks))
    out = {k: np.concatenate([p[k] for p in parts]) for k in ("H", "a", "pmax", "margin", "lock", "x_next")}
    out["Hbar"] = float(out["H"].mean())
    return out


def routing_adoptions(w, r, gpu_ids, tol, what):
    """Rows whose GPU top-k set differs from the oracle's own: every chosen
    expert must lie within tol * rms(logits) of the oracle's k-th logit."""
    k = w["k"]
    own = np.argsort(-r, axis=1, kind="stable")[:, :k]
    kth = np.sort(r, axis=1)[:, ::-1][:, k - 1]
    rms = np.sqrt(np.mean(r ** 2, axis=1))
    adopted = 0
    for t in range(r.shape[0]):
        if set(gpu_ids[t]) != set(own[t]):
            short = (kth[t] - r[t, gpu_ids[t]].min()) / rms[t]
            assert short <= tol, (what, t, f"chosen expert {short:.3g} rms below the k-th logit")
            adopted += 1
    return adopted


def check_layer(w, l, items, tol, W=None):
    """Check layer l for several groups of rows (items), each a dict:
    h_in [n][d] GPU input rows of layer l; h_out [n][d] the GPU's input rows
    of layer l+1 (or final residual); pos [n] their positions; K, V
    [Hkv][m][dh] the GPU's cache of layer l (keys 0..m-1); causal (prefill
    rows see keys <= their position, canvas rows every key); ids [n][k] the
    GPU's routing; k_got, v_got [n][Hkv][dh] the GPU's new keys/values.
    Returns, per item, the max per-row relative L2 errors of k, v and h_out
    and the routing adoptions; asserts each against tol."""
    W = Weights(w, cache=False) if W is None else W
    Hq, Hkv, dh = w["Hq"], w["Hkv"], w["dh"]
    wq, wk, wv, wo = (W.get(n, l) for n in ("wq", "wk", "wv", "wo"))
    mids, res = [], []
    for it in items:
        n = it["h_in"].shape[0]
        u = model.rmsnorm(it["h_in"], w["eps"])
        q = model.rope((u @ wq.T).reshape(n, Hq, dh), it["pos"], w["theta"])
        k = model.rope((u @ wk.T).reshape(n, Hkv, dh), it["pos"], w["theta"])
        v = (u @ wv.T).reshape(n, Hkv, dh)
        m = it["K"].shape[1]
        allowed = (np.arange(m)[None, :] <= np.asarray(it["pos"])[:, None]) if it["causal"] else None
        o = model.attention(q, np.asarray(it["K"], np.float64), np.asarray(it["V"], np.float64),
                            allowed).reshape(n, Hq * dh)
        mids.append(it["h_in"] + o @ wo.T)
        res.append(dict(err_k=rel_l2_rows(it["k_got"].reshape(n, -1), k.reshape(n, -1)).max(),
                        err_v=rel_l2_rows(it["v_got"].reshape(n, -1), v.reshape(n, -1)).max()))
    h_mid = np.concatenate(mids)
    ids = np.concatenate([it["ids"] for it in items]).astype(np.int64)
    u2 = model.rmsnorm(h_mid, w["eps"])
    f, r, _, _ = model.moe(w, W, l, u2, forced_ids=ids)
    h_out = h_mid + f
    i0 = 0
    for it, rs in zip(items, res):
        n = it["h_in"].shape[0]
        rs["err_h"] = rel_l2_rows(it["h_out"], h_out[i0:i0 + n]).max()
        rs["n"] = n
        for key in ("err_k", "err_v", "err_h"):
            assert rs[key] <= tol, (l, it.get("name"), key, rs[key])
        rs["adopted"] = routing_adoptions(w, r[i0:i0 + n], ids[i0:i0 + n], tol, (l, it.get("name")))
        i0 += n
    return res


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
    adopted = routing_adoptions(w, r, gpu_ids, tol, l)
    f, _, _, _ = model.moe(w, W, l, u2, forced_ids=gpu_ids)
    return h + f, k, v, adopted


class Summary:
    """Largest errors and adoption counts over a test, printed as one line."""

    def __init__(self, name):
        self.name = name
        self.err = {}
        self.adopted = 0
        self.decisions = 0

    def add(self, key, value):
        self.err[key] = max(self.err.get(key, 0.0), float(value))

    def add_layer(self, res, prefix=""):
        for r in res:
            for key in ("err_k", "err_v", "err_h"):
                self.add(prefix + key, r[key])
            self.adopted += r["adopted"]
            self.decisions += r["n"]

    def report(self, max_adopt_frac):
        line = {"case": self.name, "adopted": self.adopted, "decisions": self.decisions,
                **{k: float(f"{v:.3e}") for k, v in sorted(self.err.items())}}
        print(f"[parity] {line}", flush=True)
        assert self.adopted <= max(2, max_adopt_frac * self.decisions), line
        return line


# ---- the W8A8 path of the batched fp8 model, modelled in the test -----------------
# The oracle does not emulate GPU roundings (reading R18), so with activations
# quantised to E4M3 its keys and outputs differ from the GPU's by the
# quantisation itself (about 3e-2).  The functions below model the GPU's
# arithmetic step by step on the same inputs -- bf16 activation rows, the
# per-row E4M3 quantiser, bf16 intermediate and output rows -- with the
# oracle's stored weights and its rounding functions, so that the W8A8 kernels
# are checked against what they are meant to compute to about the bf16 output
# rounding.

def e4m3_rows(x):
    """Model of the activation quantiser: each row in bf16, scaled by
    448 / max|row| in fp32, clamped to +-448 and rounded to E4M3 (nearest
    even); returned as the codes times the row scale max|row| / 448 (fp32)."""
    xb = round_bf16(np.asarray(x, np.float64)).astype(np.float32)
    amax = np.abs(xb).max(axis=1)
    live = amax > 0
    safe = np.where(live, amax, np.float32(1))
    inv = np.where(live, np.float32(448) / safe, np.float32(1)).astype(np.float32)
    f = np.clip(xb * inv[:, None], np.float32(-448), np.float32(448)).astype(np.float32)
    codes = round_e4m3(f.astype(np.float64))
    scale = np.where(live, safe / np.float32(448), np.float32(1)).astype(np.float32)
    return codes * scale[:, None].astype(np.float64)


def check_layer_w8a8(w, l, items, tol_kv, tol_h, experts, qkv8=True, tol_moe=None):
    """Layer l along the GPU's arithmetic for the rows of items (as in
    check_layer): queries, keys and values from E4M3-quantised bf16 rows
    (qkv8; else from the bf16 rows);
    attention over the GPU's cache, its output rounded to bf16 before the
    output projection; the MoE input rounded to bf16; when experts is set the
    routed experts' gate/up input quantised per token row and their down input
    (the bf16 SwiGLU rows) per row, else both in bf16; bf16 expert output
    rows; the shared FFN in bf16.  Routing follows the GPU's choice; the
    gates are the softmax of the modelled router logits over it.

    An item may carry h_mid, the GPU's residual rows after the attention
    block (the MoE block's input).  The modelled rows are then checked
    against it (within tol_h), and the MoE block is modelled from the GPU's
    own h_mid, so that its E4M3 rounding decisions are the GPU's (from the
    modelled h_mid, input differences of about 1e-3 flip some of them, which
    leaves about 2% of the MoE output unexplained).  The MoE output
    h_out - h_mid of every row is then checked within tol_moe, relative to
    its own norm, and the per-row errors are returned as "moe_rows": fp32
    rounding upstream of the down projection's quantiser (the SwiGLU in
    fp32, for one) still moves an occasional element of its input across an
    E4M3 rounding boundary, one E4M3 step of one element (about 0.6% of a
    row's output at the widths tested), so the callers bound the median of
    these errors tightly and each row loosely.

    Asserts the keys/values within tol_kv and (tol_h not None) the layer
    output within tol_h; returns the largest errors."""
    W = Weights(w, cache=False)
    Hq, Hkv, dh, eps = w["Hq"], w["Hkv"], w["dh"], w["eps"]
    wq, wk, wv = (W.get(n, l) for n in ("wq", "wk", "wv"))
    out = {"err_k8": 0.0, "err_v8": 0.0}
    mids = []
    for it in items:
        n = it["h_in"].shape[0]
        u = model.rmsnorm(it["h_in"], eps)
        uq = e4m3_rows(u) if qkv8 else round_bf16(u)
        q = model.rope((uq @ wq.T).reshape(n, Hq, dh), it["pos"], w["theta"])
        k = model.rope((uq @ wk.T).reshape(n, Hkv, dh), it["pos"], w["theta"])
        v = (uq @ wv.T).reshape(n, Hkv, dh)
        ek = rel_l2_rows(it["k_got"].reshape(n, -1), k.reshape(n, -1)).max()
        ev = rel_l2_rows(it["v_got"].reshape(n, -1), v.reshape(n, -1)).max()
        assert ek <= tol_kv and ev <= tol_kv, (l, it.get("name"), "w8a8 k/v", ek, ev)
        out["err_k8"] = max(out["err_k8"], float(ek))
        out["err_v8"] = max(out["err_v8"], float(ev))
        if tol_h is not None:
            m = it["K"].shape[1]
            allowed = (np.arange(m)[None, :] <= np.asarray(it["pos"])[:, None]) if it["causal"] else None
            o = model.attention(q, np.asarray(it["K"], np.float64), np.asarray(it["V"], np.float64), allowed)
            mid = it["h_in"] + round_bf16(o.reshape(n, Hq * dh)) @ W.get("wo", l).T
            if it.get("h_mid") is not None:
                em = rel_l2_rows(it["h_mid"], mid).max()
                assert em <= tol_h, (l, it.get("name"), "w8a8 h_mid", em)
                out["err_mid8"] = max(out.get("err_mid8", 0.0), float(em))
                mid = np.asarray(it["h_mid"], np.float64)
            mids.append(mid)
    if tol_h is None:
        return out
    h_mid = np.concatenate(mids)
    ids = np.concatenate([it["ids"] for it in items]).astype(np.int64)
    u2 = round_bf16(model.rmsnorm(h_mid, eps))
    r = u2 @ W.get("wr", l).T
    sel = np.take_along_axis(r, ids, axis=1)
    gates = np.exp(sel - sel.max(axis=1, keepdims=True))
    gates /= gates.sum(axis=1, keepdims=True)
    xin = e4m3_rows(u2) if experts else u2
    f = np.zeros_like(u2)
    for e in np.unique(ids):
        rows, slot = np.nonzero(ids == e)
        g = xin[rows] @ W.get("wg", l, e).T
        up = xin[rows] @ W.get("wu", l, e).T
        hid = round_bf16(model.silu(g) * up)
        y = round_bf16((e4m3_rows(hid) if experts else hid) @ W.get("wd", l, e).T)
        f[rows] += gates[rows, slot][:, None] * y
    if w["fs"] > 0:
        hs = round_bf16(model.silu(u2 @ W.get("sg", l).T) * (u2 @ W.get("su", l).T))
        f += hs @ W.get("sd", l).T
    h_out = h_mid + f
    i0 = 0
    out["err_h8"] = 0.0
    for it in items:
        n = it["h_in"].shape[0]
        eh = rel_l2_rows(it["h_out"], h_out[i0:i0 + n]).max()
        assert eh <= tol_h, (l, it.get("name"), "w8a8 h", eh)
        out["err_h8"] = max(out["err_h8"], float(eh))
        if it.get("h_mid") is not None:
            ef = rel_l2_rows(np.asarray(it["h_out"], np.float64) - h_mid[i0:i0 + n], f[i0:i0 + n])
            assert tol_moe is None or ef.max() <= tol_moe, (l, it.get("name"), "w8a8 moe", ef.max())
            out["err_moe8"] = max(out.get("err_moe8", 0.0), float(ef.max()))
            out["moe_rows"] = np.concatenate([out.get("moe_rows", np.zeros(0)), ef])
        i0 += n
    return out
