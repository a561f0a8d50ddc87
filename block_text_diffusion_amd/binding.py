"""ctypes binding of libcd (include/cd.h): same names, argument marshalling only.

Device buffers are torch tensors on the HIP device (torch is the allocator and
the stream provider); every computation runs in libcd's HIP kernels.  Loading
fails loudly when libcd.so has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcd.so")

c_int32, c_uint64, c_size_t, c_void_p, c_float, c_double = (
    ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float, ctypes.c_double)

CD_OK, CD_ERR_INVALID_ARG, CD_ERR_BAD_STATE, CD_ERR_CAPACITY, CD_ERR_HIP, CD_ERR_UNSUPPORTED, CD_ERR_NUMERIC = (
    0, -1, -2, -3, -4, -5, -6)
CD_F32, CD_BF16, CD_FP8, CD_MXFP4 = 0, 1, 2, 3
CD_LOCK_MAXPROB, CD_LOCK_ENTROPY = 0, 1
(CD_W_EMBED, CD_W_LM, CD_W_Q, CD_W_K, CD_W_V, CD_W_O, CD_W_ROUTER, CD_W_GATE, CD_W_UP, CD_W_DOWN,
 CD_W_SHARED_GATE, CD_W_SHARED_UP, CD_W_SHARED_DOWN) = range(13)
(CD_BUF_LOGITS, CD_BUF_CANVAS, CD_BUF_ARGMAX, CD_BUF_ENTROPY, CD_BUF_PMAX, CD_BUF_LOCK, CD_BUF_KCACHE,
 CD_BUF_VCACHE, CD_BUF_HIDDEN) = range(9)


class cd_config(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in (
        "n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "n_experts", "top_k",
        "expert_hidden", "shared_hidden", "vocab", "canvas_len", "max_steps")] + [
        (n, c_float) for n in ("lock_threshold", "stop_entropy", "rms_eps", "rope_theta")] + [
        (n, c_int32) for n in ("weight_dtype", "max_requests", "max_ctx", "max_prefill")] + [
        ("attn_rescale_log2", c_float), ("lock_rule", c_int32), ("entropy_bound", c_float)]


class cd_step_info(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in ("step", "stop", "n_locked", "stable", "canvas_is_argmax",
                                       "nonfinite", "after_stop")] + [("mean_entropy", c_double)]


STEP_INFO_BYTES = ctypes.sizeof(cd_step_info)


class CDError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libcd error {code}: {msg}")
        self.code = code


_lib = None


def lib():
    """Load libcd.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m block_text_diffusion_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        sig = {
            "cd_weights_bytes": [P(cd_config), P(c_size_t)],
            "cd_state_bytes": [P(cd_config), P(c_size_t)],
            "cd_ctx_create": [P(cd_config), c_void_p, c_void_p, P(c_void_p)],
            "cd_ctx_destroy": [c_void_p],
            "cd_reset": [c_void_p, c_void_p],
            "cd_synth_weights": [c_void_p, c_uint64, c_void_p],
            "cd_set_weight": [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p],
            "cd_get_weight": [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p],
            "cd_prefill": [c_void_p, c_int32, c_void_p, c_int32, c_void_p],
            "cd_init_canvas": [c_void_p, c_int32, c_uint64, c_int32, c_void_p],
            "cd_denoise_step": [c_void_p, c_int32, c_void_p, c_void_p],
            "cd_read_step_info": [c_void_p, c_void_p, c_int32, c_void_p, c_void_p],
            "cd_commit_block": [c_void_p, c_int32, c_void_p, c_void_p],
            "cd_generate": [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_uint64, c_void_p,
                            P(c_int32), c_void_p],
            "cd_sample_workspace_bytes": [c_int32, c_int32, P(c_size_t)],
            "cd_sample_step": [P(cd_config), c_void_p, c_int32, c_void_p, c_uint64, c_int32, c_int32,
                               c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                               c_void_p, c_void_p],
            "cd_sample_step_noalloc": [P(cd_config), c_void_p, c_int32, c_void_p, c_uint64, c_int32, c_int32,
                                       c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_void_p],
            "cd_get_buffer": [c_void_p, c_int32, P(c_void_p), P(c_size_t)],
            "cd_get_length": [c_void_p, c_int32, P(c_int32)],
            "cd_get_config": [c_void_p, P(cd_config)],
            "cd_set_trace": [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p],
            "cd_abort_canvas": [c_void_p, c_int32],
            "cd_release": [c_void_p, c_int32, c_void_p],
            "cd_move_request": [c_void_p, c_int32, c_int32, c_void_p],
            "cd_serve": [c_void_p, c_int32, c_void_p, P(ctypes.c_int64), P(c_int32), P(c_int32),
                         P(c_uint64), c_int32, c_void_p, P(ctypes.c_int64), P(c_int32), c_void_p],
            "cd_profile": [c_void_p, c_int32],
            "cd_set_graphs": [c_void_p, c_int32],
            "cd_profile_read": [c_void_p, c_void_p, c_void_p, c_int32],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = c_int32
        L.cd_last_error.argtypes = []
        L.cd_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def exported_names():
    return ["cd_weights_bytes", "cd_state_bytes", "cd_ctx_create", "cd_ctx_destroy", "cd_reset",
            "cd_synth_weights", "cd_set_weight", "cd_get_weight", "cd_prefill", "cd_init_canvas",
            "cd_denoise_step", "cd_read_step_info", "cd_commit_block", "cd_generate",
            "cd_sample_workspace_bytes", "cd_sample_step", "cd_sample_step_noalloc", "cd_get_buffer", "cd_get_config", "cd_get_length",
            "cd_set_trace", "cd_abort_canvas", "cd_release", "cd_move_request", "cd_serve", "cd_profile", "cd_set_graphs", "cd_profile_read",
            "cd_last_error"]


def _check(code):
    if code != CD_OK:
        raise CDError(code, lib().cd_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def make_config(w: dict, max_requests=None, max_ctx=None, max_prefill=None) -> cd_config:
    """cd_config from a workload dict (synth_inputs layout)."""
    dt = {"f32": CD_F32, "bf16": CD_BF16, "fp8": CD_FP8, "mxfp4": CD_MXFP4}[w["wdtype"]]
    R = max_requests or w.get("R", 1)
    P0 = w.get("P0", 0)
    return cd_config(
        n_layers=w["L"], d_model=w["d"], n_q_heads=w["Hq"], n_kv_heads=w["Hkv"], head_dim=w["dh"],
        n_experts=w["E"], top_k=w["k"], expert_hidden=w["fe"], shared_hidden=w["fs"], vocab=w["V"],
        canvas_len=w["C"], max_steps=w["max_steps"], lock_threshold=w["lock"], stop_entropy=w["stop_H"],
        rms_eps=w["eps"], rope_theta=w["theta"], weight_dtype=dt, max_requests=R,
        max_ctx=max_ctx or (P0 + w.get("blocks", 1) * w["C"]),
        max_prefill=max_prefill or max(P0, 1), attn_rescale_log2=w.get("attn_rescale_log2", 0.0),
        lock_rule={"maxprob": CD_LOCK_MAXPROB, "entropy": CD_LOCK_ENTROPY}[w.get("lock_rule", "maxprob")],
        entropy_bound=w.get("entropy_bound", 0.1))


def cd_weights_bytes(cfg):
    n = c_size_t()
    _check(lib().cd_weights_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def cd_state_bytes(cfg):
    n = c_size_t()
    _check(lib().cd_state_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def cd_ctx_create(cfg, weights, state):
    h = c_void_p()
    _check(lib().cd_ctx_create(ctypes.byref(cfg), _ptr(weights), _ptr(state), ctypes.byref(h)))
    return h


def cd_ctx_destroy(ctx):
    _check(lib().cd_ctx_destroy(ctx))


def cd_reset(ctx, stream=None):
    _check(lib().cd_reset(ctx, _stream(stream)))


def cd_synth_weights(ctx, seed, stream=None):
    _check(lib().cd_synth_weights(ctx, seed, _stream(stream)))


def cd_set_weight(ctx, kind, layer, expert, t, stream=None):
    _check(lib().cd_set_weight(ctx, kind, layer, expert, _ptr(t), _stream(stream)))


def cd_get_weight(ctx, kind, layer, expert, t, stream=None):
    _check(lib().cd_get_weight(ctx, kind, layer, expert, _ptr(t), _stream(stream)))


def cd_prefill(ctx, req, ids, n=None, stream=None):
    _check(lib().cd_prefill(ctx, req, _ptr(ids), ids.numel() if n is None else n, _stream(stream)))


def cd_init_canvas(ctx, req, seed, block, stream=None):
    _check(lib().cd_init_canvas(ctx, req, seed, block, _stream(stream)))


def cd_denoise_step(ctx, n_req, info, stream=None):
    _check(lib().cd_denoise_step(ctx, n_req, _ptr(info), _stream(stream)))


def cd_read_step_info(ctx, info, n_req, stream=None):
    out = (cd_step_info * n_req)()
    _check(lib().cd_read_step_info(ctx, _ptr(info), n_req, out, _stream(stream)))
    return list(out)


def _check_ids(t, n, what):
    """Output ids: a contiguous int32 tensor of exactly n elements."""
    import torch
    if not (isinstance(t, torch.Tensor) and t.dtype == torch.int32 and t.is_contiguous() and t.numel() == n):
        raise ValueError(f"{what}: needs a contiguous int32 tensor of exactly {n} ids")


def cd_commit_block(ctx, req, out_ids, stream=None):
    _check_ids(out_ids, cd_get_config(ctx).canvas_len, "cd_commit_block out_ids")
    _check(lib().cd_commit_block(ctx, req, _ptr(out_ids), _stream(stream)))


def cd_generate(ctx, req, prefix, n_blocks, seed, out_ids, stream=None):
    _check_ids(out_ids, n_blocks * cd_get_config(ctx).canvas_len, "cd_generate out_ids")
    steps = (c_int32 * n_blocks)()
    n_prefix = 0 if prefix is None else prefix.numel()
    _check(lib().cd_generate(ctx, req, _ptr(prefix), n_prefix, n_blocks, seed, _ptr(out_ids), steps,
                             _stream(stream)))
    return list(steps)


def cd_release(ctx, req, stream=None):
    _check(lib().cd_release(ctx, req, _stream(stream)))


def cd_move_request(ctx, src, dst, stream=None):
    _check(lib().cd_move_request(ctx, src, dst, _stream(stream)))


def cd_serve(ctx, prefixes, n_blocks, seeds, n_slots, out_ids, stream=None):
    """Queue of requests: prefixes (list of 1-D int32 device tensors), blocks
    and seeds per request.  out_ids (1-D int32 device) holds exactly
    sum(n_blocks) * canvas_len ids; request q's blocks land at the offset of
    the blocks of requests before it.  Returns the passes per block, one list
    per request."""
    import torch
    n_q = len(prefixes)
    assert len(n_blocks) == n_q and len(seeds) == n_q
    flat = torch.cat([p.reshape(-1) for p in prefixes]).to(torch.int32).contiguous()
    lens = [int(p.numel()) for p in prefixes]
    poff = [0] * n_q
    for q in range(1, n_q):
        poff[q] = poff[q - 1] + lens[q - 1]
    # out_ids holds exactly sum(n_blocks) blocks of the context's canvas_len ids
    C = cd_get_config(ctx).canvas_len
    _check_ids(out_ids, sum(n_blocks) * C, "cd_serve out_ids")
    ooff = [0] * n_q
    for q in range(1, n_q):
        ooff[q] = ooff[q - 1] + n_blocks[q - 1] * C
    steps = (c_int32 * sum(n_blocks))()
    code = lib().cd_serve(ctx, n_q, _ptr(flat), (ctypes.c_int64 * n_q)(*poff), (c_int32 * n_q)(*lens),
                          (c_int32 * n_q)(*n_blocks), (c_uint64 * n_q)(*seeds), n_slots, _ptr(out_ids),
                          (ctypes.c_int64 * n_q)(*ooff), steps, _stream(stream))
    if code != CD_OK:
        # a failing call may leave prefills of the concatenated prompts queued
        torch.cuda.synchronize()
    _check(code)
    out, i = [], 0
    for nb in n_blocks:
        out.append(list(steps[i:i + nb]))
        i += nb
    return out


def cd_sample_workspace_bytes(rows, vocab):
    n = c_size_t()
    _check(lib().cd_sample_workspace_bytes(rows, vocab, ctypes.byref(n)))
    return n.value


def cd_sample_step(cfg, logits, rows, prev_argmax, seed, step, block, req0, tokens, argmax, lock,
                   entropy, pmax, info, workspace, stream=None):
    _check(lib().cd_sample_step(ctypes.byref(cfg), _ptr(logits), rows, _ptr(prev_argmax), seed, step,
                                block, req0, _ptr(tokens), _ptr(argmax), _ptr(lock), _ptr(entropy),
                                _ptr(pmax), _ptr(info), _ptr(workspace), _stream(stream)))


def cd_sample_step_noalloc(cfg, logits, rows, prev_argmax, seed, step, block, req0, tokens, argmax, lock,
                           entropy, pmax, info, stream=None):
    _check(lib().cd_sample_step_noalloc(ctypes.byref(cfg), _ptr(logits), rows, _ptr(prev_argmax), seed, step,
                                        block, req0, _ptr(tokens), _ptr(argmax), _ptr(lock), _ptr(entropy),
                                        _ptr(pmax), _ptr(info), _stream(stream)))


def cd_get_buffer(ctx, which):
    p, n = c_void_p(), c_size_t()
    _check(lib().cd_get_buffer(ctx, which, ctypes.byref(p), ctypes.byref(n)))
    return p.value, n.value


def cd_get_config(ctx):
    cfg = cd_config()
    _check(lib().cd_get_config(ctx, ctypes.byref(cfg)))
    return cfg


def cd_get_length(ctx, req):
    P = c_int32()
    _check(lib().cd_get_length(ctx, req, ctypes.byref(P)))
    return P.value


def cd_set_trace(ctx, h_layers=None, topk_ids=None, topk_gates=None, h_mid=None):
    _check(lib().cd_set_trace(ctx, _ptr(h_layers), _ptr(topk_ids), _ptr(topk_gates), _ptr(h_mid)))


PROF_CLASSES = ["embed", "rmsnorm", "qkv", "attention", "attn_merge", "o_proj", "router", "route",
                "expert_gate_up", "expert_down", "combine", "shared_gate_up", "shared_down", "lm_head",
                "sampler_part", "sampler_final", "other", "act_quant"]


def cd_abort_canvas(ctx, req):
    _check(lib().cd_abort_canvas(ctx, req))


def cd_profile(ctx, enable):
    _check(lib().cd_profile(ctx, 1 if enable else 0))


def cd_set_graphs(ctx, enable):
    _check(lib().cd_set_graphs(ctx, 1 if enable else 0))


def cd_profile_read(ctx):
    n = len(PROF_CLASSES)
    ms = (c_double * n)()
    cnt = (c_int32 * n)()
    _check(lib().cd_profile_read(ctx, ms, cnt, n))
    return {PROF_CLASSES[i]: (ms[i], cnt[i]) for i in range(n)}


def cd_last_error():
    return lib().cd_last_error().decode()
