"""Host-side checks of libcd: it loads, exports every entry point of
include/cd.h, and validates arguments and request state before enqueuing
anything (these calls return before any HIP call, so they run without a GPU).
"""
import ctypes
import os
import re

import pytest

import synth_inputs
from block_text_diffusion_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "cd.h")).read()
    return sorted(set(re.findall(r"\b(cd_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = B.lib()
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert sorted(B.exported_names()) == names


def _cfg(name="tiny", **kw):
    return B.make_config(synth_inputs.workload(name, **kw))


def test_config_validation_and_sizes():
    cfg = _cfg()
    wb, sb = B.cd_weights_bytes(cfg), B.cd_state_bytes(cfg)
    # weights: fp32 parameters of the tiny model (embed, head, 2 layers)
    n_params = 2 * 4096 * 256 + 2 * (256 * 256 * 2 + 2 * 128 * 256 + 8 * 256 + 8 * 3 * 512 * 256)
    assert 4 * n_params <= wb <= 4 * n_params * 1.1
    assert sb > 4 * 256 * 4096
    big = _cfg("step_bf16")
    assert 2 * 25.0e9 < B.cd_weights_bytes(big) < 2 * 26.5e9
    for field, val, code in [("head_dim", 96, B.CD_ERR_UNSUPPORTED), ("vocab", 1000, B.CD_ERR_UNSUPPORTED),
                             ("n_kv_heads", 3, B.CD_ERR_INVALID_ARG), ("top_k", 9, B.CD_ERR_UNSUPPORTED),
                             ("d_model", 250, B.CD_ERR_UNSUPPORTED), ("max_ctx", 100, B.CD_ERR_INVALID_ARG),
                             ("weight_dtype", 7, B.CD_ERR_INVALID_ARG), ("attn_rescale_log2", -1.0, B.CD_ERR_INVALID_ARG),
                             ("attn_rescale_log2", 65.0, B.CD_ERR_INVALID_ARG), ("lock_rule", 2, B.CD_ERR_INVALID_ARG),
                             ("entropy_bound", -0.5, B.CD_ERR_INVALID_ARG),
                             ("entropy_bound", float("inf"), B.CD_ERR_INVALID_ARG)]:
        bad = _cfg()
        setattr(bad, field, val)
        with pytest.raises(B.CDError) as e:
            B.cd_weights_bytes(bad)
        assert e.value.code == code, field
        assert B.cd_last_error()


def _fake_ctx(cfg):
    # 256-aligned fake device addresses: the calls below must fail validation
    # before touching device memory or the HIP runtime
    return B.cd_ctx_create(cfg, 1 << 20, 1 << 30)


def test_state_machine_rejects_out_of_order_calls_without_side_effects():
    cfg = _cfg()
    ctx = _fake_ctx(cfg)
    L = B.lib()
    info = 1 << 12
    assert L.cd_denoise_step(ctx, 1, info, None) == B.CD_ERR_BAD_STATE
    assert L.cd_commit_block(ctx, 0, 1 << 12, None) == B.CD_ERR_BAD_STATE
    assert L.cd_denoise_step(ctx, 2, info, None) == B.CD_ERR_INVALID_ARG    # beyond max_requests
    assert L.cd_denoise_step(ctx, 1, None, None) == B.CD_ERR_INVALID_ARG
    assert L.cd_prefill(ctx, 0, 1 << 12, cfg.max_prefill + 1, None) == B.CD_ERR_INVALID_ARG
    assert L.cd_prefill(ctx, 1, 1 << 12, 4, None) == B.CD_ERR_INVALID_ARG
    assert L.cd_init_canvas(ctx, 0, 1, -1, None) == B.CD_ERR_INVALID_ARG
    assert L.cd_set_weight(ctx, B.CD_W_Q, 5, 0, 1 << 12, None) == B.CD_ERR_INVALID_ARG
    assert L.cd_set_weight(ctx, B.CD_W_GATE, 0, 8, 1 << 12, None) == B.CD_ERR_INVALID_ARG
    assert L.cd_set_weight(ctx, B.CD_W_SHARED_UP, 0, 0, 1 << 12, None) == B.CD_ERR_INVALID_ARG
    assert L.cd_get_buffer(ctx, 99, ctypes.byref(ctypes.c_void_p()), None) == B.CD_ERR_INVALID_ARG
    steps = (ctypes.c_int32 * 1)()
    assert L.cd_generate(ctx, 0, None, 0, 0, 1, 1 << 12, steps, None) == B.CD_ERR_INVALID_ARG
    assert L.cd_generate(ctx, 0, None, 0, 9, 1, 1 << 12, steps, None) == B.CD_ERR_CAPACITY
    assert B.cd_get_length(ctx, 0) == 0
    B.cd_ctx_destroy(ctx)


def test_serve_and_release_argument_checks():
    cfg = _cfg()
    cfg.max_requests = 2
    ctx = _fake_ctx(cfg)
    L = B.lib()
    assert L.cd_release(ctx, -1, None) == B.CD_ERR_INVALID_ARG
    assert L.cd_release(ctx, 2, None) == B.CD_ERR_INVALID_ARG
    for a, b in [(0, 0), (-1, 0), (0, 2), (2, 1)]:
        assert L.cd_move_request(ctx, a, b, None) == B.CD_ERR_INVALID_ARG
    i64, i32, u64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64
    C = cfg.canvas_len

    def serve(n_q=1, lens=(16,), blocks=(1,), slots=1, poff=(0,), ooff=(0,)):
        n = len(lens)
        steps = (i32 * 8)()
        return L.cd_serve(ctx, n_q, 1 << 12, (i64 * n)(*poff), (i32 * n)(*lens), (i32 * n)(*blocks),
                          (u64 * n)(*([1] * n)), slots, 1 << 12, (i64 * n)(*ooff), steps, None)
    assert serve(n_q=0) == B.CD_ERR_INVALID_ARG
    assert serve(slots=0) == B.CD_ERR_INVALID_ARG
    assert serve(slots=3) == B.CD_ERR_INVALID_ARG                        # beyond max_requests
    assert serve(lens=(0,)) == B.CD_ERR_INVALID_ARG
    assert serve(lens=(cfg.max_prefill + 1,)) == B.CD_ERR_INVALID_ARG
    assert serve(blocks=(0,)) == B.CD_ERR_INVALID_ARG
    assert serve(poff=(-1,)) == B.CD_ERR_INVALID_ARG
    assert serve(ooff=(-1,)) == B.CD_ERR_INVALID_ARG
    n_fit = (cfg.max_ctx - 16) // C
    assert serve(blocks=(n_fit + 1,)) == B.CD_ERR_CAPACITY
    assert serve(n_q=2, lens=(16, 16), blocks=(1, n_fit + 1), poff=(0, 16), ooff=(0, C)) == B.CD_ERR_CAPACITY
    B.cd_ctx_destroy(ctx)
    bad = _cfg()
    bad.max_requests = 257
    with pytest.raises(B.CDError) as e:
        B.cd_state_bytes(bad)
    assert e.value.code == B.CD_ERR_UNSUPPORTED


def test_capacity_checked_before_prefill():
    cfg = _cfg(P0=128)
    cfg.max_ctx = 300                                   # 128 + 256 does not fit
    ctx = _fake_ctx(cfg)
    assert B.lib().cd_prefill(ctx, 0, 1 << 12, 128, None) == B.CD_ERR_CAPACITY
    assert B.cd_get_length(ctx, 0) == 0
    B.cd_ctx_destroy(ctx)


def test_sampler_argument_checks():
    cfg = _cfg("sampler", L=1, d=64, Hq=1, Hkv=1, dh=64, E=1, k=1, fe=64, fs=0, wdtype="f32", P0=0)
    # one 16-byte partial per (row, chunk of at most 8192 logits)
    assert B.cd_sample_workspace_bytes(256, 262144) == 16 * 256 * (262144 // 8192)
    L = B.lib()
    args = [1 << 12] * 8
    assert L.cd_sample_step(ctypes.byref(cfg), 1 << 12, 100, None, 1, 1, 0, 0, *args[:7], None) == B.CD_ERR_INVALID_ARG
    assert L.cd_sample_step(ctypes.byref(cfg), 1 << 12, 256, None, 1, 0, 0, 0, *args[:7], None) == B.CD_ERR_INVALID_ARG


def test_get_config_and_binding_output_size_checks():
    import torch
    cfg = _cfg()
    ctx = _fake_ctx(cfg)
    got = B.cd_get_config(ctx)
    assert (got.canvas_len, got.vocab, got.n_layers, got.max_requests) == (
        cfg.canvas_len, cfg.vocab, cfg.n_layers, cfg.max_requests)
    C = cfg.canvas_len
    for bad in (torch.empty(C - 1, dtype=torch.int32), torch.empty(C, dtype=torch.int64),
                torch.empty(2 * C, dtype=torch.int32)[::2]):
        with pytest.raises(ValueError):
            B.cd_commit_block(ctx, 0, bad)
    with pytest.raises(B.CDError) as e:            # right size: the library's own state check
        B.cd_commit_block(ctx, 0, torch.empty(C, dtype=torch.int32), stream=0)
    assert e.value.code == B.CD_ERR_BAD_STATE
    with pytest.raises(ValueError):
        B.cd_generate(ctx, 0, None, 2, 1, torch.empty(C, dtype=torch.int32))
    with pytest.raises(ValueError):
        # a buffer of half-size blocks must not pass as two blocks of the context's canvas
        B.cd_serve(ctx, [torch.zeros(8, dtype=torch.int32)] * 2, [1, 1], [1, 2], 1,
                   torch.empty(C, dtype=torch.int32))
    assert B.cd_get_length(ctx, 0) == 0
    B.cd_ctx_destroy(ctx)
