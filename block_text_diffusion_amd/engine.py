"""Plumbing around libcd: torch allocates the weight and state buffers and
provides the stream; every step of the method runs in libcd's kernels."""
from __future__ import annotations

import torch

from . import binding as B

_DT = {torch.float32: 4, torch.int32: 4, torch.float64: 8, torch.uint8: 1, torch.bfloat16: 2}


class Engine:
    def __init__(self, workload: dict, device="cuda", max_requests=None, max_ctx=None, max_prefill=None):
        B.lib()
        self.w = workload
        self.cfg = B.make_config(workload, max_requests, max_ctx, max_prefill)
        self.device = torch.device(device)
        self.weights = torch.empty(B.cd_weights_bytes(self.cfg), dtype=torch.uint8, device=self.device)
        self.state = torch.empty(B.cd_state_bytes(self.cfg), dtype=torch.uint8, device=self.device)
        self.ctx = B.cd_ctx_create(self.cfg, self.weights, self.state)
        B.cd_reset(self.ctx)
        self.info = torch.zeros(self.cfg.max_requests * B.STEP_INFO_BYTES, dtype=torch.uint8, device=self.device)

    def close(self):
        if self.ctx is not None:
            B.cd_ctx_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def act_dtype(self):
        return torch.float32 if self.cfg.weight_dtype == B.CD_F32 else torch.bfloat16

    def view(self, which, dtype, shape):
        """A tensor view of one of libcd's internal buffers."""
        ptr, n = B.cd_get_buffer(self.ctx, which)
        off = ptr - self.state.data_ptr()
        count = 1
        for s in shape:
            count *= s
        nbytes = count * _DT[dtype]
        assert 0 <= off and off + nbytes <= self.state.numel() and nbytes <= n
        return self.state[off:off + nbytes].view(dtype).view(*shape)

    def kcache(self):
        c = self.cfg
        ctx = (c.max_ctx + 63) // 64 * 64
        return self.view(B.CD_BUF_KCACHE, self.act_dtype,
                         (c.max_requests, c.n_layers, c.n_kv_heads, ctx, c.head_dim))

    def vcache(self):
        c = self.cfg
        ctx = (c.max_ctx + 63) // 64 * 64
        return self.view(B.CD_BUF_VCACHE, self.act_dtype,
                         (c.max_requests, c.n_layers, c.n_kv_heads, c.head_dim, ctx))

    def logits(self, n_req=1):
        c = self.cfg
        return self.view(B.CD_BUF_LOGITS, torch.float32, (c.max_requests * c.canvas_len, c.vocab))[
            : n_req * c.canvas_len]

    def canvas(self):
        c = self.cfg
        return self.view(B.CD_BUF_CANVAS, torch.int32, (c.max_requests, c.canvas_len))

    def argmax(self):
        c = self.cfg
        return self.view(B.CD_BUF_ARGMAX, torch.int32, (c.max_requests, c.canvas_len))

    def step_info(self, n_req=1):
        return B.cd_read_step_info(self.ctx, self.info, n_req)

    def weight(self, kind, layer=0, expert=0, shape=None):
        out = torch.empty(shape, dtype=torch.float32, device=self.device)
        B.cd_get_weight(self.ctx, kind, layer, expert, out)
        return out
