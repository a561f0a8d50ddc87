"""Synthetic model weights: N(0, 0.02^2) from Philox4x32-10 + Box-Muller.

The pages give the model family (a 26B-total / 3.8B-active MoE on the Gemma 4
26B-A4B backbone with a new diffusion head: [P1] §2.2 table, [P4]
"architecture", [P5] intro) but no checkpoint is available, so weights are
synthetic and seeded.  Every tensor is stored [out][in] row-major; element n
of tensor tau is drawn from counter (n//4 low 32 bits, n//4 high 32 bits, tau,
TAG_WEIGHTS << 24) under key = weight seed.  Of the four output words, the
pair (r0, r1) feeds elements 4q, 4q+1 and (r2, r3) feeds 4q+2, 4q+3 through
Box-Muller in fp64: u1 = (r_a + 1) / 2^32, u2 = r_b / 2^32,
z = sqrt(-2 ln u1) * cos(2 pi u2) (even element) or * sin(2 pi u2) (odd).
w = 0.02 z, rounded once to the storage format.

Tensor ids: 0 embedding [V][d], 1 LM head [V][d]; layer l uses
2 + l*S + j with S = 8 + 3E and j = 0 Wq [Hq*dh][d], 1 Wk [Hkv*dh][d],
2 Wv [Hkv*dh][d], 3 Wo [d][Hq*dh], 4 router [E][d], 5+3e+{0,1,2} expert e
gate [fe][d], up [fe][d], down [d][fe], 5+3E+{0,1,2} shared gate/up/down.

Storage: ``f32`` workloads keep fp32; ``bf16`` workloads keep bf16;
``fp8`` workloads keep Wq/Wk/Wv/Wo and routed experts as E4M3FN with a bf16
scale per output row (s = bf16(max|w_row| / 448), q = e4m3(w / s)) and every
other tensor in bf16; ``mxfp4`` workloads keep the routed experts as MXFP4
(one E8M0 scale 2^e per 32 input columns of a row, e = floor(log2 of the
block's largest magnitude) - 2, elements rounded to E2M1), Wq/Wk/Wv/Wo as
fp8 like the ``fp8`` workloads, and every other tensor in bf16.

Pins (tests/test_oracle_weights.py): Kolmogorov-Smirnov against the normal CDF,
the chi-square(2) law of z0^2 + z1^2 for each Box-Muller pair, independence of
the pair, and storage values equal to the rounding routines' output.
"""
from __future__ import annotations

import numpy as np

from . import philox
from .rounding import round_bf16, round_e4m3, round_fp32, quantize_mxfp4, E4M3_MAX

STD = 0.02

LAYER_TENSORS = ("wq", "wk", "wv", "wo", "wr")


def slots_per_layer(cfg) -> int:
    return 8 + 3 * cfg["E"]


def tensor_id(cfg, name, layer=None, expert=None) -> int:
    if name == "embed":
        return 0
    if name == "lm":
        return 1
    base = 2 + layer * slots_per_layer(cfg)
    if name in LAYER_TENSORS:
        return base + LAYER_TENSORS.index(name)
    if name in ("wg", "wu", "wd"):
        return base + 5 + 3 * expert + ("wg", "wu", "wd").index(name)
    if name in ("sg", "su", "sd"):
        return base + 5 + 3 * cfg["E"] + ("sg", "su", "sd").index(name)
    raise KeyError(name)


def tensor_shape(cfg, name):
    d, dh = cfg["d"], cfg["dh"]
    return {
        "embed": (cfg["V"], d), "lm": (cfg["V"], d),
        "wq": (cfg["Hq"] * dh, d), "wk": (cfg["Hkv"] * dh, d),
        "wv": (cfg["Hkv"] * dh, d), "wo": (d, cfg["Hq"] * dh),
        "wr": (cfg["E"], d),
        "wg": (cfg["fe"], d), "wu": (cfg["fe"], d), "wd": (d, cfg["fe"]),
        "sg": (cfg["fs"], d), "su": (cfg["fs"], d), "sd": (d, cfg["fs"]),
    }[name]


def storage(cfg, name) -> str:
    """Storage format of a tensor: 'f32', 'bf16', 'fp8' or 'mxfp4'."""
    wd = cfg["wdtype"]
    if wd == "fp8":
        return "fp8" if name in ("wq", "wk", "wv", "wo", "wg", "wu", "wd") else "bf16"
    if wd == "mxfp4":
        if name in ("wg", "wu", "wd"):
            return "mxfp4"
        return "fp8" if name in ("wq", "wk", "wv", "wo") else "bf16"
    return wd


def normal_draws(seed, tau, n_idx):
    """fp64 standard normals for element indices ``n_idx`` of tensor ``tau``."""
    n_idx = np.asarray(n_idx, dtype=np.uint64)
    q = n_idx >> np.uint64(2)
    m = (n_idx & np.uint64(3)).astype(np.int64)
    k0, k1 = philox.seed_key(seed)
    r = philox.philox4x32_10(q & np.uint64(0xFFFFFFFF), q >> np.uint64(32), tau,
                             philox.TAG_WEIGHTS << 24, k0, k1)
    r = np.stack(r).astype(np.float64)          # [4][...]
    pair = m >> 1                              # 0 -> (r0, r1), 1 -> (r2, r3)
    ra = np.where(pair == 0, r[0], r[2])
    rb = np.where(pair == 0, r[1], r[3])
    u1 = (ra + 1.0) * 2.0 ** -32
    u2 = rb * 2.0 ** -32
    rad = np.sqrt(-2.0 * np.log(u1))
    ang = 2.0 * np.pi * u2
    return np.where((m & 1) == 0, rad * np.cos(ang), rad * np.sin(ang))


def raw_rows(cfg, name, layer=None, expert=None, rows=None):
    """Unrounded fp64 values 0.02*z of selected rows of a tensor."""
    n_out, n_in = tensor_shape(cfg, name)
    rows = np.arange(n_out) if rows is None else np.asarray(rows, dtype=np.int64)
    tau = tensor_id(cfg, name, layer, expert)
    idx = rows[:, None].astype(np.uint64) * np.uint64(n_in) + np.arange(n_in, dtype=np.uint64)[None, :]
    return STD * normal_draws(cfg["weight_seed"], tau, idx)


_FMT_CODE = {"f32": 0, "bf16": 1, "fp8": 2, "mxfp4": 3}
_wgen = None


def _c_generator():
    """The C version of stored_rows (oracle/csrc/wgen.c, built into
    oracle/libwgen.so), or None when it has not been built."""
    global _wgen
    if _wgen is None:
        import ctypes
        import os
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwgen.so")
        if not os.path.exists(path):
            _wgen = False
        else:
            lib = ctypes.CDLL(path)
            lib.wgen_rows.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
            lib.wgen_rows.restype = ctypes.c_int
            _wgen = lib
    return _wgen or None


def stored_rows_c(cfg, name, layer=None, expert=None, rows=None, fmt=None):
    """stored_rows computed by the C generator (same definition, pinned
    bit-exactly against the numpy code in tests/test_oracle_wgen.py);
    fmt="raw" returns the unrounded values.  Requires libwgen.so."""
    lib = _c_generator()
    if lib is None:
        raise RuntimeError("oracle/libwgen.so is not built")
    n_out, n_in = tensor_shape(cfg, name)
    rows = np.arange(n_out, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    fmt = storage(cfg, name) if fmt is None else fmt
    code = 4 if fmt == "raw" else _FMT_CODE[fmt]
    out = np.empty((rows.size, n_in))
    aux = np.empty(rows.size * (n_in // 32 if code == 3 else 1))
    st = lib.wgen_rows(int(cfg["weight_seed"]) & 0xFFFFFFFFFFFFFFFF, tensor_id(cfg, name, layer, expert), n_in,
                       rows.ctypes.data, rows.size, code, out.ctypes.data, aux.ctypes.data)
    if st:
        raise ValueError(f"wgen_rows refused format {fmt} for {name}")
    if code == 2:
        return out, aux
    if code == 3:
        return out, aux.reshape(rows.size, n_in // 32).astype(np.int64)
    return out, None


def stored_rows(cfg, name, layer=None, expert=None, rows=None):
    """Stored values (as fp64) of selected rows, plus per-row fp8 scales.

    Returns (values, scales); scales is None unless the tensor is fp8, in which
    case values are the dequantised q*s and scales the bf16 row scales, or
    MXFP4, in which case scales are the block exponents [rows][K/32].
    Tensors stored in bf16, fp8 or MXFP4 are generated by the C version when
    it is built (bit-identical, much faster); fp32 tensors always take the
    numpy code below.
    """
    fmt = storage(cfg, name)
    if fmt != "f32" and _c_generator() is not None:
        return stored_rows_c(cfg, name, layer, expert, rows)
    w = raw_rows(cfg, name, layer, expert, rows)
    if fmt == "f32":
        return round_fp32(w), None
    if fmt == "bf16":
        return round_bf16(w), None
    if fmt == "mxfp4":
        return quantize_mxfp4(w)
    s = round_bf16(np.max(np.abs(w), axis=1) / E4M3_MAX)
    q = round_e4m3(w / s[:, None])
    return q * s[:, None], s


class Weights:
    """Lazily generated, cached stored weights of one model (fp64 values)."""

    def __init__(self, cfg, cache=True):
        self.cfg = cfg
        self.cache = cache
        self._cache = {}
        self.overrides = {}

    def get(self, name, layer=None, expert=None):
        key = (name, layer, expert)
        if key in self.overrides:
            return self.overrides[key]
        if key in self._cache:
            return self._cache[key]
        val = stored_rows(self.cfg, name, layer, expert)[0]
        if self.cache:
            self._cache[key] = val
        return val

    def rows(self, name, rows, layer=None, expert=None):
        """Selected rows only (large tensors such as the LM head)."""
        key = (name, layer, expert)
        if key in self.overrides:
            return self.overrides[key][np.asarray(rows)]
        if key in self._cache:
            return self._cache[key][np.asarray(rows)]
        return stored_rows(self.cfg, name, layer, expert, rows)[0]

    def set(self, name, value, layer=None, expert=None):
        """Replace a tensor (used by special-case test models)."""
        self.overrides[(name, layer, expert)] = np.asarray(value, dtype=np.float64)
