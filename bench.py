"""Benchmark of the canvas denoise step on one MI355X.

Workload (default ``step_bf16``): 30 MoE decoder layers, d_model 2816,
16 query / 8 KV heads of 128, 128 experts top-8 (hidden 704) plus a shared
SwiGLU FFN (hidden 2112), vocabulary 262144, bf16 weights ~N(0, 0.02^2) from
seed 0, a committed 4096-token prefix KV cache built by causal prefill of
random ids, one 256-token canvas.  A step is one denoise pass: bidirectional
forward, LM head to fp32 logits, fused sampler (lock / re-noise / adaptive
stop) and the read-back of the stop flag.  Inputs are resident in HBM before
the timed region.

Prints one JSON line: steps/s (value), ms per step, committed tokens/s of a
full block (init, passes to the stop, commit), per-kernel times from HIP
events, the roofline of the dominant kernel, and the CPU oracle baseline on a
bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

import synth_inputs

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) read by the profiler."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def measured_copy_gbs(nbytes=1 << 30, reps=10):
    """Read+write bandwidth of a plain 1 GiB device-to-device copy on this
    GPU: the practical HBM ceiling the kernels are also compared against."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    return 2 * nbytes / (ms * 1e-3) / 1e9


def vendor_gemm(w, reps=96):
    """The vendor library's GEMM (torch.nn.functional.linear, hipBLASLt or
    rocBLAS as torch picks it) on the dense projection shapes of one canvas
    pass (256 rows), for comparison with the library's own launches.  Each
    shape is timed twice: 'cold' rotates over enough weight copies (at least
    1 GB) that every launch reads its weights from HBM, as every launch inside
    a denoise pass does (a pass streams about 50 GB); 'warm' reuses one weight
    matrix, which then stays in the 256 MB last-level cache.  Times are
    averages over back-to-back launches between two events."""
    import torch
    M = w["C"]
    shapes = {"qkv": ((w["Hq"] + 2 * w["Hkv"]) * w["dh"], w["d"]), "o_proj": (w["d"], w["Hq"] * w["dh"]),
              "shared_gate_up": (2 * w["fs"], w["d"]), "shared_down": (w["d"], w["fs"])}
    out = {"library": str(torch.backends.cuda.preferred_blas_library()), "rows": M}
    for name, (N, K) in shapes.items():
        x = torch.randn(M, K, device="cuda").to(torch.bfloat16)
        n_copies = max(24, -(-(1 << 30) // (N * K * 2)))
        ws = [torch.randn(N, K, device="cuda").to(torch.bfloat16) for _ in range(n_copies)]
        res = {"N": N, "K": K, "weight_mb": round(N * K * 2 / 1e6, 2), "copies": n_copies}
        for mode in ("cold", "warm"):
            for i in range(8):
                torch.nn.functional.linear(x, ws[i % n_copies if mode == "cold" else 0])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for i in range(reps):
                torch.nn.functional.linear(x, ws[i % n_copies if mode == "cold" else 0])
            e1.record()
            e1.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            res[f"{mode}_us"] = round(us, 2)
            res[f"{mode}_tbs"] = round(N * K * 2 / (us * 1e-6) / 1e12, 3)
        out[name] = res
        log(f"vendor gemm {name}: {res}")
        del ws, x
    torch.cuda.empty_cache()
    return out


def gpu_part(w, steps, warmup, prof_steps, do_block=True):
    import torch
    from block_text_diffusion_amd import binding as B
    from block_text_diffusion_amd.engine import Engine

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    C, L, E, k, R = w["C"], w["L"], w["E"], w["k"], w["R"]
    n_blocks = w.get("blocks", 1)
    eng = Engine(w, device=dev, max_ctx=w["P0"] + n_blocks * C)
    ctx = eng.ctx
    B.cd_synth_weights(ctx, w["weight_seed"])
    torch.cuda.synchronize()
    log(f"weights synthesized ({eng.weights.numel() / 1e9:.1f} GB)")
    # one untimed prefill first (the context's first launches create its side
    # stream and load the kernels), released again, so the timed prefills are
    # the steady state
    B.cd_prefill(ctx, 0, torch.from_numpy(synth_inputs.prefix_ids(w["V"], w["P0"], w["prefix_seed"], 0)).to(dev))
    B.cd_release(ctx, 0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in range(R):
        prefix = torch.from_numpy(synth_inputs.prefix_ids(w["V"], w["P0"], w["prefix_seed"], r)).to(dev)
        B.cd_prefill(ctx, r, prefix)
    torch.cuda.synchronize()
    prefill_ms = (time.perf_counter() - t0) * 1e3
    log(f"prefill of {R} x {w['P0']} tokens: {prefill_ms:.1f} ms")
    seed = w["gen_seed"]
    state = {"t": 0}

    def fresh():
        for r in range(R):
            B.cd_init_canvas(ctx, r, seed, 0)
        state["t"] = 0

    def one_step():
        if state["t"] >= w["max_steps"]:
            for r in range(R):
                B.cd_abort_canvas(ctx, r)
            fresh()
        B.cd_denoise_step(ctx, R, eng.info)
        info = B.cd_read_step_info(ctx, eng.info, R)          # the loop's stop-flag read-back
        state["t"] += 1
        if any(i.stop for i in info):
            state["t"] = w["max_steps"]                       # a stopped request takes no further pass
        return info

    fresh()
    for _ in range(warmup):
        one_step()
    torch.cuda.synchronize()
    step_ms = []
    t0 = time.perf_counter()
    for _ in range(steps):
        ts = time.perf_counter()
        one_step()                     # ends with the stop-flag read-back, so the pass is complete
        step_ms.append((time.perf_counter() - ts) * 1e3)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    log(f"timed {steps} steps: {el / steps * 1e3:.3f} ms/step")

    # per-kernel durations from HIP events recorded on the launch stream
    B.cd_profile(ctx, 1)
    for _ in range(prof_steps):
        one_step()
    torch.cuda.synchronize()
    prof = B.cd_profile_read(ctx)
    B.cd_profile(ctx, 0)

    # routing of one pass: experts actually streamed per layer
    T = R * C
    tid = torch.zeros(L, T, k, dtype=torch.int32, device=dev)
    tg = torch.zeros(L, T, k, dtype=torch.float32, device=dev)
    B.cd_set_trace(ctx, None, tid, tg)
    one_step()
    B.cd_set_trace(ctx)
    ids = tid.cpu().numpy()
    active = float(np.mean([len(np.unique(ids[l])) for l in range(L)]))
    counts = np.stack([np.bincount(ids[l].ravel(), minlength=E) for l in range(L)])
    route = {"max_tokens_per_expert": int(counts.max()),
             "mean_max_tokens_per_expert": float(counts.max(axis=1).mean()),
             "mean_row_tiles": float(np.mean([(np.ceil(c / 32)).sum() for c in counts]))}
    out = dict(elapsed=el, prof=prof, active=active, route=route, prefill_ms=prefill_ms, block_s=float("nan"),
               block_passes=0, blocks=[], device=torch.cuda.get_device_name(dev), step_ms=step_ms,
               copy_gbs=measured_copy_gbs())
    if not do_block:
        eng.close()
        return out
    # full blocks: every request starts a canvas, passes run until each request
    # has met its stop (at the latest all at the pass cap), then every request commits
    for r in range(R):
        B.cd_abort_canvas(ctx, r)
    ids_out = torch.empty(C, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    t_all = time.perf_counter()
    for b in range(n_blocks):
        t0 = time.perf_counter()
        for r in range(R):
            B.cd_init_canvas(ctx, r, seed, b)
        passes, stopped = 0, np.zeros(R, dtype=bool)
        while not stopped.all():
            B.cd_denoise_step(ctx, R, eng.info)
            infos = B.cd_read_step_info(ctx, eng.info, R)
            passes += 1
            stopped |= np.array([bool(i.stop) for i in infos])
        for r in range(R):
            B.cd_commit_block(ctx, r, ids_out)
        torch.cuda.synchronize()
        out["blocks"].append({"passes": passes, "ms": round((time.perf_counter() - t0) * 1e3, 2)})
    out["block_s"] = (time.perf_counter() - t_all) / n_blocks
    out["block_passes"] = out["blocks"][0]["passes"]
    log(f"{n_blocks} block(s) of passes + commit: {out['blocks']}")
    eng.close()
    return out


def measured_traffic(kernel_part):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, if that summary was taken on
    the current kernel source (else None)."""
    import hashlib
    import re
    root = os.path.dirname(os.path.abspath(__file__))
    prof = os.path.join(root, "profiles", f"expert_gemm_{kernel_part}_step_bf16.md")
    src = os.path.join(root, "block_text_diffusion_amd", "csrc", "k_gemm.hip")
    if not os.path.exists(prof):
        return None
    m = re.search(r"```json\n(\{.*?\})\n```", open(prof).read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    return rec["traffic_bytes_per_launch"] if rec.get("k_gemm_hip_sha256_16") == sha else None


def expert_bytes(w, active, part):
    """Algorithmic HBM bytes of one grouped expert GEMM launch: the weights of
    every expert that received tokens (bf16; fp8 plus fp32 row scales; MXFP4
    at half a byte per weight plus one scale byte per 32), the gathered bf16
    activation rows read and the output rows written."""
    T, k, d, fe = w["R"] * w["C"], w["k"], w["d"], w["fe"]
    wes = {"fp8": 1, "mxfp4": 0.5 + 1 / 32}.get(w["wdtype"], 2)
    scale = 4 if w["wdtype"] == "fp8" else 0
    if part == "gate_up":
        return active * (2 * fe * d * wes + 2 * fe * scale) + T * k * d * 2 + T * k * fe * 2
    return active * (d * fe * wes + d * scale) + T * k * fe * 2 + T * k * d * 2


def expert_flops(w, part):
    T, k, d, fe = w["R"] * w["C"], w["k"], w["d"], w["fe"]
    return 2 * T * k * d * (2 * fe if part == "gate_up" else fe)


def kernel_fractions(w, per, per_step):
    """MFMA fractions of the compute-shaped kernels at this workload against
    the bf16 dense peak (both run on the bf16 MFMA in every weight format):
    canvas attention and the LM head, from their event-timed durations."""
    R, C, L = w["R"], w["C"], w["L"]
    T = R * C
    nk = w["P0"] + C
    attn_fl = 4.0 * T * w["Hq"] * nk * w["dh"]                   # QK^T and PV per layer
    lm_fl = 2.0 * T * w["d"] * w["V"]
    out = {}
    t_attn = (per_step.get("attention", 0) + per_step.get("attn_merge", 0)) / L
    if t_attn > 0:
        out["attention_tflops"] = round(attn_fl / (t_attn * 1e-3) / 1e12, 1)
        out["attention_frac_bf16_peak"] = round(attn_fl / (t_attn * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
    if per.get("lm_head", 0) > 0:
        out["lm_head_tflops"] = round(lm_fl / (per["lm_head"] * 1e-3) / 1e12, 1)
        out["lm_head_frac_bf16_peak"] = round(lm_fl / (per["lm_head"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
    return out


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads(n):
    """A context limiting numpy's BLAS to n threads (threadpoolctl), or a no-op."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=n)
    except Exception:
        import contextlib
        return contextlib.nullcontext()


def cpu_baseline(w, active_experts):
    """The oracle, as it stands, timed on this host's cores (BLAS threads = the
    affinity set, and once more single-threaded):
    * the tiny fp32 model's whole loop (prefill, 48 passes, commit): passes/s;
    * the sampler on 256 x 262144 fp32 logits: ms per call;
    * the realistic-width bf16 step (the headline configuration), from exact
      work units with their weights generated before the timer: layer-0
      attention + router, 16 routed experts over their own rows, the shared
      FFN, the LM head on a 4096-row vocabulary slice, and the sampler,
      scaled by how often one step contains them (30 layers, the measured
      number of active experts per layer, 64 vocabulary slices)."""
    from oracle import loop, model, sampler
    from oracle.weights import Weights

    cores = len(os.sched_getaffinity(0))
    out = {"cores": cores, "cpu_model": _cpu_model()}

    # tiny model: the whole loop (weights generated before the timer)
    wt = synth_inputs.workload("tiny")
    Wt = Weights(wt)
    Wt.get("embed"); Wt.get("lm")
    for l in range(wt["L"]):
        for n in ("wq", "wk", "wv", "wo", "wr"):
            Wt.get(n, l)
        for e in range(wt["E"]):
            for n in ("wg", "wu", "wd"):
                Wt.get(n, l, e)
    pre = synth_inputs.prefix_ids(wt["V"], wt["P0"], wt["prefix_seed"])
    z = synth_inputs.sampler_logits(w["C"], w["V"], 1)
    for label, nt in (("", cores), ("_1thread", 1)):
        with _blas_threads(nt):
            t0 = time.perf_counter()
            _, blocks = loop.generate(wt, Wt, pre, 1, wt["gen_seed"])
            el = time.perf_counter() - t0
            out["tiny_loop_passes_per_s" + label] = round(blocks[0]["steps"] / el, 3)
            t0 = time.perf_counter()
            sampler.sample(w, z, 1, 1, 0, 0)
            out["sampler_ms_per_call" + label] = round((time.perf_counter() - t0) * 1e3, 1)

    # realistic-width step from work units, weights generated first
    W = Weights(w)
    rng = np.random.default_rng(0)
    C, d, dh, P0 = w["C"], w["d"], w["dh"], w["P0"]
    h = rng.standard_normal((C, d))
    Kp = rng.standard_normal((w["Hkv"], P0, dh)) * 0.3
    Vp = rng.standard_normal((w["Hkv"], P0, dh)) * 0.3
    pos = P0 + np.arange(C)
    n_exp, n_slice = 16, 4096
    for n in ("wq", "wk", "wv", "wo", "wr", "sg", "su", "sd"):
        W.get(n, 0)
    for e in range(n_exp):
        for n in ("wg", "wu", "wd"):
            W.get(n, 0, e)
    lm_rows = W.rows("lm", np.arange(n_slice))

    t0 = time.perf_counter()                       # attention half of a layer + router
    u = model.rmsnorm(h, w["eps"])
    q = model.rope((u @ W.get("wq", 0).T).reshape(C, w["Hq"], dh), pos, w["theta"])
    kk = model.rope((u @ W.get("wk", 0).T).reshape(C, w["Hkv"], dh), pos, w["theta"])
    vv = (u @ W.get("wv", 0).T).reshape(C, w["Hkv"], dh)
    K = np.concatenate([Kp, kk.transpose(1, 0, 2)], axis=1)
    V = np.concatenate([Vp, vv.transpose(1, 0, 2)], axis=1)
    o = model.attention(q, K, V).reshape(C, -1)
    h2 = h + o @ W.get("wo", 0).T
    u2 = model.rmsnorm(h2, w["eps"])
    ids, gates = model.topk_route(u2 @ W.get("wr", 0).T, w["k"])
    t_attn = time.perf_counter() - t0

    t0 = time.perf_counter()                       # routed experts 0..15, each over its own rows
    for e in range(n_exp):
        rows = np.nonzero(ids == e)[0]
        model.swiglu(u2[rows], W.get("wg", 0, e), W.get("wu", 0, e), W.get("wd", 0, e))
    t_expert = (time.perf_counter() - t0) / n_exp

    t0 = time.perf_counter()
    model.swiglu(u2, W.get("sg", 0), W.get("su", 0), W.get("sd", 0))
    t_shared = time.perf_counter() - t0

    t0 = time.perf_counter()                       # a vocabulary slice of the LM head
    model.rmsnorm(h2, w["eps"]) @ lm_rows.T
    t_lm = time.perf_counter() - t0

    t0 = time.perf_counter()
    sampler.sample(w, z, 1, 1, 0, 0)
    t_samp = time.perf_counter() - t0

    step_s = w["L"] * (t_attn + active_experts * t_expert + t_shared) + (w["V"] / n_slice) * t_lm + t_samp
    # the other configurations from the same units: a block of the four-block
    # generation at the 48-pass cap (48 passes plus the commit's forward, a
    # pass without the LM head and sampler), and one 32-request pass counted
    # for requests 0 and 31 only
    forward_s = w["L"] * (t_attn + active_experts * t_expert + t_shared)
    out["gen_block_s_from_units"] = round(48 * step_s + forward_s, 1)
    out["batch_pass_2_of_32_s_from_units"] = round(2 * step_s, 1)
    out.update({
        "value": round(1.0 / step_s, 6), "unit": "steps/s", "kind": "oracle",
        "sample": (f"fp64 numpy oracle on {cores} host cores ({out['cpu_model']}), weights generated before the "
                   f"timer; timed once each: layer-0 attention+router ({t_attn:.3f}s), {n_exp} routed experts over "
                   f"their rows ({t_expert * 1e3:.1f} ms each), shared FFN ({t_shared:.3f}s), LM head on {n_slice} "
                   f"of {w['V']} vocab rows ({t_lm:.3f}s), sampler on 256x{w['V']} ({t_samp:.2f}s); step = "
                   f"{w['L']}x(attn + {active_experts:.1f} active experts + shared) + {w['V'] // n_slice} LM slices "
                   f"+ sampler = {step_s:.1f}s. Also: the tiny fp32 model's whole loop and the sampler alone, with "
                   f"all cores and with one thread"),
    })
    return out


def prefill_flops(w, n):
    """Multiply-add FLOPs of a causal prefill of n tokens (all layers, no LM
    head): QKV, O, router, k experts and the shared FFN per token, and causal
    attention (query i sees i + 1 keys)."""
    d, dh, Hq, Hkv, k, fe, fs, E = w["d"], w["dh"], w["Hq"], w["Hkv"], w["k"], w["fe"], w["fs"], w["E"]
    per_tok = 2 * d * (Hq + 2 * Hkv) * dh + 2 * Hq * dh * d + 2 * d * E + k * 6 * d * fe + 6 * d * fs
    attn = 4 * Hq * dh * (n * (n + 1) // 2)
    return w["L"] * (n * per_tok + attn)


def prefill_line(w, ms_per_request):
    """Causal prefill of one prompt: tokens/s and MFMA rate against the bf16 peak."""
    n = w["P0"]
    if not n or not ms_per_request:
        return None
    tf = prefill_flops(w, n) / (ms_per_request * 1e-3) / 1e12
    return {"tokens": n, "ms": round(ms_per_request, 2), "tok_s": round(n / ms_per_request * 1e3, 1),
            "tflop": round(prefill_flops(w, n) / 1e12, 2), "tflops": round(tf, 1),
            "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}


def concurrency_sweep(w, counts):
    """Committed tok/s of one full block (canvas start, passes to the stop,
    commit) at several request counts, on one model: before each point the
    request state is cleared and every request gets its own prefix."""
    import torch
    from block_text_diffusion_amd import binding as B
    from block_text_diffusion_amd.engine import Engine

    dev = torch.device("cuda:0")
    C = w["C"]
    eng = Engine(w, device=dev, max_requests=max(counts), max_ctx=w["P0"] + C)
    ctx = eng.ctx
    B.cd_synth_weights(ctx, w["weight_seed"])
    ids_out = torch.empty(C, dtype=torch.int32, device=dev)
    out = []
    for R in counts:
        B.cd_reset(ctx)
        for r in range(R):
            B.cd_prefill(ctx, r, torch.from_numpy(synth_inputs.prefix_ids(w["V"], w["P0"], w["prefix_seed"], r)).to(dev))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for r in range(R):
            B.cd_init_canvas(ctx, r, w["gen_seed"], 0)
        passes, stopped = 0, np.zeros(R, dtype=bool)
        while not stopped.all():
            B.cd_denoise_step(ctx, R, eng.info)
            passes += 1
            stopped |= np.array([bool(i.stop) for i in B.cd_read_step_info(ctx, eng.info, R)])
        for r in range(R):
            B.cd_commit_block(ctx, r, ids_out)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3
        out.append({"requests": R, "passes": passes, "block_ms": round(ms, 1),
                    "ms_per_pass": round(ms / passes, 2), "committed_tok_s": round(R * C / ms * 1e3, 1)})
        log(f"sweep: {out[-1]}")
    eng.close()
    return out


def serve_queue(w, n_queue, n_slots, seed=12):
    """Committed tok/s of a queue served by cd_serve: prompts of 512..4096
    tokens and 1 or 2 blocks each (seeded), n_slots slots; wall time from
    the first prefill to the last commit."""
    import torch
    from block_text_diffusion_amd import binding as B
    from block_text_diffusion_amd.engine import Engine

    dev = torch.device("cuda:0")
    C = w["C"]
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(512, 4097, n_queue)]
    blocks = [int(x) for x in rng.integers(1, 3, n_queue)]
    eng = Engine(w, device=dev, max_requests=n_slots, max_ctx=4096 + 2 * C)
    B.cd_synth_weights(eng.ctx, w["weight_seed"])
    prefs = [torch.from_numpy(synth_inputs.prefix_ids(w["V"], n, w["prefix_seed"], q)).to(dev)
             for q, n in enumerate(lens)]
    out = torch.empty(sum(blocks) * C, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    steps = B.cd_serve(eng.ctx, prefs, blocks, [w["gen_seed"]] * n_queue, n_slots, out)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3
    eng.close()
    n_blk = sum(blocks)
    res = {"requests": n_queue, "slots": n_slots, "blocks": n_blk, "prompt_tokens": sum(lens),
           "passes_per_block": round(sum(sum(s) for s in steps) / n_blk, 2), "ms": round(ms, 1),
           "committed_tok_s": round(n_blk * C / ms * 1e3, 1)}
    log(f"serve: {res}")
    return res


def workload_line(name, w, g, steps, warmup, prof_steps):
    """The JSON fields of one measured workload from gpu_part's results."""
    ms = g["elapsed"] / steps * 1e3
    per = {k: (v[0] / v[1] if v[1] else 0.0) for k, v in g["prof"].items()}       # avg ms per launch
    per_step = {k: v[0] / prof_steps for k, v in g["prof"].items()}               # ms per step
    dom = max(("expert_gate_up", "expert_down"), key=lambda n: per_step[n])
    part = "gate_up" if dom == "expert_gate_up" else "down"
    byts = expert_bytes(w, g["active"], part)
    achieved = byts / (per[dom] * 1e-3) / 1e9
    R, C = w["R"], w["C"]
    gen = w.get("blocks", 1) > 1
    committed = (R * C / g["block_s"]) if g["block_passes"] else None
    wl = (f"{name}: {w['L']} MoE layers, d={w['d']}, {w['Hq']}/{w['Hkv']} heads x {w['dh']}, "
          f"{w['E']} experts top-{w['k']} (hidden {w['fe']}) + shared {w['fs']}, vocab {w['V']}, "
          f"{w['wdtype']} weights, {R} request(s) x prefix {w['P0']}, canvas {C}")
    if gen:
        wl += f", {w['blocks']} blocks"
    roof = {"kernel": f"grouped expert GEMM ({part.replace('_', '/')})", "bound": "hbm",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            # the counters were taken at step_bf16; a gen_bf16 pass runs the same launch shapes
            "traffic": measured_traffic(part) if name in ("step_bf16", "gen_bf16") else None,
            "bytes_per_launch": int(byts), "avg_launch_ms": round(per[dom], 5), "active_experts": g["active"],
            # the same bytes against the read+write rate of a plain 1 GiB copy on this GPU
            "measured_copy_gbs": round(g["copy_gbs"], 1), "frac_of_measured_copy": round(achieved / g["copy_gbs"], 4)}
    w8a8 = False
    if R * C * w["k"] / w["E"] >= 256:
        # many rows per expert: the grouped GEMM is bound by its MFMA pipe; with
        # fp8 weights it runs W8A8 on the fp8 MFMA (activations quantised per
        # row), with MXFP4 weights fp4 x fp8 on the block-scaled MFMA (whose
        # rate with one fp8 operand is the fp8 rate), else on the bf16 MFMA
        w8a8 = w["wdtype"] in ("fp8", "mxfp4")
        peak = FP8_PEAK_TFLOPS if w8a8 else BF16_PEAK_TFLOPS
        tf = expert_flops(w, part) / (per[dom] * 1e-3) / 1e12
        kind = {"fp8": ", fp8 x fp8", "mxfp4": ", fp4 x fp8 (block-scaled)"}.get(w["wdtype"], "")
        roof = {"kernel": roof["kernel"] + kind, "bound": "mfma", "achieved": round(tf, 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(tf / peak, 4), "traffic": None,
                "flops_per_launch": int(expert_flops(w, part)), "avg_launch_ms": round(per[dom], 5),
                "hbm_gbs": round(achieved, 1)}
    return {
        "value": round(committed, 3) if gen else round(1e3 / ms, 3),
        "unit": "committed tok/s" if gen else "steps/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        # arithmetic type: fp8 x fp8 MFMA for the QKV GEMM and the routed experts of
        # the W8A8 batch (fp4 x fp8 with MXFP4 experts), bf16 for everything else
        "dtype": "f32" if w["wdtype"] == "f32" else (
            ("fp8+fp4+bf16" if w["wdtype"] == "mxfp4" else "fp8+bf16") if w8a8 else "bf16"),
        "data": "synthetic",
        "config": {"workload": wl, "weights": w["wdtype"], "requests": R, "canvas": C, "prefix": w["P0"],
                   "blocks": w.get("blocks", 1)},
        "steps_per_s": round(1e3 / ms, 3),
        "canvas_tok_s": round(R * C * 1e3 / ms, 1),
        "committed_tok_s": round(committed, 2) if committed else None,
        "block_passes": g["block_passes"], "blocks": g["blocks"],
        "prefill_ms": round(g["prefill_ms"], 2),
        "prefill": prefill_line(w, g["prefill_ms"] / R),
        "roofline": roof,
        "ms_per_step_median": round(float(np.median(g["step_ms"])), 4),
        "ms_per_step_p95": round(float(np.percentile(g["step_ms"], 95)), 4),
        "kernel_fractions": kernel_fractions(w, per, per_step),
        "kernels_ms_per_step": {k: round(v, 4) for k, v in per_step.items() if v > 0},
        "routing": g["route"],
        "device": g["device"],
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--prof-steps", type=int, default=10)
    ap.add_argument("--workload", default="step_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-block", action="store_true", help="skip the full-block measurement")
    ap.add_argument("--no-extra", action="store_true",
                    help="step_bf16 only: skip the gen_bf16 and batch_fp8 lines added to the default run")
    ap.add_argument("--copy-calib", action="store_true", help="only run the byte-counter calibration copy")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only time the vendor library's GEMM on the dense projection shapes (cold and warm)")
    ap.add_argument("--sweep", action="store_true",
                    help="also time one full block at 1, 2, 4 and 32 requests (the 32-request fp8 model)")
    ap.add_argument("--serve", action="store_true",
                    help="also time a queue of 64 requests served on 32 slots (the fp8 model)")
    args = ap.parse_args()
    if args.copy_calib:
        copy_calibration()
        return
    if args.vendor_gemm:
        print(json.dumps({"vendor_gemm": vendor_gemm(synth_inputs.workload(args.workload))}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the canvas denoise step here runs on a single MI355X "
              "(multi-GPU sharding is a design note, not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    w = synth_inputs.workload(args.workload)
    g = gpu_part(w, args.steps, args.warmup, args.prof_steps, do_block=not args.no_block)
    line = {"metric": "canvas denoise steps/s + committed tok/s (256-tok block), % MFMA/HBM peak"}
    line.update(workload_line(args.workload, w, g, args.steps, args.warmup, args.prof_steps))
    if args.workload == "step_bf16" and not args.no_extra:
        # the other measured configurations, each timed the same way in this run
        for name, steps, warmup, prof, block in (("gen_bf16", 3, 1, 2, True), ("batch_fp8", 10, 2, 3, False)):
            log(f"extra workload {name}")
            we = synth_inputs.workload(name)
            ge = gpu_part(we, steps, warmup, prof, do_block=block)
            ex = workload_line(name, we, ge, steps, warmup, prof)
            for k in ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "data", "device",
                      "routing"):
                ex.pop(k, None)
            line[name] = ex
    if not args.no_cpu_baseline and args.workload == "step_bf16":
        log("cpu baseline (oracle sample)")
        line["cpu_baseline"] = cpu_baseline(w, g["active"])
    if args.sweep:
        line["concurrency_sweep"] = {"workload": "batch_fp8 model, one 256-token block per request after a "
                                                 f"{w['P0']}-token prefix",
                                     "points": concurrency_sweep(synth_inputs.workload("batch_fp8"), (1, 2, 4, 32))}
    if args.serve:
        line["serve_queue"] = {"workload": "batch_fp8 model, 64 queued requests (prompts 512..4096 tokens, 1 or 2 "
                                           "blocks each) on 32 slots, prefills included",
                               **serve_queue(synth_inputs.workload("batch_fp8"), 64, 32)}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
