#!/usr/bin/env python3
"""Benchmark of the GMA forward mixer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload I] [--no-cpu-baseline]

A step is one full forward (parameter prep, responsibilities, write and read -- or the
causal scan) over one batch of seeded synthetic inputs already resident in HBM.  W
untimed warm-up steps, then exactly K timed steps bracketed by torch.cuda.synchronize()
on both sides.  The same K steps are then run once more through gma_forward_timed, which
records a HIP event pair on the launch stream around every kernel; those events give each
kernel's average duration (the roofline's denominator), without their recording overhead
entering the headline time.  Prints one JSON line.

value = whole-job throughput in token-heads/s (B*H*N / seconds per step).  The
default workload is the bidirectional bf16 K=128 workload (B=8, H=8, N=4096,
d_r=d_v=64); the causal LM-shaped workload (B=16, H=8, N=2048, K=256) is measured the
same way and reported under "causal", the cross variant (1024 queries reading a
memory of 16384 keys per head, K=128) under "cross", the single-token causal decode
step at the causal workload's shape under "decode", the responsibility statistics of
that workload's key rows under "stats", and the backward of the headline and causal
workloads under "backward".
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 MFMA, TFLOP/s
FP32_VALU_PEAK_TFLOPS = 157.3


METRIC = "GMA forward tokens/s per head-layer; % of HBM/MFMA roofline (bidir+causal)"


def metric_name() -> str:
    return METRIC


def algorithmic(w, kernel: str):
    """Algorithmic bytes and flops of one launch of `kernel` on workload `w`, or None for
    a kernel that carries no algorithmic share (parameter prep, the causal segment totals
    and carries, the sum of the write kernel's split partials: workspace traffic and
    recompute, not work the method itself must do).

    Per token-head the whole forward must read q, k, v once and write out once:
    s*(2 d_r + 2 d_v) bytes; it must do 4K(2d_r+1) flops for the Q and K log-density
    contractions and 4K(d_v+1) for the write and read of [Vt | Z].  A kernel that does one
    part of that work is charged that part only.
    """
    s = 4 if w.dtype == "f32" else 2
    th = w.B * w.H * w.N          # query (and output) rows
    thk = w.B * w.H * w.Nk        # key (and value) rows; = th except in the cross variant
    K, dr, dv = w.K, w.d_r, w.d_v
    logits_side = 2 * K * (2 * dr + 1)   # one side's log-density contraction
    memory_side = 2 * K * (dv + 1)       # Gamma^T [V | 1] or Gamma [Vt | Z]
    if "prep" in kernel or "totals" in kernel or "carry" in kernel or "split_reduce" in kernel:
        return None
    if "causal_fused_scan" in kernel:  # the whole causal forward, responsibilities on chip
        return (th + thk) * s * (dr + dv), (th + thk) * (logits_side + memory_side)
    if "bidir_write" in kernel:   # reads k and v, forms Gamma_K and Gamma_K^T [V, 1]
        return thk * s * (dr + dv), thk * (logits_side + memory_side)
    if "bidir_read" in kernel:    # reads q, forms Gamma_Q, Gamma_Q [Vt, Z], writes out
        return th * s * (dr + dv), th * (logits_side + memory_side)
    if "causal_resp" in kernel:   # reads q and k, forms both responsibility maps
        return th * s * 2 * dr, th * 2 * logits_side
    if "causal_scan" in kernel:   # reads v, writes out: the prefix [S | z] write and read
        return th * s * 2 * dv, th * 2 * memory_side
    # the whole forward
    return (th + thk) * s * (dr + dv), (th + thk) * (logits_side + memory_side)


def hip_events(n):
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = (ctypes.c_void_p * n)()
    for i in range(n):
        e = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        evs[i] = e
    return hip, evs


def elapsed_ms(hip, a, b) -> float:
    t = ctypes.c_float(0.0)
    if hip.hipEventElapsedTime(ctypes.byref(t), a, b) != 0:
        raise RuntimeError("hipEventElapsedTime failed")
    return float(t.value)


# Sources the forward kernels (whose HBM traffic profiles/traffic.json records) are built
# and dispatched from; the backward, decode, statistics and SIMT files do not enter them.
FORWARD_SOURCES = ("gma_api.cpp", "gma_internal.h", "gma_mfma.hip", "gma_mfma_causal.hip", "gma_causal_fused.hip",
                   "gma_mfma_common.h", "gma_mfma_geo.h", "gma_numeric.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gaussian_mixture_sequence_resp_amd", "csrc")
    for f in FORWARD_SOURCES:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        table = json.load(open(p))
    except Exception:
        return None
    # a launch recorded under one name may run one of several kernel forms, which the
    # profiler names apart (gma_causal_resp: gma_causal_resp or gma_causal_resp_cp)
    forms = [k for k in table if k == f"{workload}:{kernel}" or k.startswith(f"{workload}:{kernel}_")]
    rec = table[forms[0]] if len(forms) == 1 else None
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def run_workload(w, steps, warmup, per_rep=True):
    import torch
    import gaussian_mixture_sequence_resp_amd as gma
    from gaussian_mixture_sequence_resp_amd.inputs import make_inputs

    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    d = {k: v.to(dev) for k, v in inp.items()}
    out = torch.empty((w.B, w.H, w.N, w.d_v), dtype=d["qr"].dtype, device=dev)
    desc = gma.make_desc(w.B, w.H, w.N, w.d_r, w.d_v, w.K, w.dtype, w.var_floor)
    cross = w.N_k is not None
    need = gma.workspace_size_cross(desc, w.Nk) if cross else gma.workspace_size(desc, w.causal)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    max_k = 24
    hip, evs = hip_events(2 * max_k * steps)
    names = (ctypes.c_char_p * max_k)()

    fwd = gma.forward_cross if cross else gma.forward
    kw = {} if cross else {"causal": w.causal}

    def step(i=None):
        if i is None:
            fwd(d["qr"], d["kr"], d["v"], d["mu"], d["var_raw"], d["prior_logits"], eps=w.eps,
                var_floor=w.var_floor, out=out, workspace=ws, stream=stream, **kw)
            return
        sub = (ctypes.c_void_p * (2 * max_k)).from_buffer(evs, ctypes.sizeof(ctypes.c_void_p) * 2 * max_k * i)
        fwd(d["qr"], d["kr"], d["v"], d["mu"], d["var_raw"], d["prior_logits"], eps=w.eps,
            var_floor=w.var_floor, out=out, workspace=ws, stream=stream, events=sub, names=names, **kw)

    for _ in range(warmup):
        step()
    # timed region: exactly `steps` plain forwards (no instrumentation)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # the same `steps` forwards again through gma_forward_timed: a HIP event pair on the
    # launch stream around every kernel gives each kernel's duration
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    nk = fwd.last_kernel_count
    per_kernel = {}
    for j in range(min(nk, max_k)):
        name = names[j].decode()
        ts = [elapsed_ms(hip, evs[2 * max_k * i + 2 * j], evs[2 * max_k * i + 2 * j + 1]) for i in range(steps)]
        # a kernel launched several times per forward (one launch per slab of heads) counts once
        # per step with the sum of its launches
        per_kernel[name] = per_kernel.get(name, 0.0) + sum(ts) / len(ts)
    for e in evs:
        hip.hipEventDestroy(e)
    cold = rep_timing(step, torch, dev) if per_rep else None
    return {"ms_per_step": (t1 - t0) * 1e3 / steps,
            "ms_per_step_with_events": (t3 - t2) * 1e3 / steps,
            "per_kernel_ms": per_kernel,
            "per_rep": cold,
            "workspace_bytes": need,
            "inputs": inp}


def device_peaks():
    """Practical peaks of this device under load, next to the datasheet ones: the bf16 MFMA
    rate of a register-only loop of the instruction the GMA kernels use (libgma_probe.so), and
    the HBM bandwidth of a plain 1 GiB device-to-device copy (read + write bytes)."""
    import torch
    dev = torch.device("cuda:0")
    probe = ctypes.CDLL(os.path.join(ROOT, "gaussian_mixture_sequence_resp_amd", "libgma_probe.so"))
    probe.gma_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    probe.gma_probe_mfma.restype = ctypes.c_int
    blocks, iters = 2048, 2048
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def mfma():
        rc = probe.gma_probe_mfma(blocks, iters, out.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"gma_probe_mfma failed: {rc}")

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    flops = blocks * 4 * iters * 4 * 32 * 32 * 16 * 2
    tf = flops / timed(mfma) / 1e12
    probe.gma_probe_mfma_lds.argtypes = probe.gma_probe_mfma.argtypes
    probe.gma_probe_mfma_lds.restype = ctypes.c_int

    def mfma_lds():
        rc = probe.gma_probe_mfma_lds(blocks, iters, out.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"gma_probe_mfma_lds failed: {rc}")

    tf_lds = flops / timed(mfma_lds) / 1e12
    probe.gma_probe_mfma_lds2.argtypes = probe.gma_probe_mfma.argtypes
    probe.gma_probe_mfma_lds2.restype = ctypes.c_int

    def mfma_lds2():
        rc = probe.gma_probe_mfma_lds2(blocks, iters, out.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"gma_probe_mfma_lds2 failed: {rc}")

    tf_lds2 = flops / timed(mfma_lds2) / 1e12
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    gbs = 2 * src.numel() / timed(lambda: dst.copy_(src)) / 1e9
    del src, dst, out
    return {"mfma_bf16_tflops": round(tf, 1), "mfma_bf16_lds_operand_tflops": round(tf_lds, 1),
            "mfma_bf16_lds_both_operands_tflops": round(tf_lds2, 1),
            "hbm_copy_gbs": round(gbs, 1),
            "datasheet": {"mfma_bf16_tflops": BF16_PEAK_TFLOPS, "hbm_gbs": HBM_PEAK_GBS},
            "note": "register-only loop of v_mfma_f32_32x32x16_bf16 (4 accumulators per wave, 8192 waves); "
                    "the same loop with each MFMA's A operand read from LDS (1 KB per wave per MFMA), and with both "
                    "operands read from LDS (2 KB); "
                    "1 GiB device copy, read + write bytes"}


def rep_timing(step, torch, dev, reps=100, warmup=10, flush_bytes=512 << 20):
    """Per-rep timing: `warmup` untimed reps, then `reps` reps each timed alone with an event
    pair on the launch stream, (a) cold: a 512 MiB scratch buffer written before each rep
    (outside the timed pair) so that the 256 MB Infinity Cache holds none of the inputs,
    (b) warm: back to back.  Returns median, p10 and p90 of each, in ms."""
    import statistics
    scratch = torch.empty(flush_bytes // 4, dtype=torch.float32, device=dev)
    for _ in range(warmup):
        step()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        scratch.fill_(1.0)
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    cold = sorted(a.elapsed_time(b) for a, b in ev)
    for a, b in ev:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    warm = sorted(a.elapsed_time(b) for a, b in ev)

    def q(x, f):
        return round(x[min(len(x) - 1, int(f * len(x)))], 5)
    return {"reps": reps, "cold_median_ms": round(statistics.median(cold), 5), "cold_p10_ms": q(cold, 0.1),
            "cold_p90_ms": q(cold, 0.9), "warm_median_ms": round(statistics.median(warm), 5),
            "warm_p10_ms": q(warm, 0.1), "warm_p90_ms": q(warm, 0.9),
            "flush": "512 MiB scratch fill before each cold rep, outside the timed pair"}


def roofline_for(w, per_kernel):
    """Roofline of the dominant kernel: the longest one that carries an algorithmic share."""
    name = max((k for k in per_kernel if algorithmic(w, k) is not None), key=per_kernel.get)
    ms = per_kernel[name]
    nbytes, nflops = algorithmic(w, name)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    peak_flops = (FP32_VALU_PEAK_TFLOPS if w.dtype == "f32" else BF16_PEAK_TFLOPS) * 1e12
    t_mfma = nflops / peak_flops
    if t_hbm >= t_mfma:
        ach = nbytes / (ms * 1e-3) / 1e9
        rl = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
              "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        ach = nflops / (ms * 1e-3) / 1e12
        pk = FP32_VALU_PEAK_TFLOPS if w.dtype == "f32" else BF16_PEAK_TFLOPS
        rl = {"bound": "mfma", "achieved": round(ach, 3), "peak": pk, "unit": "TFLOP/s",
              "frac": round(ach / pk, 4)}
    rl["kernel"] = name
    rl["kernel_ms"] = round(ms, 5)
    rl["traffic"] = traffic_from_profiles(name, w.name)
    return rl


TARGET_FRAC = 0.6  # the whole forward's target share of its binding roofline


def step_roofline(w, ms):
    """The whole forward (one step, ms) against its binding roofline: algorithmic bytes at
    8 TB/s or algorithmic flops at the dense bf16 MFMA peak, whichever takes longer."""
    nbytes, nflops = algorithmic(w, "step")
    sec = ms * 1e-3
    hbm = nbytes / sec / (HBM_PEAK_GBS * 1e9)
    mfma = nflops / sec / (BF16_PEAK_TFLOPS * 1e12)
    t_hbm, t_mfma = nbytes / (HBM_PEAK_GBS * 1e9), nflops / (BF16_PEAK_TFLOPS * 1e12)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    frac = hbm if bound == "hbm" else mfma
    return {"hbm_frac": round(hbm, 4), "mfma_frac": round(mfma, 4), "bound": bound, "frac": round(frac, 4),
            "target_frac": TARGET_FRAC, "roofline_ms": round(max(t_hbm, t_mfma) * 1e3, 5),
            "target_ms": round(max(t_hbm, t_mfma) / TARGET_FRAC * 1e3, 5)}


def run_decode(w, steps, warmup):
    """Single-token causal decode at workload w's (B, H, K, d) shape: the memory of a
    prefix of w.N positions (gma_memory, timed on its own as the prefill), then decode steps
    over every (b, h), each one kernel: gma_decode_step on the raw parameters and
    gma_decode_step_prepared on parameters prepared once (gma_decode_prepare, timed on its
    own).  The steps of each kind are captured in one HIP graph of `steps` launches and
    replayed, as a serving loop would run them: the per-step time is the GPU's, not the
    Python binding's.  Returns ms per step of each kind, the prefill's and the preparation's
    ms, and the bytes a step must move."""
    import torch
    import gaussian_mixture_sequence_resp_amd as gma
    from gaussian_mixture_sequence_resp_amd.inputs import make_inputs

    inp = make_inputs(w.with_(N=w.N + steps))
    dev = torch.device("cuda:0")
    d = {k: v.to(dev) for k, v in inp.items()}
    kp, vp = d["kr"][:, :, :w.N].contiguous(), d["v"][:, :, :w.N].contiguous()
    state = torch.empty((w.B, w.H, w.K, w.d_v + 1), dtype=torch.float32, device=dev)
    mdesc = gma.make_desc(w.B, w.H, w.N, w.d_r, w.d_v, w.K, w.dtype, w.var_floor)
    mws = torch.empty(max(int(gma.load_library().gma_memory_workspace_size(ctypes.byref(mdesc))), 1),
                      dtype=torch.uint8, device=dev)

    def prefill():
        gma.memory(kp, vp, d["mu"], d["var_raw"], d["prior_logits"], var_floor=w.var_floor, state=state,
                   workspace=mws)

    def timed(f, reps):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            f()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / reps

    prefill_ms = timed(prefill, 5)
    params = [None]

    def prepare():
        params[0] = gma.decode_prepare(d["mu"], d["var_raw"], d["prior_logits"], dtype=w.dtype,
                                       var_floor=w.var_floor)

    prepare_ms = timed(prepare, 5)
    rows = [(d["qr"][:, :, t].contiguous(), d["kr"][:, :, t].contiguous(), d["v"][:, :, t].contiguous())
            for t in range(w.N, w.N + steps)]
    out = torch.empty((w.B, w.H, 1, w.d_v), dtype=d["qr"].dtype, device=dev)

    def raw_step(i):
        q, k, v = rows[i]
        gma.decode_step(q, k, v, d["mu"], d["var_raw"], d["prior_logits"], state, eps=w.eps,
                        var_floor=w.var_floor, out=out)

    def prepared_step(i):
        q, k, v = rows[i]
        gma.decode_step_prepared(q, k, v, params[0], state, eps=w.eps, out=out)

    res = {}
    for name, step in (("raw", raw_step), ("prepared", prepared_step)):
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            for i in range(min(steps, max(warmup, 3))):
                step(i)
        torch.cuda.current_stream(dev).wait_stream(side)
        prefill()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                step(i)
        graph.replay()  # warm
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / (reps * steps)
    # state read and written once per step, plus this position's q, k, v and out
    s = 4 if w.dtype == "f32" else 2
    nbytes = w.B * w.H * (2 * 4 * w.K * (w.d_v + 1) + s * (2 * w.d_r + 2 * w.d_v))
    return {"ms_per_step": res["prepared"], "raw_ms_per_step": res["raw"], "bytes_per_step": nbytes,
            "prefill_ms": prefill_ms, "prepare_ms": prepare_ms}


def run_stats(w, steps, warmup):
    """Responsibility statistics (gma_resp_stats: hard assignments, counts, soft usage, used,
    entropy) of the key rows of workload w, one call per step; returns ms per call and the
    call's algorithmic bytes and flops (one side's log-density; x read, hard written)."""
    import torch
    import gaussian_mixture_sequence_resp_amd as gma
    from gaussian_mixture_sequence_resp_amd.inputs import make_inputs

    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    d = {k: inp[k].to(dev) for k in ("kr", "mu", "var_raw", "prior_logits")}
    desc = gma.make_desc(w.B, w.H, w.N, w.d_r, 1, w.K, w.dtype, w.var_floor)
    ws = torch.empty(max(int(gma.load_library().gma_stats_workspace_size(ctypes.byref(desc))), 1),
                     dtype=torch.uint8, device=dev)

    def call():
        return gma.resp_stats(d["kr"], d["mu"], d["var_raw"], d["prior_logits"], var_floor=w.var_floor,
                              workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    s = 4 if w.dtype == "f32" else 2
    th = w.B * w.H * w.N
    return {"ms_per_call": ms, "bytes": th * (s * w.d_r + 4), "flops": th * 2 * w.K * (2 * w.d_r + 1)}


def run_backward(w, steps, warmup):
    """Backward (gma_backward: gradients of qr, kr, v, mu, var_raw, prior logits) of workload
    w with a seeded dO, one call per step; ms per call and the call's algorithmic bytes
    (read q, k, v, dO; write dq, dk, dv) and flops (twice the forward's: the recomputed
    forward, then the same contractions transposed)."""
    import torch
    import gaussian_mixture_sequence_resp_amd as gma
    from gaussian_mixture_sequence_resp_amd.inputs import make_inputs

    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    d = {k: v.to(dev) for k, v in inp.items()}
    g = torch.Generator().manual_seed(w.seed + 7)
    dout = torch.randn(w.B, w.H, w.N, w.d_v, generator=g).to(d["v"].dtype).to(dev)
    desc = gma.make_desc(w.B, w.H, w.N, w.d_r, w.d_v, w.K, w.dtype, w.var_floor)
    ws = torch.empty(max(int(gma.load_library().gma_backward_workspace_size(ctypes.byref(desc), int(w.causal))), 1),
                     dtype=torch.uint8, device=dev)

    def call():
        return gma.backward(d["qr"], d["kr"], d["v"], d["mu"], d["var_raw"], d["prior_logits"], dout, w.causal,
                            eps=w.eps, var_floor=w.var_floor, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    s = 4 if w.dtype == "f32" else 2
    th = w.B * w.H * w.N
    nbytes = th * s * 2 * (2 * w.d_r + 2 * w.d_v)
    _, fwd_flops = algorithmic(w, "step")
    return {"ms_per_call": ms, "bytes": nbytes, "flops": 2 * fwd_flops}


def cpu_baseline(w, inp, budget_s=12.0):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload (whole batch
    elements, all heads of each), timed on this host's cores.  The oracle spreads its
    (b, h) slices over OpenMP threads, so the threads used are min(threads, slices)."""
    import oracle
    threads = oracle.num_threads()

    def run(nb, nh=None):
        nh = w.H if nh is None else nh
        t = time.perf_counter()
        oracle.forward(inp["qr"][:nb, :nh], inp["kr"][:nb, :nh], inp["v"][:nb, :nh],
                       inp["mu"][:nh], inp["var_raw"][:nh], inp["prior_logits"][:nh],
                       w.causal, w.eps, w.var_floor)
        return time.perf_counter() - t

    per_slice = max(run(1, 1), 1e-6)          # one (b, h) slice on one thread
    waves = max(1, int(budget_s / per_slice))  # slices each thread can do in the budget
    nb = int(min(w.B, max(1, (waves * threads) // w.H)))
    t = run(nb)
    reps = 1
    if t < 10.0:                               # short: the median of three runs
        t = sorted([t, run(nb), run(nb)])[1]
        reps = 3
    n = nb * w.H
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(n * w.N / t, 1), "unit": "token-heads/s", "cores": min(threads, n),
            "kind": "oracle", "cpu_model": model,
            "sample": f"{nb} of {w.B} batch elements x {w.H} heads x N={w.N} "
                      f"(fp64 C oracle, OpenMP over (b,h) slices, {t:.2f} s, "
                      f"{'median of 3 runs' if reps == 3 else 'one run'})"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-causal", action="store_true")
    ap.add_argument("--no-cross", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-stats", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-per-rep", action="store_true",
                    help="skip the per-rep (cold / warm) timing, e.g. under a profiler whose kernel "
                         "averages should cover the timed steps only")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the device peak probes (MFMA loop, 1 GiB copy)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the measurement, copy one 256 MiB device buffer, so that a profiler's "
                         "memory counters can be scaled by a copy of known size")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the lines of the other forward workloads (tiny, causal LM, long bidirectional, "
                         "long causal)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the GMA forward here has no multi-GPU path "
              "(its (b, h) slices would shard across GPUs with no communication). Run --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    from gaussian_mixture_sequence_resp_amd.inputs import WORKLOADS
    w = WORKLOADS[args.workload]
    pr = not args.no_per_rep
    r = run_workload(w, args.steps, args.warmup, pr)
    th = w.token_heads
    # headline: the cache-flushed (cold) per-rep median when measured, else the timed loop
    value_ms = r["per_rep"]["cold_median_ms"] if r["per_rep"] else r["ms_per_step"]
    value = th / (value_ms * 1e-3)
    line = {
        "metric": metric_name(),
        "value": round(value, 1),
        "value_basis": ("median of 100 single forwards, each after a 512 MiB cache flush (Infinity Cache "
                        "holds none of the inputs); ms_per_step is the back-to-back timed loop"
                        if r["per_rep"] else "the timed loop (ms_per_step)"),
        "value_ms": round(value_ms, 5),
        "warm_value": round(th / (r["ms_per_step"] * 1e-3), 1),
        "unit": "token-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normal draws, see gaussian_mixture_sequence_resp_amd/inputs.py)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d_r": w.d_r, "d_v": w.d_v,
                   "K": w.K, "causal": w.causal, "global_batch": w.B, "seq_len": w.N,
                   "parallelism": "none (1 GPU)"},
        "ms_per_step_with_events": round(r["ms_per_step_with_events"], 5),
        "per_kernel_ms": {k: round(v, 5) for k, v in r["per_kernel_ms"].items()},
        "per_rep": r["per_rep"],
        "workspace_bytes": r["workspace_bytes"],
        "roofline": roofline_for(w, r["per_kernel_ms"]),
    }
    line["step_roofline"] = step_roofline(w, value_ms)
    if not args.no_configs and args.workload == 2:
        # every other forward workload, each measured the same way (its own line inside this one)
        line["configs"] = {}
        for ci in (1, 3, 4, 5):
            wc = WORKLOADS[ci]
            st = max(5, args.steps // 2)
            rc = run_workload(wc, st, max(2, args.warmup // 2), pr)
            vm = rc["per_rep"]["cold_median_ms"] if rc["per_rep"] else rc["ms_per_step"]
            ent = {"workload": wc.name, "B": wc.B, "H": wc.H, "N": wc.N, "d_r": wc.d_r, "d_v": wc.d_v, "K": wc.K,
                   "causal": wc.causal, "dtype": wc.dtype, "steps": st,
                   "value": round(wc.token_heads / (vm * 1e-3), 1), "unit": "token-heads/s",
                   "value_ms": round(vm, 5), "ms_per_step": round(rc["ms_per_step"], 5),
                   "per_kernel_ms": {k: round(v, 5) for k, v in rc["per_kernel_ms"].items()},
                   "per_rep": rc["per_rep"]}
            if ci == 1:
                ent["roofline"] = {"bound": "latency", "note": "64 kB and 0.4 MFLOP of algorithmic work: "
                                   "launch-latency bound, exempt from the roofline target"}
            else:
                ent["roofline"] = roofline_for(wc, rc["per_kernel_ms"])
                ent["step_roofline"] = step_roofline(wc, vm)
            if not args.no_cpu_baseline:
                ent["cpu_baseline"] = cpu_baseline(wc, rc["inputs"], budget_s=6.0)
            line["configs"][wc.name] = ent
    if not args.no_causal and args.workload == 2:
        wc = WORKLOADS[3]
        if "configs" in line:  # measured above: the causal line is that entry
            line["causal"] = line["configs"][wc.name]
        else:
            rc = run_workload(wc, max(5, args.steps // 2), max(2, args.warmup // 2), pr)
            vm = rc["per_rep"]["cold_median_ms"] if rc["per_rep"] else rc["ms_per_step"]
            line["causal"] = {"workload": wc.name, "ms_per_step": round(rc["ms_per_step"], 5),
                              "value": round(wc.token_heads / (vm * 1e-3), 1), "value_ms": round(vm, 5),
                              "per_kernel_ms": {k: round(v, 5) for k, v in rc["per_kernel_ms"].items()},
                              "per_rep": rc["per_rep"],
                              "roofline": roofline_for(wc, rc["per_kernel_ms"]),
                              "step_roofline": step_roofline(wc, vm)}
    if not args.no_cross and args.workload == 2:
        wx = WORKLOADS[6]
        rx = run_workload(wx, max(5, args.steps // 2), max(2, args.warmup // 2), pr)
        sec = rx["ms_per_step"] * 1e-3
        line["cross"] = {"workload": wx.name, "N_q": wx.N, "N_k": wx.Nk, "ms_per_step": round(rx["ms_per_step"], 5),
                         "value": round(wx.B * wx.H * wx.N / sec, 1), "unit": "query token-heads/s",
                         "key_token_heads_per_s": round(wx.B * wx.H * wx.Nk / sec, 1),
                         "per_kernel_ms": {k: round(v, 5) for k, v in rx["per_kernel_ms"].items()},
                         "roofline": roofline_for(wx, rx["per_kernel_ms"])}
    if not args.no_decode and args.workload == 2:
        wd = WORKLOADS[3]
        rd = run_decode(wd, max(20, args.steps), max(5, args.warmup))
        sec = rd["ms_per_step"] * 1e-3
        line["decode"] = {"workload": f"{wd.name} decode (prefix {wd.N}, one position per step)",
                          "us_per_step": round(rd["ms_per_step"] * 1e3, 2),
                          "step": "gma_decode_step_prepared, steps replayed from one HIP graph",
                          "raw_parameters_us_per_step": round(rd["raw_ms_per_step"] * 1e3, 2),
                          "prepare_ms": round(rd["prepare_ms"], 4),
                          "prefill_ms": round(rd["prefill_ms"], 4),
                          "prefill_token_heads_per_s": round(wd.B * wd.H * wd.N / (rd["prefill_ms"] * 1e-3), 1),
                          "value": round(wd.B * wd.H / sec, 1), "unit": "token-heads/s",
                          "roofline": {"bound": "hbm", "achieved": round(rd["bytes_per_step"] / sec / 1e9, 2),
                                       "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": round(rd["bytes_per_step"] / sec / 1e9 / HBM_PEAK_GBS, 4),
                                       "note": "whole step (one kernel, graph replay); latency-bound"}}
    if not args.no_stats and args.workload == 2:
        ws_ = WORKLOADS[3]
        rs = run_stats(ws_, max(10, args.steps // 2), max(3, args.warmup // 2))
        sec = rs["ms_per_call"] * 1e-3
        tf = rs["flops"] / sec / 1e12
        line["stats"] = {"workload": f"{ws_.name} key rows: responsibility statistics (hard assignments, counts, "
                                     "soft usage, components used, usage entropy)",
                         "ms_per_call": round(rs["ms_per_call"], 5),
                         "value": round(ws_.B * ws_.H * ws_.N / sec, 1), "unit": "token-heads/s",
                         "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS,
                                      "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                                      "note": "whole call (prep, responsibilities, usage, finish) against the "
                                              "log-density flops of one side"}}
    if not args.no_backward and args.workload == 2:
        bl = {}
        for wb in (w, WORKLOADS[3]):
            rb = run_backward(wb, 2, 1)
            sec = rb["ms_per_call"] * 1e-3
            tf = rb["flops"] / sec / 1e12
            bl[wb.name] = {"ms_per_call": round(rb["ms_per_call"], 4),
                           "value": round(wb.B * wb.H * wb.N / sec, 1), "unit": "token-heads/s",
                           "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": BF16_PEAK_TFLOPS,
                                        "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 6),
                                        "note": "whole call against twice the forward's algorithmic flops"}}
        line["backward"] = bl
    if not args.no_peaks:
        pk = device_peaks()
        line["device_peaks"] = pk
        rls = [line["roofline"]] + [line[k]["roofline"] for k in ("causal", "cross") if k in line]
        rls += [e["roofline"] for e in line.get("configs", {}).values() if e["roofline"] not in rls]
        for rl in rls:
            m = pk["hbm_copy_gbs"] if rl["bound"] == "hbm" else pk["mfma_bf16_tflops"]
            if rl["bound"] in ("hbm", "mfma") and rl["peak"] in (HBM_PEAK_GBS, BF16_PEAK_TFLOPS):
                rl["frac_of_measured_peak"] = round(rl["achieved"] / m, 4)
    if args.copy_calibration:
        import torch
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = src.numel()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, r["inputs"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
