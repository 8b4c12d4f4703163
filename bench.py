#!/usr/bin/env python3
"""Throughput of the attention backward on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--mode atomic|deterministic]
                    [--workload headline_2x32x4096_causal] [--no-cpu-baseline]

A step is one full backward (prepare_workspace + the dot, main and reduce kernels) over one
batch of seeded synthetic input already resident in HBM.  Before the W counted warm-up steps,
untimed steps run for 0.3 s so that the GPU clocks have ramped up after the host-side input
preparation.  Prints one JSON line.

Workload: B=2, Hq=Hkv=32, S=4096, d=128, causal (top-left), BSHD, bf16 -- the B*H*S*d =
2*32*4096*128 causal shape the throughput target is quoted on.  Q, K, V, dO are N(0,1) draws
rounded to bf16; O and LSE (the forward's outputs, inputs of the backward) are prepared once,
untimed, with fp32 torch matrix products on the GPU.

FLOPs are counted as 2*(3*d_qk + 2*d_v) per allowed (query, key) pair (exact causal pair count),
i.e. 2.5 * 4 * B*H*S^2*d, halved for causal, up to the diagonal.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


# dQ accumulation modes: (deterministic flag, accumulator type)
MODE_ARGS = {"deterministic": (True, "fp32"), "atomic": (False, "fp32"), "atomic16": (False, "bf16")}
MODES = list(MODE_ARGS)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--mode", choices=MODES, default="deterministic")
    ap.add_argument("--workload", default="headline_2x32x4096_causal")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-mode", action="store_true",
                    help="time only --mode (profiling runs); by default both modes are timed")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the graded configurations reported beside the headline")
    ap.add_argument("--workload-steps", type=int, default=10,
                    help="timed steps per mode of each graded configuration")
    ap.add_argument("--bias", choices=["none", "11ss", "1hss", "b1ss", "bhss"], default="none",
                    help="add a seeded bf16 bias of this shape (and compute dbias)")
    ap.add_argument("--dropout", type=float, default=0.0, help="dropout probability (Philox)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (steps times), "
                         "the reference kernel for scaling HBM byte counters")
    return ap.parse_args()


def copy_probe(mib, steps):
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_mib": mib, "bytes_read_per_copy": n * 4,
                      "bytes_written_per_copy": n * 4, "copies": steps}))


def prepare_thd_inputs(w, device):
    """Ragged (THD) workload: seeded segment lengths (the workload's fixed prefix, then seed 3,
    uniform in [56, 2048]), seeded
    Q, K, V, dO [T, H, d] (bf16); O and LSE from the device forward.  Returns the tensors and
    the sequence-offset arguments of make_call."""
    import torch
    import attention_backward_fmha_amd as F
    from attention_backward_fmha_amd import inputs as I

    lens = I.ragged_lengths(3, w["total"], 56, 2048, prefix=w.get("prefix", ()))
    T, Hq, Hkv, dqk, dv = w["total"], w["Hq"], w["Hkv"], w["d_qk"], w["d_v"]
    x = I.draw(w["seed"], [(T, Hq, dqk), (T, Hkv, dqk), (T, Hkv, dv), (T, Hq, dv)], w["sigmas"])
    dev = {n: torch.from_numpy(x[n]).to(torch.bfloat16).to(device) for n in x}
    ss = I.seqstart(lens)
    seq = dict(cu_seqlens_q=torch.from_numpy(ss).to(device), cu_seqlens_k=torch.from_numpy(ss).to(device),
               cu_seqlens_q_host=ss, cu_seqlens_k_host=ss)
    scale = 1.0 / math.sqrt(dqk)
    o, lse = F.fwd(dev["q"], dev["k"], dev["v"], scale=scale, mask_type=w["mask"], **seq)
    torch.cuda.synchronize()
    return dev["q"], dev["k"], dev["v"], o, lse, dev["do"], scale, seq, lens


def prepare_inputs(w, device):
    """Seeded Q, K, V, dO (bf16) plus O, LSE of the forward computed on the GPU in fp32."""
    import torch
    from attention_backward_fmha_amd import inputs as I

    B, Hq, Hkv, Sq, Sk, dqk, dv = (w[k] for k in ("B", "Hq", "Hkv", "Sq", "Sk", "d_qk", "d_v"))
    x = I.draw(w["seed"], [(B, Sq, Hq, dqk), (B, Sk, Hkv, dqk), (B, Sk, Hkv, dv), (B, Sq, Hq, dv)],
               w["sigmas"])
    dev = {n: torch.from_numpy(x[n]).to(torch.bfloat16).to(device) for n in x}
    scale = 1.0 / math.sqrt(dqk)
    o = torch.empty((B, Sq, Hq, dv), dtype=torch.bfloat16, device=device)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=device)
    grp = Hq // Hkv
    mask = w["mask"]
    wl, wr = w.get("window", (-1, -1))
    delta = Sk - Sq if mask in (2, 3) else 0
    left, right = (-1, -1) if mask == 0 else ((-1, 0) if mask in (1, 2) else (wl, wr))
    i = torch.arange(Sq, device=device)[:, None]
    j = torch.arange(Sk, device=device)[None, :]
    allowed = torch.ones((Sq, Sk), dtype=torch.bool, device=device)
    if left >= 0:
        allowed &= j >= i + delta - left
    if right >= 0:
        allowed &= j <= i + delta + right
    for b in range(B):
        for h in range(Hq):
            qf = dev["q"][b, :, h, :].float().contiguous()
            kf = dev["k"][b, :, h // grp, :].float().contiguous()
            vf = dev["v"][b, :, h // grp, :].float().contiguous()
            s = (qf @ kf.t().contiguous()) * scale
            s = s.masked_fill(~allowed, float("-inf"))
            l = torch.logsumexp(s, dim=-1)
            p = torch.exp(s - l[:, None])
            p = torch.nan_to_num(p, nan=0.0)
            o[b, :, h, :] = (p @ vf).to(torch.bfloat16)
            lse[b, h, :] = l
    torch.cuda.synchronize()
    return dev["q"], dev["k"], dev["v"], o, lse, dev["do"], scale


# main-kernel name -> the source file that holds it
KERNEL_SOURCES = {"k_bwd_main": "kernels.hip", "k_bwd_wide": "kernels_wide.hip"}


def main_kernel_name(plan):
    """The main kernel a plan launches (plan.kernel: 1 four-wave layout, 2 wide layout)."""
    return "k_bwd_wide" if plan.kernel == 2 else "k_bwd_main"


def measured_traffic(kernel, workload, mode):
    """HBM bytes per launch of the main kernel from the committed rocprofv3 counter summary,
    or None when there is none or the kernel source changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "%s_%s_%s_traffic.txt" % (kernel, workload, mode))
    src = os.path.join(ROOT, "attention_backward_fmha_amd", "csrc", KERNEL_SOURCES[kernel])
    if not os.path.exists(path) or not os.path.exists(src):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k_, v_ = line.split(":", 1)
            fields[k_.strip()] = v_.strip()
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("kernel_source_sha256") != sha:
        return None
    return int(float(fields["read_bytes_per_launch"]) + float(fields["write_bytes_per_launch"]))


def cpu_baseline(w, budget_s):
    """The fp64 oracle on the host cores, on a bounded sample of the workload: single
    (batch, query head) problems of the same shape and mask, as many as fit the time budget."""
    import oracle
    from attention_backward_fmha_amd import inputs as I
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([t.get("num_threads", 1) for t in info] or [1])
        blas = ", ".join(sorted({"%s %s" % (t.get("internal_api", "?"), t.get("version", "")) for t in info
                                 if t.get("user_api") == "blas"})) or blas
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    Sq, Sk, dqk, dv = w["Sq"], w["Sk"], w["d_qk"], w["d_v"]
    x = I.draw(w["seed"] + 100, [(1, Sq, 1, dqk), (1, Sk, 1, dqk), (1, Sk, 1, dv), (1, Sq, 1, dv)],
               w["sigmas"])
    wl, wr = w.get("window", (-1, -1))
    pairs = int(oracle.allowed(w["mask"], wl, wr, Sq, Sk).sum())
    flops_per = 2.0 * (3 * dqk + 2 * dv) * pairs
    done = 0
    t0 = time.perf_counter()
    while True:
        oracle.backward(x["q"], x["k"], x["v"], x["do"], scale=1.0 / math.sqrt(dqk),
                        mask_type=w["mask"], window_left=wl, window_right=wr)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count()
    return {
        "value": flops_per * done / dt / 1e12,
        "unit": "TFLOP/s",
        # threads the oracle's BLAS ran with (its matrix products are the only parallel part),
        # never more than the cores this process may run on
        "cores": int(min(threads, avail)),
        "host_cores_available": int(avail),
        "cpu_model": cpu_model,
        "blas": blas,
        "kind": "oracle",
        "sample": "%d repetitions of one (batch, head) problem of the workload (Sq=%d, Sk=%d, d=%d, "
                  "same mask; the workload has %d such problems), fp64 numpy; each repetition "
                  "recomputes the forward (P, O, LSE) before the gradients, %.1f s"
                  % (done, Sq, Sk, dqk, w["B"] * w["Hq"], dt),
    }


# The graded configurations reported beside the headline: (workload, modes, timed steps).
# Each is timed in every dQ-accumulation mode it is run in; the 16384-token ones use fewer
# steps (about 8 ms each).
GRADED = [
    ("bshd_causal_2x16x2048", MODES, None),
    ("thd_gqa_llama3_8192", MODES, None),
    ("thd_gqa_llama3_8192_mixed", MODES, None),
    ("long_16384_causal_br", ("deterministic", "atomic"), 3),
    ("long_16384_window_4096", ("deterministic", "atomic"), 3),
    ("cross_192_128", MODES, None),
    ("cross_64", MODES, None),
]


def warm_up(step, min_seconds):
    """Untimed steps until the GPU has been busy for ``min_seconds`` (its clocks ramp up after
    the host-side input preparation; the first steps after it run measurably slower)."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_seconds:
        for _ in range(4):
            step(None)
        torch.cuda.synchronize()


def time_steps(step, stream, steps, warmup):
    """Mean ms per step over ``steps`` back-to-back steps after ``warmup`` untimed ones, with
    events on the launch stream only around the whole loop."""
    import torch
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        step(None)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def time_stages(step, stream, steps):
    """Mean ms of each stage (prepare, dot, main, reduce) from events recorded between the
    stages' launches on the launch stream."""
    import torch
    kev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    for s_ in range(steps):
        step(kev[s_])
    torch.cuda.synchronize()
    return [sum(e[i].elapsed_time(e[i + 1]) for e in kev) / steps for i in range(4)]


def make_step(call, ws, sh, stream):
    import attention_backward_fmha_amd as F

    def step(evs):
        rec = (lambda i: evs[i].record(stream)) if evs is not None else (lambda i: None)
        rec(0)
        call.prepare(ws, sh)
        rec(1)
        call.run(ws, sh, F.STAGE_DOT)
        rec(2)
        call.run(ws, sh, F.STAGE_MAIN)
        rec(3)
        call.run(ws, sh, F.STAGE_REDUCE)
        rec(4)
    return step


def stage_entry(w, m_plan, st):
    """Stage times with the achieved GB/s of the HBM-bound stages (algorithmic bytes)."""
    rows = int(m_plan.rows_q)
    dot_bytes = rows * w["Hq"] * (2 * w["d_v"] * 2 + 4) + rows * w["Hq"] * 8  # O, dO, LSE in; D, L out
    dq_bytes = rows * w["Hq"] * w["d_qk"] * 2
    red = m_plan.reduce_read_bytes + dq_bytes
    if m_plan.kv_parts > 1:  # fp32 dK/dV partials of every part in, bf16 dK/dV out
        red += m_plan.dkv_acc_bytes + m_plan.dkv_acc_bytes // (m_plan.kv_parts * 2)
    out_ = {"prepare_ms": round(st[0], 4), "dot_ms": round(st[1], 4), "main_ms": round(st[2], 4),
            "reduce_ms": round(st[3], 4),
            "dot_GBps": round(dot_bytes / (st[1] * 1e-3) / 1e9, 1),
            "reduce_GBps": round(red / (st[3] * 1e-3) / 1e9, 1),
            "reduce_bytes": int(red)}
    if m_plan.needs_zero:
        out_["prepare_GBps"] = round(m_plan.dq_acc_bytes / (st[0] * 1e-3) / 1e9, 1)
    return out_


def device_inputs(w, device):
    """Inputs of a graded workload: seeded Q, K, V, dO and the device forward's O and LSE."""
    import torch
    import attention_backward_fmha_amd as F
    from attention_backward_fmha_amd import inputs as I
    if "total" in w:
        return prepare_thd_inputs(w, device)
    B, Hq, Hkv, Sq, Sk, dqk, dv = (w[k] for k in ("B", "Hq", "Hkv", "Sq", "Sk", "d_qk", "d_v"))
    x = I.draw(w["seed"], [(B, Sq, Hq, dqk), (B, Sk, Hkv, dqk), (B, Sk, Hkv, dv), (B, Sq, Hq, dv)],
               w["sigmas"])
    dev = {n: torch.from_numpy(x[n]).to(torch.bfloat16).to(device) for n in x}
    del x
    scale = 1.0 / math.sqrt(dqk)
    o, lse = F.fwd(dev["q"], dev["k"], dev["v"], scale=scale, mask_type=w["mask"],
                   window=w.get("window", (-1, -1)))
    torch.cuda.synchronize()
    return dev["q"], dev["k"], dev["v"], o, lse, dev["do"], scale, {}, None


def graded_workload(name, modes, steps, warmup, device):
    """TFLOP/s, share of the bf16 peak, per-stage ms and the plan's split of one graded
    workload in each of ``modes``."""
    import torch
    import attention_backward_fmha_amd as F
    from attention_backward_fmha_amd import inputs as I
    w = I.WORKLOADS[name]
    q, k, v, o, lse, do, scale, seq, lens = device_inputs(w, device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream(device)
    out = {"segments": lens} if lens is not None else {}
    res = {}
    for mode in modes:
        det, acc = MODE_ARGS[mode]
        call = F.make_call(q, k, v, o, lse, do, dq, dk, dv, scale=scale, mask_type=w["mask"],
                           window=w.get("window", (-1, -1)), deterministic=det, dq_acc_dtype=acc, **seq)
        try:
            plan = call.plan()
        except F.FmhaError as e:  # e.g. the bf16 accumulator past its key-length bound
            res[mode] = {"unsupported": str(e)}
            continue
        ws = torch.empty(call.workspace_size(), dtype=torch.uint8, device=device)
        step = make_step(call, ws, stream.cuda_stream, stream)
        warm_up(step, 0.3)
        ms = time_steps(step, stream, steps, warmup)
        st = time_stages(step, stream, steps)
        out["flops_per_step"] = plan.flops
        tf = plan.flops / (ms * 1e-3) / 1e12
        res[mode] = {"tflops": round(tf, 2), "pct_of_bf16_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2),
                     "ms_per_step": round(ms, 4), "stages": stage_entry(w, plan, st),
                     "main_kernel": main_kernel_name(plan), "nsplits": plan.nsplits,
                     "tiles_per_item": plan.tiles_per_item, "kv_parts": plan.kv_parts,
                     "tile_m": plan.tile_m, "tile_n": plan.tile_n, "steps": steps}
        del ws
    out["modes"] = res
    del q, k, v, o, lse, do, dq, dk, dv
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (each GPU would run "
              "its own share of heads/segments independently); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib, args.steps)
        return
    import torch
    import attention_backward_fmha_amd as F
    from attention_backward_fmha_amd import inputs as I

    w = I.WORKLOADS[args.workload]
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    thd = "total" in w
    seq, lens = {}, None
    if thd:
        q, k, v, o, lse, do, scale, seq, lens = prepare_thd_inputs(w, device)
        if args.bias != "none":
            sys.exit("a bias needs a batch (BSHD) workload")
    else:
        q, k, v, o, lse, do, scale = prepare_inputs(w, device)
    extra = dict(seq)
    if args.bias != "none":
        bb = w["B"] if args.bias[0] == "b" else 1
        bh = w["Hq"] if args.bias[1] == "h" else 1
        gen = torch.Generator(device=device).manual_seed(77)
        bias = torch.randn((bb, bh, w["Sq"], w["Sk"]), generator=gen, device=device).to(torch.bfloat16)
        extra.update(bias=bias, dbias=torch.empty_like(bias))
    if args.dropout > 0:
        extra.update(dropout_p=args.dropout, philox_seed=1234, philox_offset=0)
    if args.bias != "none" or args.dropout > 0:  # O and LSE of the same forward (device, with bias/dropout)
        fkw = {n: extra[n] for n in extra if n not in ("dbias",)}
        o, lse = F.fwd(q, k, v, scale=scale, mask_type=w["mask"], window=w.get("window", (-1, -1)), **fkw)
        torch.cuda.synchronize()
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    stream = torch.cuda.current_stream(device)
    sh = stream.cuda_stream

    def time_mode(mode, headline):
        det, acc = MODE_ARGS[mode]
        call = F.make_call(q, k, v, o, lse, do, dq, dk, dv, scale=scale, mask_type=w["mask"],
                           window=w.get("window", (-1, -1)), deterministic=det, dq_acc_dtype=acc, **extra)
        plan = call.plan()
        ws = torch.empty(call.workspace_size(), dtype=torch.uint8, device=device)
        step = make_step(call, ws, sh, stream)
        warm_up(step, 0.3)  # GPU clocks up before the counted warm-up steps
        # the timed region: exactly args.steps whole steps, events only around the loop
        ms = time_steps(step, stream, args.steps, args.warmup)
        # stage breakdown in a separate pass (events between the stage launches)
        stage_ms = time_stages(step, stream, args.steps)
        cold = None
        if headline:
            # cold L2/MALL: overwrite a 512 MiB scratch (twice the MALL) before each step
            flush = torch.empty(512 << 20, dtype=torch.uint8, device=device)
            times = []
            for _ in range(min(args.steps, 10)):
                flush.fill_(1)
                a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a_.record(stream)
                step(None)
                b_.record(stream)
                torch.cuda.synchronize()
                times.append(a_.elapsed_time(b_))
            cold = sorted(times)[len(times) // 2]
            del flush
        del ws
        torch.cuda.empty_cache()
        return ms, stage_ms[2], plan, stage_ms, cold

    def time_forward(bwd_flops):
        """The device forward (fmha_fwd_run) on the same inputs, into scratch outputs."""
        o2 = torch.empty_like(o)
        lse2 = torch.empty_like(lse)
        fkw = {n: extra[n] for n in extra if n not in ("dbias",)}
        call = F.make_call(q, k, v, o2, lse2, None, None, None, None, scale=scale,
                           mask_type=w["mask"], window=w.get("window", (-1, -1)), **fkw)
        for _ in range(args.warmup):
            F._lib.fwd_run(call.args, sh)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(args.steps):
            F._lib.fwd_run(call.args, sh)
        t1.record(stream)
        torch.cuda.synchronize()
        f_ms = t0.elapsed_time(t1) / args.steps
        # forward FLOPs: S and P.V, 2*(d_qk + d_v) per allowed pair
        f_flops = bwd_flops * (w["d_qk"] + w["d_v"]) / (3 * w["d_qk"] + 2 * w["d_v"])
        return {"ms_per_call": round(f_ms, 4), "tflops": round(f_flops / (f_ms * 1e-3) / 1e12, 2),
                "pct_of_bf16_peak": round(100.0 * f_flops / (f_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}

    ms, main_ms, plan, stage_ms, cold_ms = time_mode(args.mode, True)
    runs = [(args.mode, ms, main_ms, plan, stage_ms)]
    if not args.only_mode:
        runs += [(m,) + time_mode(m, False)[:4] for m in MODES if m != args.mode]
    # host-side planning (validation, tiles, workspace map) per call
    pcall = F.make_call(q, k, v, o, lse, do, dq, dk, dv, scale=scale, mask_type=w["mask"],
                        window=w.get("window", (-1, -1)), deterministic=MODE_ARGS[args.mode][0],
                        dq_acc_dtype=MODE_ARGS[args.mode][1], **extra)
    t_p = time.perf_counter()
    for _ in range(200):
        pcall.workspace_size()
    plan_us = (time.perf_counter() - t_p) / 200 * 1e6
    flops = plan.flops
    tflops = flops / (ms * 1e-3) / 1e12
    main_tflops = flops / (main_ms * 1e-3) / 1e12
    modes = {}
    for mode, m_ms, m_main, m_plan, m_st in runs:
        modes[mode] = {"stages": stage_entry(w, m_plan, m_st),
            "value": round(flops / (m_ms * 1e-3) / 1e12, 2), "ms_per_step": round(m_ms, 4),
            "main_kernel": main_kernel_name(m_plan), "main_kernel_ms": round(m_main, 4),
            "nsplits": m_plan.nsplits, "tiles_per_item": m_plan.tiles_per_item,
            "kv_parts": m_plan.kv_parts}
    forward = time_forward(flops)
    kname = main_kernel_name(plan)

    out = {
        "metric": "FMHA bwd TFLOP/s and % of bf16 MFMA peak, B*H*S*d=2*32*4096*128 causal",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "B": len(lens) if thd else w["B"], "Hq": w["Hq"], "Hkv": w["Hkv"],
            "Sq": max(lens) if thd else w["Sq"], "Sk": max(lens) if thd else w["Sk"],
            "d_qk": w["d_qk"], "d_v": w["d_v"], "mask": w["mask"], "window": w.get("window"),
            "layout": "thd" if thd else "bshd", "segments": lens,
            "dq_accumulation": args.mode, "nsplits": plan.nsplits,
            "flops_per_step": flops, "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
            "cold_cache_ms_per_step": round(cold_ms, 4) if cold_ms else None,
            "cold_cache_tflops": round(flops / (cold_ms * 1e-3) / 1e12, 2) if cold_ms else None,
            "host_plan_us": round(plan_us, 2),
            "modes": modes,
            "bias": args.bias, "dbias": args.bias != "none", "dropout_p": args.dropout,
            "forward": forward,
        },
        "roofline": {
            "kernel": kname,
            "bound": "mfma",
            "achieved": round(main_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(main_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": None if (args.bias != "none" or args.dropout > 0)
            else measured_traffic(kname, args.workload, args.mode),
            "avg_launch_ms": round(main_ms, 4),
        },
    }
    del q, k, v, o, lse, do, dq, dk, dv, pcall
    extra.clear()
    torch.cuda.empty_cache()
    if not args.no_workloads:
        out["workloads"] = {}
        for name, wmodes, wsteps in GRADED:
            if name == args.workload:
                continue
            out["workloads"][name] = graded_workload(
                name, wmodes, wsteps or args.workload_steps, min(args.warmup, 2), device)
            print("workload %s done" % name, file=sys.stderr, flush=True)
    if not args.no_cpu_baseline and not thd:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
