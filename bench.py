#!/usr/bin/env python3
"""Benchmark of the MoE layer hot path on one MI355X.

One step = one pass of the whole path over one batch of seeded synthetic
input already resident in HBM: mok_build_schedule + mok_forward (and
mok_backward for the forward+backward workloads). Default workload: the
8192-token BF16 forward (T=8192, H=2048, I=768, E=128, k=8, shared I_s=768).

Prints ONE JSON line (rank 0, N=1):
  value = tokens/s of the whole step; roofline = the dominant kernel (the
  gate/up grouped GEMM) against the bf16 (or MXFP8) MFMA peak, timed with
  HIP events on its launch stream over the timed region (the only kernel
  with events there); kernels_ms_per_step = every kernel, from a separate
  pass after the timed region; cpu_baseline = the float64 NumPy oracle on a
  bounded token sample on this host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       [--no-cpu-baseline] [--all]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import CONFIGS, MoEShape, make_inputs  # noqa: E402

METRIC = "MoE layer tokens/s + achieved TFLOP/s vs MFMA peak, BF16 & MXFP8 fwd/bwd"
PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0}
HBM_GBS = 8000.0
DEFAULT = "t8192_bf16_fwd"
CSRC = os.path.join(ROOT, "mixture_experts_layer_build_amd", "csrc")
# Sources that define the gate/up grouped-GEMM kernel and its launch.
GATE_UP_SOURCES = ("gemm_nt.h", "gemm_common.h", "device_common.h", "mok_internal.h", "forward.hip")
# HBM bytes per gate/up launch from two rocprofv3 counter passes over this
# script (FETCH_SIZE, then WRITE_SIZE, mean over the dispatches), each scaled
# by the factor the same counter gives for a plain copy kernel of known size
# (--copy-calibration): read factor 2.000, write factor 1.000. Keyed by
# (workload, sha256 of GATE_UP_SOURCES): once the kernel changes, the figure
# no longer applies and traffic is reported as null.
MEASURED_TRAFFIC = {
    ("t8192_bf16_fwd", "a750ae5e21ca5bd9"): 796578 * 1024 * 2.000 + 110592 * 1024 * 1.000,
    ("t8192_mxfp8_fwd", "a750ae5e21ca5bd9"): 435827 * 1024 * 2.000 + 57292 * 1024 * 1.000,
}


def gate_up_source_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    for n in GATE_UP_SOURCES:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(CONFIGS))
    ap.add_argument("--mult", type=float, default=None, help="override the capacity multiplier")
    ap.add_argument("--minibatch", type=int, default=0, help="minibatch_size of the forward's minibatch pipeline (0 = off)")
    ap.add_argument("--movers", type=int, default=0, help="compute units given to the combine in the pipeline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0, help="oracle chunk size; 0 = automatic")
    ap.add_argument("--all", action="store_true", help="one line per workload (diagnostics)")
    ap.add_argument("--autograd", action="store_true",
                    help="run the step through the torch.autograd layer (forward, then backward from "
                         "grad_out for the training workloads) instead of the direct library calls")
    ap.add_argument("--macrobatch", type=int, default=0,
                    help="macrobatch_size of the forward's token ring (inference workloads; 0 = one pass)")
    ap.add_argument("--dense-calibration", action="store_true",
                    help="instead of the layer: time torch.matmul (hipBLASLt) on the dense GEMMs of the "
                         "workload's shape (all routed rows and the shared rows as one matrix), a "
                         "library ceiling for the grouped GEMMs")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed steps, run one plain device-to-device copy of MIB MiB (a "
                         "known-size reference for the HBM byte counters of a profiler run)")
    return ap.parse_args()


def to_device(inp, torch):
    def bf(a):
        if a is None:
            return None
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    d = dict(x=bf(inp["x"]), top=torch.from_numpy(inp["top_experts"]).cuda(),
             w=torch.from_numpy(inp["router_weights"]).cuda(), g=bf(inp.get("grad_out")))
    d["weights"] = {"routed_gate": bf(inp["w_gate"]), "routed_up": bf(inp["w_up"]),
                    "routed_down": bf(inp["w_down"])}
    if inp.get("s_gate") is not None:
        d["weights"].update(shared_gate=bf(inp["s_gate"]), shared_up=bf(inp["s_up"]), shared_down=bf(inp["s_down"]))
    return d


def kept_assignments(sched_fields) -> int:
    return int(sched_fields["kept"].sum().item())


def cpu_baseline(c: MoEShape, inp: dict, mult: float, chunk_tokens: int, min_seconds: float = 12.0) -> dict:
    """The oracle (float64 NumPy, as it stands) on consecutive chunks of
    `chunk_tokens` tokens of the same batch (each chunk with its own
    schedule), taken in order until at least `min_seconds` of CPU work."""
    from oracle import moe as omoe
    from workloads import bf16_bits_to_f32
    np.ones((64, 64)) @ np.ones((64, 64))  # loads the BLAS library, so that it is listed below
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        threads = max([p.get("num_threads", 1) for p in libs] or [os.cpu_count() or 1])
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')} ({libs[0].get('architecture')}, " \
                   f"{libs[0].get('threading_layer')})"
    except Exception:
        threads = os.cpu_count() or 1
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    n = max(1, min(chunk_tokens, c.T))
    f = lambda a: None if a is None else bf16_bits_to_f32(a).astype(np.float64)  # noqa: E731
    w = [f(inp["w_gate"]), f(inp["w_up"]), f(inp["w_down"]), f(inp["s_gate"]), f(inp["s_up"]), f(inp["s_down"])]
    done = 0
    chunks = 0
    t0 = time.perf_counter()
    while True:
        lo = (chunks * n) % c.T
        hi = min(lo + n, c.T)
        args = [f(inp["x"][lo:hi]), inp["top_experts"][lo:hi], inp["router_weights"][lo:hi], *w]
        if c.passes == "fwd":
            if c.mode == "mxfp8":
                omoe.forward_mxfp8(*args, capacity_multiplier=mult)
            else:
                omoe.forward(*args, capacity_multiplier=mult)
        else:
            g = f(inp["grad_out"][lo:hi])
            if c.mode == "mxfp8":
                omoe.forward_mxfp8(*args, capacity_multiplier=mult)
                omoe.backward_mxfp8(g, *args, capacity_multiplier=mult)
            else:
                omoe.forward(*args, capacity_multiplier=mult)
                omoe.backward(g, *args, capacity_multiplier=mult)
        done += hi - lo
        chunks += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done / dt, 1), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model, "host_cpus": os.cpu_count(), "blas": blas,
            "sample": f"{chunks} consecutive chunks of {n} tokens ({done} tokens) of the same seeded "
                      f"{c.T}-token batch, each chunk scheduled on its own, float64 NumPy oracle "
                      f"({'fwd' if c.passes == 'fwd' else 'fwd+bwd'}, {c.mode}), {dt:.1f} s"}


def copy_calibration(mib: int) -> None:
    """One plain elementwise copy kernel (torch.neg on float32) that reads
    exactly mib MiB and writes exactly mib MiB, launched as a kernel (not a
    DMA-engine copy), so that a profiler sees its byte counters."""
    import torch
    src = torch.ones((mib << 20) // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()


def dense_calibration(c: MoEShape, steps: int, warmup: int) -> dict:
    """torch.matmul on the dense equivalents of the grouped GEMMs: the
    T*k routed rows and the T shared rows stacked into one M dimension
    (M = T*(k+1) when I_s == I). gate/up: [M, H] x [H, 2I]; down: [M, I] x
    [I, H]. Operands are N(0,1) bf16 (the chip's clock depends on the
    data); in FP8 the same shapes through torch._scaled_mm with E4M3
    operands and per-tensor scales, when this torch supports it."""
    import torch
    if c.I_s not in (0, c.I):
        raise SystemExit("dense calibration needs I_s == I or no shared expert")
    M = c.T * c.k + (c.T if c.I_s else 0)
    g = torch.Generator(device="cuda").manual_seed(7)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    res = {}
    for name, (K, N) in {"gate_up": (c.H, 2 * c.I), "down": (c.I, c.H)}.items():
        A = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
        B = torch.randn(K, N, device="cuda", generator=g).to(torch.bfloat16)
        C_ = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
        ms = timed(lambda: torch.matmul(A, B, out=C_))
        fl = 2.0 * M * K * N
        res[name + "_bf16"] = {"M": M, "K": K, "N": N, "ms": round(ms, 5),
                               "tflops": round(fl / ms / 1e9, 1), "frac": round(fl / ms / 1e9 / 2500.0, 4)}
        try:
            A8 = A.to(torch.float8_e4m3fn)
            B8 = B.t().contiguous().to(torch.float8_e4m3fn).t()  # column-major, as _scaled_mm wants
            one = torch.ones((), device="cuda")
            ms8 = timed(lambda: torch._scaled_mm(A8, B8, scale_a=one, scale_b=one, out_dtype=torch.bfloat16))
            res[name + "_fp8"] = {"ms": round(ms8, 5), "tflops": round(fl / ms8 / 1e9, 1),
                                  "frac": round(fl / ms8 / 1e9 / 5000.0, 4)}
        except Exception as e:  # not every torch build has an FP8 GEMM for this GPU
            res[name + "_fp8"] = {"error": f"{type(e).__name__}: {str(e)[:200]}"}
        del A, B, C_
    return {"dense_calibration": c.name, "steps": steps, "warmup": warmup, **res}


def run(c: MoEShape, steps: int, warmup: int, mult: float, want_cpu: bool, sample_tokens: int,
        minibatch: int = 0, movers: int = 0, use_autograd: bool = False, macrobatch: int = 0) -> dict:
    import torch
    import mixture_experts_layer_build_amd as mok

    inp = make_inputs(c)
    d = to_device(inp, torch)
    cfg = mok.MoKConfig(hidden=c.H, intermediate=c.I, num_experts=c.E, topk=c.k, max_tokens=c.T,
                        shared_intermediate=c.I_s, capacity_multiplier=mult, expert_pad=c.expert_pad,
                        minibatch_size=minibatch, num_mover_wgs=movers, macrobatch_size=macrobatch,
                        forward_only=1 if macrobatch else 0)
    # the autograd layer takes its workspace from the per-config cache; the
    # direct calls use one of their own
    ws = mok.get_workspace(cfg) if use_autograd else mok.Workspace(cfg)
    mode = mok.MOK_MODE_MXFP8 if c.mode == "mxfp8" else mok.MOK_MODE_BF16
    training = c.passes != "fwd"
    ctx = torch.empty(mok.context_bytes(cfg, mode), dtype=torch.uint8, device="cuda") if training else None
    sched = torch.empty(ws.layout.total_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["x"])
    weights = d["weights"]
    bwd_weights = weights
    if mode == mok.MOK_MODE_MXFP8:
        # weights pre-quantized once, outside the step (the pages' MXFP8
        # workflow): along each forward GEMM's contraction for the forward,
        # transposed along each backward GEMM's contraction for the backward
        q = {}
        for n, t in d["weights"].items():
            codes, sc = mok.mxfp8_quantize(t.reshape(-1, t.shape[-1]), axis=1)
            q[n] = codes.view(t.shape)
            q[n + "_scale"] = sc
        weights = q
        if training:
            bwd_weights = mok.mxfp8_backward_weights(d["weights"])
    grads = None

    def step():
        nonlocal grads
        mok.build_schedule(ws, d["top"], sched)
        mok.forward(ws, sched, d["x"], d["w"], weights, mode=mode, out=out, context=ctx)
        if training:
            grads = mok.backward(ws, sched, ctx, d["g"], d["x"], d["w"], bwd_weights, mode=mode, grads=grads)

    if use_autograd:
        from mixture_experts_layer_build_amd.autograd import MoKRuntime, moe_layer
        rt = MoKRuntime(cfg, mode)
        names = ("shared_gate", "shared_up", "shared_down", "routed_gate", "routed_up", "routed_down")
        leaves = [d["x"], d["w"]] + [d["weights"].get(n) for n in names]
        for t in leaves:
            if t is not None:
                t.requires_grad_(training)

        def step():  # noqa: F811
            # gradients start from None each step, as after an optimizer's
            # zero_grad(set_to_none=True); the weights do not change, so in
            # MXFP8 their quantized copies are reused
            for t in leaves:
                if t is not None:
                    t.grad = None
            y = moe_layer(rt, d["x"], d["w"], d["top"], *[d["weights"].get(n) for n in names])
            if training:
                y.backward(d["g"])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # timed region: HIP events around the dominant kernel only (each timed
    # launch adds two event records to the stream)
    ws.set_timing(True, kernels=["gate_up"])
    ws.read_timing()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    gate_up_timing = ws.read_timing()
    # per-kernel breakdown: a separate pass with every kernel timed, outside
    # the timed region
    ws.set_timing(True)
    ws.read_timing()
    n_breakdown = max(1, min(steps, 10))
    for _ in range(n_breakdown):
        step()
    torch.cuda.synchronize()
    breakdown = ws.read_timing()
    ws.set_timing(False)

    if use_autograd:
        mok.build_schedule(ws, d["top"], sched)
    fields = mok.schedule_fields(ws, sched)
    R_kept = kept_assignments(fields)
    fwd_flops = c.fwd_flops(kept_assignments=R_kept)
    flops = fwd_flops * (3.0 if training else 1.0)
    ms = dt / steps * 1e3
    tok_s = c.T * steps / dt
    dtype = "mxfp8" if mode == mok.MOK_MODE_MXFP8 else "bf16"
    peak = PEAK_TFLOPS[dtype]
    # dominant kernel: the gate/up grouped GEMM, 4*H*(R_kept*I + T*I_s) flops per launch
    gu_flops = 4.0 * c.H * (R_kept * c.I + (c.T * c.I_s if c.I_s else 0))
    gu_ms, gu_n = gate_up_timing.get("gate_up", (float("nan"), 0))
    gu_avg = gu_ms / max(gu_n, 1)
    achieved = gu_flops / (gu_avg * 1e-3) / 1e12 if gu_n else None
    line = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic (seeded, random-init weights)",
        "config": {"workload": c.name, "tokens": c.T, "hidden": c.H, "intermediate": c.I, "experts": c.E,
                   "topk": c.k, "shared_intermediate": c.I_s, "capacity_multiplier": mult,
                   "expert_pad": c.expert_pad, "passes": c.passes, "kept_assignments": R_kept,
                   "minibatch_size": minibatch, "num_mover_wgs": movers, "macrobatch_size": macrobatch,
                   "api": "torch.autograd layer" if use_autograd else "direct library calls",
                   "parallelism": "single GPU (one GPU's share; no all-to-all)"},
        "tflops": round(flops / (dt / steps) / 1e12, 2),
        "frac_of_peak_layer": round(flops / (dt / steps) / 1e12 / peak, 4),
        "roofline": {"bound": "mfma", "kernel": "gate_up grouped GEMM",
                     "achieved": None if achieved is None else round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": None if achieved is None else round(achieved / peak, 4),
                     "avg_launch_ms": round(gu_avg, 5), "algorithmic_flops_per_launch": gu_flops,
                     "traffic": MEASURED_TRAFFIC.get((c.name, gate_up_source_sha()))},
        "kernels_ms_per_step": {k: round(v[0] / n_breakdown, 5) for k, v in breakdown.items()},
    }
    if want_cpu:
        # chunks of about 1024 tokens' worth of the 8192-token workload's per-token work
        per_tok = c.fwd_flops() / c.T * (3.0 if c.passes != "fwd" else 1.0)
        n = sample_tokens or int(min(c.T, max(64, 1024 * 84.9e6 / per_tok)))
        line["cpu_baseline"] = cpu_baseline(c, inp, mult, n)
    return line


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this library runs on one GPU only: the all-to-all between GPUs is left out, "
                                   "so --gpus N with N > 1 is not supported"}))
        sys.exit(2)
    if a.dense_calibration:
        print(json.dumps(dense_calibration(CONFIGS[a.workload], a.steps, a.warmup)), flush=True)
        return
    names = [n for n in CONFIGS] if a.all else [a.workload]
    for n in names:
        c = CONFIGS[n]
        mult = c.capacity_multiplier if a.mult is None else a.mult
        line = run(c, a.steps, a.warmup, mult, not a.no_cpu_baseline and not a.all, a.cpu_sample_tokens,
                   a.minibatch, a.movers, a.autograd, a.macrobatch)
        print(json.dumps(line), flush=True)
    if a.copy_calibration:
        copy_calibration(a.copy_calibration)


if __name__ == "__main__":
    main()
