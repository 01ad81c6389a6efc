#!/usr/bin/env python3
"""MoE-layer throughput on one MI355X.

One step = route + dispatch + expert GEMM + combine over one batch of the
full-router workload (T=4096 tokens, d=2048, E=896 experts, top-16, SwiGLU
f=256, bf16, all experts on this GPU), inputs resident in HBM before timing.

Prints ONE JSON line: tokens/s, ms per step, the roofline of the dominant
kernel (the gate/up grouped GEMM, which streams 1.9 GB of expert weights per
step) from HIP events recorded around it on its launch stream, and the CPU
oracle timed on a bounded token sample of the same workload. With the
default workload the line also carries "workloads": the one-rank share at
EP = 64 (16384 tokens, 14 local experts, f = 1024), the skewed routing with
capacity (overflow dropped, and remapped to the next-ranked experts), the
LoRA fine-tuning step and the latent-space router, each with ms per step,
tokens/s and every stage against its roofline (fewer steps, no CPU baseline).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-cpu-baseline] [--no-backward] [--no-extra-workloads]
                  [--graph] [--calibrate-copy]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec (route+dispatch+experts+combine); % bf16 MFMA/HBM peak"
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, vendor figure
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure
PMC_FILE = os.path.join(ROOT, "profiles", "gate_up_full_router_pmc.txt")
KERNEL_SOURCES = ["expert_gemm.hip", "mfma_tile.h", "common.h"]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for n in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "sparse_mixture_experts_top_amd", "csrc", n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per gate/up launch from the committed rocprofv3 counter runs,
    or None when they are missing or the kernel source changed since."""
    if not os.path.exists(PMC_FILE):
        return None
    vals = {}
    with open(PMC_FILE) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_hash") != kernel_source_hash() or vals.get("workload") != workload:
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class LazyExperts:
    """Per-expert float64 view of a bf16 CPU tensor, converted on access."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, i):
        import torch
        return self.t[i].to(torch.float64).numpy()


def cpu_baseline(w, inp):
    """The oracle, untouched, on the first S tokens of the same workload."""
    import numpy as np
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    wr = inp["w_router"].to(torch.float64).numpy()
    wg, wu, wd = LazyExperts(inp["w_gate"]), LazyExperts(inp["w_up"]), LazyExperts(inp["w_down"])
    bias = inp["bias"].numpy() if "bias" in inp else None
    S = min(64, w.T)          # about 15-20 s of float64 NumPy on 8-16 cores
    x = inp["x"][:S].to(torch.float64).numpy()
    lora = None
    if w.lora_r:
        lora = {"scale": w.lora_alpha / w.lora_r,
                **{n: inp[n].to(torch.float64).numpy() for n in ("a_up", "b_up", "a_down", "b_down")}}
    t0 = time.perf_counter()
    fwd = oracle.moe_layer(x, wr, wg, wu, wd, w.k, bias=bias, e_lo=w.e_lo, e_hi=w.local_hi,
                           capacity=0, lora=lora, aux_coef=w.aux_coef)
    what = "route over all {E} experts, dispatch, SwiGLU experts, combine".format(E=w.E)
    if lora is not None:
        dy = inp["dy"][:S].to(torch.float64).numpy()
        oracle.lora_backward(dy, fwd["x_perm"], fwd["offsets"], fwd["row_src"], fwd["row_gate"], fwd["G"],
                             fwd["H"], wd, lora)
        what += " with LoRA, load-balance loss, LoRA adapter gradients"
    spent, total_tok = time.perf_counter() - t0, S
    log(f"[cpu_baseline] oracle on {S} tokens: {spent:.2f} s")
    return {"value": total_tok / spent, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {total_tok} of {w.T} tokens of {w.name} ({what}; float64 NumPy), {spent:.1f} s"}


def calibrate_copy(nbytes: int = 1 << 30, reps: int = 5) -> None:
    """A plain elementwise copy of known size, for scaling FETCH_SIZE / WRITE_SIZE;
    also prints the copy's own bandwidth (a practical HBM ceiling on this machine)."""
    import torch
    n = nbytes // 4
    a = torch.randn(n, device="cuda")
    b = torch.empty_like(a)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for i in range(reps):
        if i == reps - 1:
            ev[0].record()
        torch.mul(a, 1.0, out=b)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1])
    log(f"[calibrate] {reps} copies of {nbytes} bytes read + {nbytes} bytes written; "
        f"last copy {ms:.3f} ms = {2 * nbytes / ms / 1e6:.0f} GB/s")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="full_router")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurement pass")
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="with the default workload, skip the ep64_rank / skewed_capacity / lora_step lines")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--graph", dest="graph", action="store_true", default=False,
                    help="time one HIP-graph replay of the K steps (no per-kernel roofline: "
                         "HIP cannot time events recorded inside a graph)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the expert-parallel all-to-all is design only). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch

    from sparse_mixture_experts_top_amd.workloads import WORKLOADS

    if args.calibrate_copy:
        calibrate_copy()
        return 0

    w = WORKLOADS[args.workload]
    out = run_workload(args, w, args.steps, args.warmup, backward=not args.no_backward,
                       cpu=not args.no_cpu_baseline, graph=args.graph)
    if args.workload == "full_router" and not args.no_extra_workloads:
        # the other single-GPU workloads, fewer steps, each with its dominant
        # kernel against its roofline (no backward pass, no CPU baseline)
        out["workloads"] = {}
        for name in ("ep64_rank", "skewed_capacity", "lora_step", "skewed_remap", "latent_router"):
            torch.cuda.empty_cache()
            res = run_workload(args, WORKLOADS[name], min(args.steps, 10), min(args.warmup, 3),
                               backward=False, cpu=False, graph=False)
            out["workloads"][name] = summarise(res)
    print(json.dumps(out), flush=True)
    return 0


def summarise(res):
    """The figures of one extra workload that the bench line carries."""
    keep = ("ms_per_step", "value", "steps", "warmup")
    s = {k: res[k] for k in keep}
    s["tokens_per_s"] = s.pop("value")
    s["config"] = res["config"]
    s["dominant_kernel"] = res["dominant_kernel"]
    s["roofline"] = res["roofline"]
    s["stage_roofline"] = res.get("stage_roofline")
    s["kernels_us"] = res.get("kernels_us", res.get("kernels_us_per_step"))
    return s


def gemm_roofline(name, flops, nbytes, us):
    """A grouped GEMM against both of its roofs: the bound is whichever of
    flops / MFMA peak and bytes / HBM peak takes longer."""
    tf = flops / (us * 1e-6) / 1e12
    gbs = nbytes / (us * 1e-6) / 1e9
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    return {"bound": "mfma" if t_mfma > t_hbm else "hbm", "us": round(us, 2), "tflops": round(tf, 1),
            "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "gbs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "frac": round(max(t_mfma, t_hbm) / (us * 1e-6), 4)}


def run_workload(args, w, steps, warmup, backward, cpu, graph):
    """Time ``steps`` forward steps of workload ``w`` (the LoRA step for a
    LoRA workload) and return its bench record."""
    import torch

    from sparse_mixture_experts_top_amd import binding as B
    from sparse_mixture_experts_top_amd import layer
    from sparse_mixture_experts_top_amd.workloads import generate

    log(f"[bench] generating {w.name}: T={w.T} d={w.d} E={w.E} k={w.k} f={w.f} L={w.L}")
    t0 = time.time()
    inp = generate(w, seed=0)
    dev = {k: v.to("cuda") for k, v in inp.items()}
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f} s")
    shape = layer.shape_of(w)
    if w.lora_r:
        return lora_step_bench(args, w, inp, dev, shape, steps, warmup, cpu)
    buf = layer.alloc(shape)
    # the frozen expert weights live in their packed layout (one-time, outside the step)
    packed = layer.pack_weights(shape, dev["w_gate"], dev["w_up"], dev["w_down"])
    variant = layer.variant_buffers(w, dev)
    torch.cuda.synchronize()
    args_fw = (dev["x"], dev["w_router"], dev.get("bias"), None, None, None)

    for _ in range(warmup):
        layer.forward(buf, *args_fw, packed=packed, variant=variant)
    torch.cuda.synchronize()

    # timed region: K steps. The library brackets only the gate/up kernel with
    # HIP events (on its launch stream), for the roofline figure. With
    # --graph the K steps are captured once into one HIP graph and the timed
    # region is one replay of it (the roofline kernel is then timed in the
    # breakdown pass below instead).
    g = None
    if graph:
        g = layer.capture(lambda: [layer.forward(buf, *args_fw, packed=packed, variant=variant)
                                   for _ in range(steps)])
        g.replay()
        torch.cuda.synchronize()
    else:
        B.moe_timing_enable(["gate_up"])
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    if g is not None:
        g.replay()
    else:
        for _ in range(steps):
            layer.forward(buf, *args_fw, packed=packed, variant=variant)
    stop.record(stream)
    torch.cuda.synchronize()
    elapsed_ms = start.elapsed_time(stop)
    gu_ms, gu_n = (0.0, 0) if g else B.moe_timing_read("gate_up")
    log(f"[bench] {w.name}: {steps} steps in {elapsed_ms:.3f} ms ({'one graph replay' if g else 'eager launches'})")
    # per-kernel breakdown from extra steps outside the timed region (every
    # kernel bracketed by events)
    B.moe_timing_enable(True)
    nb = max(1, min(steps, 10))
    for _ in range(nb):
        layer.forward(buf, *args_fw, packed=packed, variant=variant)
    torch.cuda.synchronize()
    kernels = {}
    for name in B.KERNELS:
        ms, n = B.moe_timing_read(name)
        if n:
            # per launch, and per step (a kind can run more than once a step:
            # the two dispatch passes of remapping, the latent router's GEMMs)
            kernels[name] = {"avg_us": 1000.0 * ms / n, "launches": n, "step_us": 1000.0 * ms / nb}
    B.moe_timing_enable(False)

    ms_step = elapsed_ms / steps
    tok_s = w.T / (ms_step / 1000.0)

    # algorithmic bytes of one gate/up launch: the gate and up weights of every
    # expert that received a row, the dispatched rows read once, H written once
    counts = buf.offsets.diff().cpu().numpy()
    R = int(buf.offsets[-1].item())
    active = int((counts > 0).sum())
    gu_bytes = 2 * active * w.f * w.d * 2 + R * w.d * 2 + R * w.f * 2
    gu_us = 1000.0 * gu_ms / gu_n if gu_n else kernels["gate_up"]["avg_us"]
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    traffic = recorded_traffic(w.name)
    gu_flops = 4.0 * R * w.d * w.f
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic, "kernel": "gate_up_bf16", "algorithmic_bytes": gu_bytes,
            "avg_us": round(gu_us, 2),
            "mfma_tflops": round(gu_flops / (gu_us * 1e-6) / 1e12, 1),
            "mfma_frac": round(gu_flops / (gu_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    # layer-level figures for context
    router_flops = (2.0 * w.T * w.latent_dc * (w.d + w.E)) if w.latent_dc else 2.0 * w.T * w.d * w.E
    flops = router_flops + 6 * R * w.d * w.f
    # every stage against its own roofline, from the breakdown pass (durations
    # there include the event pair around each launch), per step
    stage_work = {
        "router_gemm": ("mfma", router_flops),
        "topk": ("hbm", w.T * w.E * 4 + w.T * w.k * 8),
        "dispatch": ("hbm", 3 * w.T * w.k * 4 + w.T * w.k * 4 + R * 8),
        "combine": ("hbm", R * w.d * 2 + w.T * w.k * 8 + w.T * w.d * 2),
    }
    gemm_work = {
        "gate_up": (gu_flops, gu_bytes),
        "down": (2.0 * R * w.d * w.f, active * w.d * w.f * 2 + R * w.f * 2 + R * w.d * 2),
    }
    stage_us = {k: v["step_us"] for k, v in kernels.items()}
    stage_us["dispatch"] = sum(stage_us.get(n, 0.0) for n in ("hist", "scan", "scatter", "capacity"))
    stages = {}
    for name, (bound, work) in stage_work.items():
        us = stage_us.get(name)
        if not us:
            continue
        rate = work / (us * 1e-6)
        if bound == "mfma":
            stages[name] = {"bound": "mfma", "us": round(us, 2), "tflops": round(rate / 1e12, 1),
                            "frac": round(rate / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        else:
            stages[name] = {"bound": "hbm", "us": round(us, 2), "gbs": round(rate / 1e9, 1),
                            "frac": round(rate / 1e9 / HBM_PEAK_GBS, 4)}
    for name, (fl, nb) in gemm_work.items():
        if stage_us.get(name):
            stages[name] = gemm_roofline(name, fl, nb, stage_us[name])
    dominant = max(stages, key=lambda n: stages[n]["us"]) if stages else None
    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) weights)",
        "config": {"workload": w.name, "launch": "hip_graph" if g else "eager",
                   "T": w.T, "d": w.d, "E": w.E, "k": w.k, "f": w.f,
                   "local_experts": w.L, "capacity": w.capacity, "rows": R,
                   "active_experts": active},
        "roofline": roof,
        "dominant_kernel": {"name": dominant, **stages[dominant]} if dominant else None,
        "layer_tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "kernels_us": {k: round(v["step_us"], 2) for k, v in kernels.items()},
        "stage_roofline": stages,
    }
    if w.remap:
        out["config"]["moved"] = int(variant.moved.item())
        out["config"]["dropped"] = int(buf.dropped.item())
    if w.latent_dc:
        out["config"]["latent_dc"] = w.latent_dc
    if backward:
        out["backward"] = backward_pass(w, dev, shape, packed, R, active)
    if cpu:
        out["cpu_baseline"] = cpu_baseline(w, inp)
    return out


def lora_step_bench(args, w, inp, dev, shape, steps, warmup, cpu):
    """One LoRA fine-tuning step of the layer: the forward with the rank-r
    adapters on the up and down projections (route with the softmax sums,
    dispatch, expert GEMMs saving G/H/U, combine), the load-balance loss, and
    the four adapter gradients for an upstream gradient dY. The frozen expert
    weights are packed once before timing; router and base weights get no
    gradient. tokens/s counts the layer's T tokens per step."""
    import torch

    from sparse_mixture_experts_top_amd import binding as B
    from sparse_mixture_experts_top_amd import layer

    L, r, d, f = w.L, w.lora_r, w.d, w.f
    buf = layer.alloc(shape, lora_r=r, prob=True, act_save=True)
    packed = layer.pack_weights(shape, dev["w_gate"], dev["w_up"], dev["w_down"])
    # the forward keeps the rows' rank-r projections for the backward
    z_save = torch.empty((2, max(B.moe_max_rows(shape), 1), r), dtype=torch.float32, device="cuda")
    lora = B.make_lora(r, w.lora_alpha, dev["a_up"], dev["b_up"], dev["a_down"], dev["b_down"], z_save)
    grads = [torch.empty(sz, dtype=torch.float32, device="cuda")
             for sz in ((L, r, d), (L, f, r), (L, r, f), (L, d, r))]
    # W_d^T packed once for the adapter backward's dH product (W_d is frozen)
    dgu_packed = None
    if d % 128 == 0 and f % 128 == 0:
        dgu_packed = torch.empty((L, f, d), dtype=torch.bfloat16, device="cuda")
        B.moe_pack_backward_weights(shape, dev["w_gate"], dev["w_up"], dev["w_down"], dgu_packed, None)
    torch.cuda.synchronize()

    def step():
        layer.forward(buf, dev["x"], dev["w_router"], dev.get("bias"), None, None, None, lora, packed=packed)
        B.moe_aux_loss(shape, buf.counts, buf.prob_sum, w.aux_coef, buf.aux)
        xr, xs = layer.x_rows(buf, dev["x"])
        if dgu_packed is not None:
            B.moe_lora_bwd_packed(shape, lora, dev["dy"], buf.offsets, buf.row_src, buf.row_gate, xr, xs,
                                  buf.act_save, dgu_packed, *grads, buf.ws)
        else:
            B.moe_lora_bwd(shape, lora, dev["dy"], buf.offsets, buf.row_src, buf.row_gate, xr, xs, buf.act_save,
                           dev["w_down"], *grads, buf.ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    B.moe_timing_enable(["gate_up"])
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    elapsed_ms = start.elapsed_time(stop)
    gu_ms, gu_n = B.moe_timing_read("gate_up")
    B.moe_timing_enable(True)
    nb = max(1, min(steps, 10))
    for _ in range(nb):
        step()
    torch.cuda.synchronize()
    kernels = {}  # microseconds per step, summed over a kind's launches in the step
    launches = {}
    for name in B.KERNELS:
        ms, n = B.moe_timing_read(name)
        if n:
            kernels[name] = round(1000.0 * ms / nb, 2)
            launches[name] = n
    B.moe_timing_enable(False)
    ms_step = elapsed_ms / steps
    counts = buf.offsets.diff().cpu().numpy()
    R = int(buf.offsets[-1].item())
    active = int((counts > 0).sum())
    gu_bytes = 2 * active * f * d * 2 + R * d * 2 + R * f * 2
    gu_us = 1000.0 * gu_ms / gu_n
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    gu_flops = 4.0 * R * d * f
    out = {
        "metric": METRIC, "value": round(w.T / (ms_step / 1000.0), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) tokens and dY, N(0,1/fan_in) weights, LoRA A ~ N(0,1/d), "
                "B ~ N(0,1e-3))",
        "config": {"workload": w.name, "launch": "eager", "T": w.T, "d": d, "E": w.E, "k": w.k, "f": f,
                   "local_experts": L, "lora_rank": r, "lora_alpha": w.lora_alpha, "aux_coef": w.aux_coef,
                   "rows": R, "active_experts": active,
                   "step": "forward with LoRA + load-balance loss + LoRA adapter gradients"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(w.name),
                     "kernel": "gate_up_bf16", "algorithmic_bytes": gu_bytes, "avg_us": round(gu_us, 2),
                     "mfma_tflops": round(gu_flops / (gu_us * 1e-6) / 1e12, 1),
                     "mfma_frac": round(gu_flops / (gu_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        "kernels_us_per_step": kernels,
    }
    # the step's grouped GEMMs and router against their roofs (per launch)
    per_launch = {n: kernels[n] * nb / launches[n] for n in kernels}
    stages = {}
    if "router_gemm" in per_launch:
        rt = 2.0 * w.T * d * w.E / (per_launch["router_gemm"] * 1e-6) / 1e12
        stages["router_gemm"] = {"bound": "mfma", "us": round(per_launch["router_gemm"], 2),
                                 "tflops": round(rt, 1), "frac": round(rt / MFMA_BF16_PEAK_TFLOPS, 4)}
    if "gate_up" in per_launch:
        stages["gate_up"] = gemm_roofline("gate_up", gu_flops, gu_bytes, per_launch["gate_up"])
    if "down" in per_launch:
        stages["down"] = gemm_roofline("down", 2.0 * R * d * f, active * d * f * 2 + R * f * 2 + R * d * 2,
                                       per_launch["down"])
    out["stage_roofline"] = stages
    dominant = max(kernels, key=lambda n: kernels[n])
    out["dominant_kernel"] = {"name": dominant, "us_per_step": kernels[dominant],
                              **({k: v for k, v in stages[dominant].items()} if dominant in stages else {})}
    if cpu:
        out["cpu_baseline"] = cpu_baseline(w, inp)
    return out


def backward_pass(w, dev, shape, packed, R, active, reps=5):
    """The full backward of the layer (gate / logit gradients with the
    load-balance term, dx through the experts and the router) on the forward's
    saved activations, outside the timed region: every kernel bracketed by
    HIP events, averaged over ``reps`` passes, each against its roofline."""
    import torch

    from sparse_mixture_experts_top_amd import binding as B
    from sparse_mixture_experts_top_amd import layer

    T, d, E, k, f = w.T, w.d, w.E, w.k, w.f
    buf = layer.alloc(shape, logits=True, prob=True, act_save=True)
    layer.forward(buf, dev["x"], dev["w_router"], dev.get("bias"), None, None, None, packed=packed)
    rmax = max(B.moe_max_rows(shape), 1)
    dgate = torch.empty((T, k), device="cuda")
    dlogits = torch.empty((T, E), device="cuda")
    dgu = torch.empty((rmax, 2 * f), dtype=torch.bfloat16, device="cuda")
    dx_rows = torch.empty((rmax, d), device="cuda")
    dx = torch.empty((T, d), device="cuda")
    # the frozen expert weights' transposes, packed once (outside the step)
    bwd_packed = None
    if f % 128 == 0 and d % 128 == 0:
        bwd_packed = (torch.empty((w.L, f, d), dtype=torch.bfloat16, device="cuda"),
                      torch.empty((w.L, d, 2 * f), dtype=torch.bfloat16, device="cuda"))
        B.moe_pack_backward_weights(shape, dev["w_gate"], dev["w_up"], dev["w_down"], *bwd_packed)

    wr_packed = None
    if E % 64 == 0 and d % 128 == 0:
        wr_packed = torch.empty((d, E), dtype=torch.bfloat16, device="cuda")
        B.moe_pack_router_bwd(shape, dev["w_router"], wr_packed)

    # both packed: the router product is stored into dx and the expert rows
    # are added only for tokens with a kept local slot
    fused = bwd_packed is not None and wr_packed is not None
    t_kept = int((buf.slot >= 0).any(dim=1).sum().item())

    def step(fuse):
        B.moe_gate_bwd(shape, dev["dy"], buf.y_perm, buf.slot, buf.topk_idx, buf.topk_gate, buf.logits,
                       buf.counts, 0.01, dgate, dlogits)
        if bwd_packed is not None:
            B.moe_expert_bwd_packed(shape, None, dev["dy"], buf.offsets, buf.row_src, buf.row_gate, buf.slot,
                                    buf.act_save, bwd_packed[0], bwd_packed[1], dgu, dx_rows,
                                    None if fuse else dx, buf.ws)
        else:
            B.moe_expert_bwd(shape, None, dev["dy"], buf.offsets, buf.row_src, buf.row_gate, buf.slot,
                             buf.act_save, dev["w_gate"], dev["w_up"], dev["w_down"], dgu, dx_rows, dx, buf.ws)
        if fuse:
            B.moe_router_bwd_unpermute_packed(shape, dlogits, wr_packed, dx_rows, buf.slot, dx, buf.ws)
        elif wr_packed is not None:
            B.moe_router_bwd_packed(shape, dlogits, wr_packed, dx, buf.ws)
        else:
            B.moe_router_bwd(shape, dlogits, dev["w_router"], dx, buf.ws)

    names = ["gate_bwd", "tiles", "expert_dgu", "expert_dx", "unpermute", "router_bwd"]

    def timed(fuse):
        step(fuse)
        torch.cuda.synchronize()
        B.moe_timing_enable(names)
        for _ in range(reps):
            step(fuse)
        torch.cuda.synchronize()
        us = {}
        for n in names:
            ms, cnt = B.moe_timing_read(n)
            if cnt:
                us[n] = 1000.0 * ms / cnt
        B.moe_timing_enable(False)
        return us

    two_pass = timed(False) if fused else None
    us = timed(fused)
    work = {
        "gate_bwd": ("hbm", R * d * 2 + T * d * 2 + 2 * T * E * 4 + T * k * 16),
        "expert_dgu": ("hbm", active * d * f * 2 + R * d * 2 + 4 * R * f * 2),
        "expert_dx": ("hbm", 2 * active * f * d * 2 + 2 * R * f * 2 + R * d * 4),
        # two-pass: every token's dx written; combined: dx read and written
        # for the tokens with a kept slot only
        "unpermute": ("hbm", R * d * 4 + T * k * 4 + (2 * t_kept * d * 4 if fused else T * d * 4)),
        "router_bwd": ("mfma", 2.0 * T * E * d),
    }
    flops = {"expert_dgu": 2.0 * R * d * f, "expert_dx": 4.0 * R * f * d, "router_bwd": 2.0 * T * E * d}
    stages = {}
    for name, (bound, wk) in work.items():
        if name not in us:
            continue
        rate = wk / (us[name] * 1e-6)
        st = {"bound": bound, "us": round(us[name], 2)}
        if bound == "mfma":
            st.update(tflops=round(rate / 1e12, 1), frac=round(rate / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4))
        else:
            st.update(gbs=round(rate / 1e9, 1), frac=round(rate / 1e9 / HBM_PEAK_GBS, 4))
            if name in flops:
                st["tflops"] = round(flops[name] / (us[name] * 1e-6) / 1e12, 1)
        stages[name] = st
    total = sum(us.values())
    res = {"us_per_step": round(total, 2), "tokens_per_s": round(T / (total * 1e-6), 1),
           "kernels_us": {n: round(v, 2) for n, v in us.items()}, "stage_roofline": stages,
           "packed_weights": bwd_packed is not None, "router_then_row_sums": fused,
           "tokens_with_local_rows": t_kept,
           "note": "gate + logit gradients (load-balance coef 0.01), dx through experts and router; "
                   "sum of per-kernel event times, outside the timed region"}
    if two_pass is not None:
        res["two_pass"] = {"us_per_step": round(sum(two_pass.values()), 2),
                           "kernels_us": {n: round(v, 2) for n, v in two_pass.items()}}
    return res


if __name__ == "__main__":
    sys.exit(main())
