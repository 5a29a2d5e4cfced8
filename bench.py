#!/usr/bin/env python3
"""Benchmark of the MoE-FFN layer forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]

A step is one moe_forward call (route, permute, grouped expert FFN, shared expert if any, combine)
over one batch of seeded synthetic tokens already resident in HBM. Default workload: the
Mixtral-8x7B-shaped prefill layer (T=8192, d_model=4096, d_ff=14336, E=8, top-2, bf16 SwiGLU,
fp32 router). Prints ONE JSON line with the throughput, the roofline of the dominant kernel
(the gate/up grouped GEMM, timed with HIP events on the stream it runs on), per-stage timings
and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
FP32_PEAK_TFLOPS = 157.3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="mixtral_prefill")
    ap.add_argument("--stage-reps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle sample size (0: automatic)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="also time hipBLASLt (torch.mm) on the gate/up shape, dense and per expert, for context")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from a HIP graph captured once (every kernel of the step runs "
                         "on each replay; the output is checked bit for bit against the eager step)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run two plain 1 GiB device copies (calibration for the HBM byte counters)")
    return ap.parse_args()


def stage_bytes_flops(cfg, used_experts=None):
    """Algorithmic bytes / flops per stage call (each input read once, each output written once).
    The expert projections carry both: their flops, and their bytes = weights (and biases) of the
    experts that received rows (all E when used_experts is None) + the activations read + written."""
    T, d, F, E, k = cfg.T, cfg.d, cfg.F, cfg.E, cfg.k
    A, b = T * k, cfg.elem_bytes
    gemm1_n = 2 * F if cfg.act == "swiglu" else F
    nu = E if used_experts is None else used_experts
    bias = cfg.act != "swiglu"
    out = {
        # x, router weights, top-k indices + gates, counts (logits not requested in the forward)
        "route": dict(bytes=T * d * b + E * d * 4 + A * 8 + E * 4),
        # top-k indices, x once, x_perm, sorted_token + inv_pos, offsets
        "permute": dict(bytes=A * 4 + T * d * b + A * d * b + 2 * A * 4 + (E + 1) * 4),
        # the forward's form: top-k indices, sorted_token + inv_pos, offsets (no row copy)
        "permute_positions": dict(bytes=A * 4 + 2 * A * 4 + (E + 1) * 4),
        "expert_up": dict(flops=2.0 * A * d * gemm1_n,
                          bytes=nu * (gemm1_n * d + (F if bias else 0)) * b + A * d * b + A * F * b),
        "expert_down": dict(flops=2.0 * A * F * d, bytes=nu * (d * F + (d if bias else 0)) * b + A * F * b + A * d * b),
        # y_perm, gates + positions, y (+ shared output)
        "combine": dict(bytes=A * d * b + A * 8 + T * d * b + (T * d * b if cfg.Fs else 0)),
    }
    if cfg.Fs:
        out["shared"] = dict(flops=2.0 * T * d * 2 * cfg.Fs + 2.0 * T * cfg.Fs * d,
                             bytes=3 * d * cfg.Fs * b + 2 * T * d * b)
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the library has no multi-GPU "
                                   "path, so --gpus must be 1", "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_routing_expert_amd import inputs as I
    from sparse_routing_expert_amd.layer import MoeLayer

    cfg = I.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    tens = I.gen_layer(cfg, device=dev)
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    L = MoeLayer(cfg, tens, device=dev)
    stream = torch.cuda.current_stream()

    # ---- the timed region: K forward steps ----------------------------------------------------
    for _ in range(args.warmup):
        L.forward()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        L.forward()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = wall * 1e3 / args.steps
    ev_ms = ev0.elapsed_time(ev1) / args.steps
    value = cfg.T / (ms_per_step / 1e3)
    step_stats = per_step_timings(L, stream, args.steps)

    graph = graph_timing(L, args.steps) if args.graph else None

    # ---- per-stage timings (HIP events on the launch stream, caches flushed before each) ------
    flush = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device=dev)
    L.route()
    L.permute()
    torch.cuda.synchronize()
    from sparse_routing_expert_amd import _lib as LIB

    def permute_positions():  # the forward's permute: positions only, the up projection gathers x's rows
        LIB.moe_permute(L.shape, L.topk_idx, L.t["x"], L.offsets, L.sorted_token, L.inv_pos, None,
                        L.ws(LIB.MOE_STAGE_PERMUTE))

    stage_calls = [("route", lambda: L.route(with_logits=False)), ("permute", L.permute),
                   ("permute_positions", permute_positions), ("expert_up", L.up), ("expert_down", L.down)]
    if cfg.Fs:
        stage_calls.append(("shared", L.shared))
    stage_calls.append(("combine", L.combine))
    times = {name: [] for name, _ in stage_calls}
    for _ in range(args.stage_reps):
        for name, fn in stage_calls:
            flush.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            times[name].append(a.elapsed_time(b))
    next_rows = next_row_timings(cfg, L, flush, stream, args.stage_reps)
    del flush
    if args.copy_probe:  # a plain copy of known size: FETCH_SIZE and WRITE_SIZE should each read 1 GiB
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev).fill_(3)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    vendor = vendor_gemm(cfg, L, stream) if args.vendor_gemm and cfg.dtype == "bf16" else None
    probes = peak_probes(dev, stream)
    used = int((L.counts > 0).sum().item())
    work = stage_bytes_flops(cfg, used)
    peak_tf = BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else FP32_PEAK_TFLOPS
    stages = {}
    for name, ts in times.items():
        ms = float(np.median(ts))
        ent = {"ms": round(ms, 5), "ms_min": round(float(np.min(ts)), 5)}
        w = work[name]
        if "bytes" in w:
            gbs = w["bytes"] / (ms * 1e-3) / 1e9
            ent.update({"GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "bytes": w["bytes"]})
        if "flops" in w:
            tf = w["flops"] / (ms * 1e-3) / 1e12
            ent.update({"TFLOP/s": round(tf, 1), "frac_mfma": round(tf / peak_tf, 4), "flops": w["flops"]})
        if "bytes" in w and "flops" in w:  # the roofline that binds: the larger of the two floors
            mfma_floor = w["flops"] / (peak_tf * 1e12)
            hbm_floor = w["bytes"] / (HBM_PEAK_GBS * 1e9)
            ent["bound"] = "mfma" if mfma_floor >= hbm_floor else "hbm"
            ent["frac_roofline"] = round(max(mfma_floor, hbm_floor) / (ms * 1e-3), 4)
        stages[name] = ent
    up = stages["expert_up"]
    ffn_ms = stages["expert_up"]["ms"] + stages["expert_down"]["ms"]
    ffn_tf = (work["expert_up"]["flops"] + work["expert_down"]["flops"]) / (ffn_ms * 1e-3) / 1e12
    # the library's dispatch: expert groups averaging >= 2048 rows take the four-wave wide-K kernel
    wide = cfg.T * cfg.k >= 2048 * cfg.E
    kernel = ((("gemm_bf16_wide_kernel" if wide else "gemm_bf16_persistent_kernel")
               + " (expert_up: gate/up grouped GEMM + SwiGLU)") if cfg.dtype == "bf16"
              else "gemm_f32_kernel (expert_up)")
    if cfg.dtype == "bf16" and up["bound"] == "hbm":
        # weight streaming binds: groups of a few dozen rows take the four-wave 64-row kernel
        if cfg.T * cfg.k / cfg.E <= 32:
            kernel = "gemm_bf16_kernel (expert_up: gate/up grouped GEMM + SwiGLU, 64-row tiles)"
        roofline = {"kernel": kernel, "bound": "hbm", "achieved": up["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": up["frac_hbm"], "traffic": measured_traffic(cfg.name),
                    "algorithmic_bytes_per_launch": work["expert_up"]["bytes"], "avg_launch_ms": up["ms"],
                    "frac_of_measured_copy": round(up["GB/s"] / probes["copy"]["GB/s"], 4)}
    else:
        roofline = {"kernel": kernel, "bound": "mfma" if cfg.dtype == "bf16" else "alu", "achieved": up["TFLOP/s"],
                    "peak": peak_tf, "unit": "TFLOP/s", "frac": round(up["TFLOP/s"] / peak_tf, 4),
                    "traffic": measured_traffic(cfg.name) if cfg.dtype == "bf16" else None,
                    "algorithmic_flops_per_launch": work["expert_up"]["flops"], "avg_launch_ms": up["ms"]}
        if cfg.dtype == "bf16":
            roofline["frac_of_measured_mfma_loop"] = round(up["TFLOP/s"] / probes["mfma_loop"]["TFLOP/s"], 4)

    # ---- CPU oracle on a bounded sample of the same workload ----------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, L, args.cpu_tokens)

    out = {
        "metric": "routed tokens/sec per MoE layer fwd; grouped-GEMM % MFMA peak; route GB/s",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; random-init weights of the layer's shape)",
        "config": {"workload": cfg.name, "T": cfg.T, "d_model": cfg.d, "d_ff": cfg.F, "E": cfg.E, "k": cfg.k,
                   "act": cfg.act, "score": cfg.score, "d_ff_shared": cfg.Fs, "router": cfg.router},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "stages": stages,
        "grouped_ffn": {"ms": round(ffn_ms, 4), "TFLOP/s": round(ffn_tf, 1), "frac_mfma": round(ffn_tf / peak_tf, 4)},
        "route_GB/s": stages["route"]["GB/s"],
        "assignments_per_s": round(value * cfg.k, 1),
        "event_ms_per_step": round(ev_ms, 4),
        "step_timing": step_stats,
        "peaks_measured": probes,
        "graph_replay": graph,
        "vendor_gemm": vendor,
        "capacity_permute": next_rows["capacity_permute"],
        "bias_update": next_rows["bias_update"],
        "noisy_route": next_rows["noisy_route"],
        "backward": next_rows["backward"],
        "input_gen_s": round(gen_s, 2),
    }
    print(json.dumps(out), flush=True)


def per_step_timings(L, stream, steps):
    """The forward step timed one by one with HIP events on its stream: warm (back to back, as in the
    headline) and cold (a 1 GiB fill before each step evicts the 256 MiB last-level cache and the L2s,
    so weights and activations come from HBM); median and minimum of each."""
    import numpy as np
    import torch

    flush = torch.empty(1 << 30, dtype=torch.uint8, device=L.dev)

    def run(cold):
        ts = []
        for _ in range(steps):
            if cold:
                flush.fill_(7)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            L.forward()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return {"median_ms": round(float(np.median(ts)), 4), "min_ms": round(float(np.min(ts)), 4),
                "tokens_per_s_median": round(L.T / (float(np.median(ts)) * 1e-3), 1)}

    out = {"warm": run(False), "cold": run(True), "steps": steps, "flush_bytes": 1 << 30}
    del flush
    return out


def peak_probes(dev, stream):
    """What this card reaches right now on a streaming copy (read + write) and on bf16 matrix
    instructions alone (register operands), next to the published 8 TB/s and 2.5 PFLOP/s."""
    import numpy as np
    import torch

    from sparse_routing_expert_amd import _lib as LIB

    def timed(fn, reps=5):
        fn()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(3)
    dst = torch.empty_like(src)
    ms_c = timed(lambda: LIB.moe_probe_copy(src, dst, n, 2048))
    ms_t = timed(lambda: dst.copy_(src))
    del src, dst
    blocks, iters = 1024, 4000
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    flops = LIB.moe_probe_mfma(blocks, iters, out)
    ms_m = timed(lambda: LIB.moe_probe_mfma(blocks, iters, out))
    del out
    copy_gbs = 2 * n / (ms_c * 1e-3) / 1e9
    mfma_tf = flops / (ms_m * 1e-3) / 1e12
    return {"copy": {"kernel": "moe_probe_copy (64 KB chunks per block, 16 loads then 16 stores per lane, non-temporal)", "bytes_moved": 2 * n,
                     "ms": round(ms_c, 4), "GB/s": round(copy_gbs, 1), "frac_of_published": round(copy_gbs / HBM_PEAK_GBS, 4),
                     "torch_copy_GB/s": round(2 * n / (ms_t * 1e-3) / 1e9, 1)},
            "mfma_loop": {"kernel": "moe_probe_mfma (v_mfma_f32_32x32x16_bf16 on registers)", "flops": flops,
                          "ms": round(ms_m, 4), "TFLOP/s": round(mfma_tf, 1),
                          "frac_of_published": round(mfma_tf / BF16_PEAK_TFLOPS, 4)}}


def graph_timing(L, steps):
    """The step captured once into a HIP graph (torch.cuda.CUDAGraph over the library's launches on
    the capture stream) and replayed `steps` times; the replayed output must equal the eager one bit
    for bit (the kernels are deterministic)."""
    import torch

    L.forward()
    torch.cuda.synchronize()
    ref = L.y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.forward()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(L.y.view(torch.int16) if L.y.dtype == torch.bfloat16 else L.y, ref.view(torch.int16)
                            if ref.dtype == torch.bfloat16 else ref))
    w0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - w0) * 1e3 / steps
    del g
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(L.T / (ms / 1e3), 1), "matches_eager": same}


def next_row_timings(cfg, L, flush, stream, reps):
    """Expert capacity (moe_permute with C = ceil(1.0 * T * k / E)) and the aux-loss-free bias step
    (moe_update_bias) on the same layer, HIP events on the launch stream, caches flushed before each."""
    import math

    import numpy as np
    import torch

    from sparse_routing_expert_amd import _lib as LIB

    T, k, E, d, b = cfg.T, cfg.k, cfg.E, cfg.d, cfg.elem_bytes
    cap = int(math.ceil(1.0 * T * k / E))
    shape_c = LIB.shape_of(cfg, T, cap)
    ws = L.ws(LIB.MOE_STAGE_PERMUTE)
    bias = L.t["sel_bias"].clone() if L.t["sel_bias"] is not None else torch.zeros(E, dtype=torch.float32,
                                                                                  device=L.dev)

    def timed(fn):
        ts = []
        for _ in range(reps):
            flush.fill_(1)
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            e.record(stream)
            e.synchronize()
            ts.append(a.elapsed_time(e))
        return float(np.median(ts))

    ms = timed(lambda: LIB.moe_permute(shape_c, L.topk_idx, L.t["x"], L.offsets, L.sorted_token, L.inv_pos,
                                       L.x_perm, ws))
    kept = int(L.offsets[-1].item())
    A = T * k
    nbytes = A * 4 + T * d * b + kept * d * b + 2 * A * 4 + (E + 1) * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    perm = {"capacity_rows": cap, "kept": kept, "dropped": A - kept, "ms": round(ms, 5), "bytes": nbytes,
            "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    ms_b = timed(lambda: LIB.moe_update_bias(L.shape, L.counts, 1e-3, bias))
    # noisy top-k routing: x once, both fp32 projections, the noise, and the route outputs
    from sparse_routing_expert_amd import inputs as I

    w_n, noise = I.gen_noisy_router(cfg, device=L.dev)
    ms_n = timed(lambda: L.route_noisy(w_n, noise, with_logits=False, with_stats=False))
    nb = T * d * b + 2 * E * d * 4 + T * E * 4 + T * k * 8 + E * 4
    L.route(with_logits=True)
    L.permute()  # back to the plain routing and dropless permutation the other stages use
    L.ffn()
    if cfg.Fs:
        L.shared()
    torch.cuda.synchronize()
    # layer backward (dy ~ N(0,1), balancing coefficient 0.01): the recomputed up projection, two
    # dgrad and two wgrad products per expert, plus the shared expert's five
    dy = I.gen_dy(cfg, device=L.dev)
    grads = L.alloc_grads()
    L.backward(dy, grads, aux_coef=0.01)
    torch.cuda.synchronize()
    ms_bw = timed(lambda: L.backward(dy, grads, aux_coef=0.01))
    rows = int(L.offsets[-1].item())
    n_in = cfg.n_in
    fl = 2.0 * rows * d * (3 * n_in + 2 * cfg.F) + 16.0 * T * d * cfg.Fs + 4.0 * T * E * d
    del grads
    return {"capacity_permute": perm,
            "bias_update": {"ms": round(ms_b, 5), "bytes": E * 12, "note": "E-length, launch-bound"},
            "noisy_route": {"ms": round(ms_n, 5), "bytes": nb, "GB/s": round(nb / (ms_n * 1e-3) / 1e9, 1)},
            "backward": {"ms": round(ms_bw, 4), "flops": fl, "TFLOP/s": round(fl / (ms_bw * 1e-3) / 1e12, 1),
                         "frac_mfma_bf16": round(fl / (ms_bw * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}}


def vendor_gemm(cfg, L, stream):
    """hipBLASLt through torch.mm on the gate/up product: all routed rows against one expert's
    [2F, d] weights (a dense GEMM of the same total size), and one expert's share of the rows."""
    import torch

    A = L.x_perm
    W = L.t["w_in"][0]
    out = {}
    for name, rows in (("dense_all_rows", A.shape[0]), ("one_expert_rows", A.shape[0] // cfg.E)):
        a = A[:rows]
        torch.mm(a, W.t())
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            torch.mm(a, W.t())
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[len(ts) // 2]
        flops = 2.0 * rows * W.shape[0] * W.shape[1]
        out[name] = {"m": rows, "n": W.shape[0], "k": W.shape[1], "ms": round(ms, 4),
                     "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1)}
    return out


COPY_PROBE_BYTES = 1 << 30
GEMM_SOURCE = os.path.join(ROOT, "sparse_routing_expert_amd", "csrc", "grouped_gemm.hip")


def measured_traffic(workload: str):
    """HBM bytes per gate/up GEMM launch from the committed counter summary, or None.

    The summary (profiles/traffic_expert_up_<workload>.md) records FETCH_SIZE + WRITE_SIZE of the
    kernel, each scaled by the same counter's reading for a plain 1 GiB copy, together with the
    SHA-256 of the GEMM source it was taken on. A changed kernel source makes the figure stale: None.
    """
    import hashlib

    path = os.path.join(ROOT, "profiles", f"traffic_expert_up_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("- `") and "`: " in line:
            key, val = line[3:].split("`: ", 1)
            fields[key] = val.strip().strip("`")
    with open(GEMM_SOURCE, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if fields.get("kernel_source_sha256") != sha or "hbm_bytes_per_launch" not in fields:
        return None
    return int(fields["hbm_bytes_per_launch"])


def oracle_stages(cfg, t, x):
    """The oracle's layer on the tokens x, stage by stage: the calls of oracle.moe_ref.layer_forward in
    its order (route, permute with the row gather, the per-expert FFN loop, the shared expert, combine),
    each timed. Returns the layer output and the seconds of each stage."""
    from oracle import moe_ref as R

    sec = {}
    t0 = time.perf_counter()
    xf = R.f64(x)
    r = R.route(xf, t["w_r"], cfg.k, cfg.score, cfg.renorm, t["sel_bias"])
    t1 = time.perf_counter()
    offsets, sorted_token, inv_pos = R.permute(r.idx, cfg.E)
    x_perm = xf[sorted_token]
    t2 = time.perf_counter()
    get = R.stacked_experts(t["w_in"], t["b_in"], t["w_out"], t["b_out"])
    y_perm = R.experts_on_rows(x_perm, offsets, get, cfg.act)
    t3 = time.perf_counter()
    ys = R.shared_ffn(xf, R.f64(t["ws_in"]), R.f64(t["ws_out"])) if t["ws_in"] is not None else None
    t4 = time.perf_counter()
    y = R.combine(y_perm, inv_pos, r.gates, ys)
    t5 = time.perf_counter()
    sec = {"route": t1 - t0, "permute": t2 - t1, "expert_ffn": t3 - t2, "shared": t4 - t3, "combine": t5 - t4}
    return y, sec


def cpu_baseline(cfg, L, n_tokens: int):
    """The float64 oracle, as it stands, on the first n tokens of the same layer (host cores)."""
    import numpy as np

    try:
        from threadpoolctl import threadpool_info

        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    allowed = len(os.sched_getaffinity(0))
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    if n_tokens <= 0:  # about 10-30 s of CPU work on a many-core host
        per_tok = 6.0 * cfg.k * cfg.d * cfg.F + 2.0 * cfg.E * cfg.d + (6.0 * cfg.d * cfg.Fs if cfg.Fs else 0)
        n_tokens = int(max(16, min(cfg.T, 1e13 / per_tok)))
    n_tokens = min(n_tokens, cfg.T)
    y, sec = oracle_stages(cfg, L.t, L.t["x"][:n_tokens])
    dt = sum(sec.values())
    assert np.isfinite(y).all()
    return {"value": round(n_tokens / dt, 3), "unit": "tokens/s", "cores": min(threads, allowed), "kind": "oracle",
            "blas_threads": threads, "cpus_allowed": allowed, "cpu_model": model,
            "sample": f"first {n_tokens} of {cfg.T} tokens of the same layer, full oracle forward (route, permute, "
                      f"per-expert fp64 loop incl. converting each used expert's bf16 weights, combine)",
            "seconds": round(dt, 2), "stage_seconds": {k: round(v, 3) for k, v in sec.items()}}


if __name__ == "__main__":
    main()
