#!/usr/bin/env python3
"""Benchmark of the fused MoE backward d_x on one MI355X.

One step = one fused call (index preparation, grouped-GEMM producer, ordered
scatter-add consumer) over a seeded synthetic batch whose inputs are already
resident in HBM.  Prints one JSON line.  After the W warm-up steps, untimed
steps continue until 30 ms of work have run, so the timed steps see the GPU's
steady-state clocks.

Default workload: decode-sized bf16 (batch 16, topK 8, G 16 with 4 empty
experts, K 7168, N 4096), where streaming the non-empty experts' weights
dominates; `value` is its effective GB/s.  The same line carries the large
fp16 workload (batch 13824, topK 8, G 60, K 7168, N 2048; TFLOP/s) under
"large" unless --no-large is given.

The roofline's kernel duration comes from HIP events around back-to-back
launches of that kernel alone (pgg_moe_dx_kernel_time, on the stream the
calls use); an event pair around each launch inside the calls would add the
launch's dispatch latency to every measurement.  The CPU baseline is the oracle on a bounded sample of the same
workload, timed on this host.

Each workload also reports the layer's forward (Permute + GroupedMatmul,
pgg_moe_fwd) under "forward", its weight gradient (pgg_moe_dw) under
"dweight", on-device routing (pgg_moe_routing) under "routing" and unpermute
with its gradient under "unpermute", on the workload's routing, weights and
d_y (--no-forward skips them); the headline value stays the fused backward's.
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

HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}
SETTLE_S = 0.03
METRIC = "fused d_x TFLOP/s (% bf16 MFMA peak) and GB/s (% HBM) at M=110K and M=128"


def kernel_sources():
    """Every source of the library: a counter run is valid only for the sources it was taken on."""
    d = os.path.join(ROOT, "permute_grouped_gemm_amd", "csrc")
    return sorted(os.path.join("permute_grouped_gemm_amd", "csrc", f) for f in os.listdir(d)
                  if f.endswith((".hip", ".cpp", ".h")))


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when they were taken on other kernel sources or another workload."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            table = json.load(f)
        h = hashlib.sha256()
        for src in kernel_sources():
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
    except OSError:
        return None
    e = table.get(f"{kernel}@{workload}") or table.get(kernel)
    if not e or e.get("workload") != workload or e.get("sources_sha") != h.hexdigest()[:16]:
        return None
    return e["traffic_bytes_per_launch"]


def algorithmic(case):
    """Algorithmic flops and bytes of one fused call (no ring / re-read traffic).

    bytes = d_y + weights of non-empty experts + routing index + group_list
    + d_x written once; flops = 2*M*N*K."""
    import numpy as np
    s = {"f32": 4, "f16": 2, "bf16": 2}[case.dtype]
    g_ne = int(np.count_nonzero(case.group_list))
    flops = 2.0 * case.M * case.N * case.K
    bytes_ = (case.M * case.N * s + g_ne * case.K * case.N * s + 8 * case.M + 8 * case.G
              + 4 * case.batch * case.K)
    producer_bytes = case.M * case.N * s + g_ne * case.K * case.N * s
    return flops, bytes_, producer_bytes


def algorithmic_forward(case):
    """Algorithmic flops and bytes of one forward call: x (each token row once)
    + weights of non-empty experts + routing index + group_list + y written
    once (fp32); flops = 2*M*K*N."""
    import numpy as np
    s = {"f32": 4, "f16": 2, "bf16": 2}[case.dtype]
    g_ne = int(np.count_nonzero(case.group_list))
    flops = 2.0 * case.M * case.N * case.K
    kernel_bytes = case.batch * case.K * s + g_ne * case.K * case.N * s + 4 * case.M * case.N
    return flops, kernel_bytes + 8 * case.M + 8 * case.G, kernel_bytes


def measure_forward(case, w, eri, gl, steps, log):
    """The layer's forward (Permute + GroupedMatmul) on the workload's own
    routing and weights, with seeded activations x [batch, K]."""
    import numpy as np
    import torch

    import permute_grouped_gemm_amd as pgg
    import synth

    dev = w.device
    x = synth.forward_input(case)
    if case.dtype == "bf16":
        xt = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        xt = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    plan = pgg.fwd_plan(xt, w, eri, gl, case.topk, case.row_idx_type)
    ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device=dev)
    y = torch.empty((case.M, case.N), dtype=torch.float32, device=dev)

    def step():
        pgg.moe_fwd(xt, w, eri, gl, case.topk, case.row_idx_type, out=y, workspace=ws)

    t_settle = time.time()
    while time.time() - t_settle < SETTLE_S:
        for _ in range(4):
            step()
        torch.cuda.synchronize()
    code, detail = pgg.read_device_error(ws)
    if code != 0:
        raise RuntimeError(f"forward device error {code} ({detail})")
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    k_ms = pgg.fwd_kernel_time(xt, w, eri, gl, case.topk, case.row_idx_type, repeats=steps, out=y,
                               workspace=ws)
    flops, bytes_, kernel_bytes = algorithmic_forward(case)
    kname = {0: "forward_large", 1: "forward_stream", 2: "forward_f32"}[plan["regime"]]
    if plan["regime"] == 1:
        achieved = kernel_bytes / (k_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    else:
        peak = PEAK_TFLOPS[case.dtype]
        achieved = flops / (k_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak}
    roof.update({"kernel": kname, "avg_launch_us": k_ms * 1e3, "launches_per_step": 1,
                 "traffic": measured_traffic(kname, case.name),
                 "traffic_unit": "bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)"})
    log(f"[bench] {case.name} forward: {ms * 1e3:.1f} us/call, {kname} {k_ms * 1e3:.1f} us "
        f"(back to back), {flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s, {bytes_ / (ms * 1e-3) / 1e9:.0f} GB/s")
    return {"ms_per_call": ms, "tflops": flops / (ms * 1e-3) / 1e12,
            "gbs": bytes_ / (ms * 1e-3) / 1e9, "frac_bf16_peak": flops / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"],
            "frac_hbm": bytes_ / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "roofline": roof,
            "algorithmic_bytes": bytes_, "flops": flops, "plan": plan,
            "what": "y[i,n] = sum_k x[p(i)//topK, k] W[g(i),k,n] on the workload's routing and "
                    "weights, x ~ N(0,1) seeded; time covers the index preparation and the kernel"}


def algorithmic_dw(case):
    """Algorithmic flops and bytes of one weight-gradient call: x (each token row
    once) + d_y + grad_w written once (fp32, all G experts); flops = 2*M*K*N."""
    s = {"f32": 4, "f16": 2, "bf16": 2}[case.dtype]
    flops = 2.0 * case.M * case.N * case.K
    kernel_bytes = case.batch * case.K * s + case.M * case.N * s + 4 * case.G * case.K * case.N
    return flops, kernel_bytes + 8 * case.M + 8 * case.G, kernel_bytes


def measure_dw(case, gy, eri, gl, steps, log):
    """The weight gradient (expanded_x^T · d_y per expert) on the workload's
    routing and upstream gradient, with the forward's seeded activations x."""
    import numpy as np
    import torch

    import permute_grouped_gemm_amd as pgg
    import synth

    dev = gy.device
    x = synth.forward_input(case)
    if case.dtype == "bf16":
        xt = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        xt = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    ws = torch.empty(pgg.dw_workspace_size(xt, gy, eri, gl, case.topk, case.row_idx_type),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((case.G, case.K, case.N), dtype=torch.float32, device=dev)

    def step():
        pgg.moe_dw(xt, gy, eri, gl, case.topk, case.row_idx_type, out=out, workspace=ws)

    t_settle = time.time()
    while time.time() - t_settle < SETTLE_S:
        for _ in range(4):
            step()
        torch.cuda.synchronize()
    code, detail = pgg.read_device_error(ws)
    if code != 0:
        raise RuntimeError(f"weight-gradient device error {code} ({detail})")
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    k_ms = pgg.dw_kernel_time(xt, gy, eri, gl, case.topk, case.row_idx_type, repeats=steps, out=out,
                              workspace=ws)
    flops, bytes_, kernel_bytes = algorithmic_dw(case)
    if case.M <= 64 * case.G:
        achieved = kernel_bytes / (k_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    else:
        peak = PEAK_TFLOPS[case.dtype]
        achieved = flops / (k_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak}
    kname = "dweight_stream" if case.M <= 64 * case.G else "dweight_large"
    roof.update({"kernel": kname, "avg_launch_us": k_ms * 1e3, "launches_per_step": 1,
                 "traffic": measured_traffic(kname, case.name),
                 "traffic_unit": "bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)"})
    log(f"[bench] {case.name} weight gradient: {ms * 1e3:.1f} us/call, {kname} {k_ms * 1e3:.1f} us "
        f"(back to back), {flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s, {bytes_ / (ms * 1e-3) / 1e9:.0f} GB/s")
    return {"ms_per_call": ms, "tflops": flops / (ms * 1e-3) / 1e12,
            "gbs": bytes_ / (ms * 1e-3) / 1e9, "roofline": roof,
            "algorithmic_bytes": bytes_, "flops": flops,
            "what": "grad_w[g] = (x rows of expert g)^T d_y[rows of g], fp32 [G,K,N], on the "
                    "workload's routing and d_y, x ~ N(0,1) seeded; time covers the index "
                    "preparation and the kernel"}


def measure_routing(case, steps, log):
    """MoeInitRouting on the device (pgg_moe_routing) for the workload's router
    choices: the tables alone, and with the permuted copy of x."""
    import numpy as np
    import torch

    import permute_grouped_gemm_amd as pgg
    import synth

    dev = torch.device("cuda:0")
    ids = torch.from_numpy(np.ascontiguousarray(case.expert, dtype=np.int64)).to(dev)
    x = synth.forward_input(case)
    if case.dtype == "bf16":
        xt = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        xt = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    ws = torch.empty(pgg.routing_workspace_size_desc(
        pgg.make_routing_desc(case.batch, case.topk, case.G, case.K, pgg.DTYPE_CODE[xt.dtype])),
        dtype=torch.uint8, device=dev)
    res = {}
    for label, xin in (("tables_only", None), ("with_expanded_x", xt)):
        def step():
            pgg.moe_routing(ids, case.G, xin, workspace=ws)
        for _ in range(5):
            step()
        torch.cuda.synchronize()
        # GPU time of the call's launches (events around them on its stream);
        # at the decode size a call's host-side work exceeds its GPU time
        with pgg.KernelTimer(capacity=steps + 4) as timer:
            for _ in range(steps):
                step()
            torch.cuda.synchronize()
        n, tot = timer.result["routing"]
        res[label + "_us"] = tot / n * 1e3
    code, _ = pgg.read_device_error(ws)
    if code != 0:
        raise RuntimeError(f"routing device error {code}")
    s = {"f32": 4, "f16": 2, "bf16": 2}[case.dtype]
    moved = case.batch * case.K * s + case.M * case.K * s + 8 * case.M * 3 + 8 * case.G
    res["expanded_x_bytes"] = case.M * case.K * s
    res["gbs_with_expanded_x"] = moved / (res["with_expanded_x_us"] * 1e-6) / 1e9
    res["what"] = ("group_list + both index encodings from expert_ids [batch, topK]; then also "
                   "expanded_x [M, K] gathered from x; GPU time per call, from HIP events "
                   "around the call's launches")
    log(f"[bench] {case.name} routing: tables {res['tables_only_us']:.1f} us, with expanded_x "
        f"{res['with_expanded_x_us']:.1f} us ({res['gbs_with_expanded_x']:.0f} GB/s)")
    return res


def measure_unpermute(case, eri, steps, log):
    """Unpermute (weighted topK sum) and its gradient at the workload's routing,
    with hidden size K and seeded random tokens, probabilities and gradients."""
    import torch

    import permute_grouped_gemm_amd as pgg

    dev = eri.device
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[case.dtype]
    gen = torch.Generator(device=dev)
    gen.manual_seed(case.seed + 100)
    perm = torch.randn((case.M, case.K), generator=gen, device=dev).to(tdt)
    probs = torch.rand((case.batch, case.topk), generator=gen, device=dev).to(tdt)
    grad = torch.randn((case.batch, case.K), generator=gen, device=dev).to(tdt)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    res = {}
    calls = {
        "unpermute": lambda: pgg.moe_unpermute(perm, eri, case.batch, case.topk, case.row_idx_type,
                                               probs, workspace=ws),
        "unpermute_grad": lambda: pgg.moe_unpermute_grad(grad, eri, case.batch, case.topk,
                                                         case.row_idx_type, perm, probs, workspace=ws),
    }
    s = {"f32": 4, "f16": 2, "bf16": 2}[case.dtype]
    moved = {"unpermute": case.M * case.K * s + case.batch * case.K * s,
             "unpermute_grad": case.batch * case.K * s + 2 * case.M * case.K * s}
    for name, fn in calls.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        with pgg.KernelTimer(capacity=steps + 4) as timer:
            for _ in range(steps):
                fn()
            torch.cuda.synchronize()
        n, tot = timer.result[name]
        us = tot / n * 1e3
        res[name] = {"us": us, "gbs": moved[name] / (us * 1e-6) / 1e9, "bytes": moved[name]}
    code, _ = pgg.read_device_error(ws)
    if code != 0:
        raise RuntimeError(f"unpermute device error {code}")
    res["what"] = ("unpermute: out[t] = sum_j probs[t,j] permuted[row(t,j)] ([batch, K], K = hidden); "
                   "grad: perm_grad and probs_grad; GPU time per call from HIP events around its launches")
    log(f"[bench] {case.name} unpermute: {res['unpermute']['us']:.1f} us ({res['unpermute']['gbs']:.0f} GB/s), "
        f"grad {res['unpermute_grad']['us']:.1f} us ({res['unpermute_grad']['gbs']:.0f} GB/s)")
    del perm, probs, grad
    return res


def measure(name, steps, warmup, cpu_baseline, log, forward=True, cold_variant=None):
    import numpy as np
    import torch

    import permute_grouped_gemm_amd as pgg
    import synth

    t0 = time.time()
    case = synth.make_config(name)
    log(f"[bench] {name}: generated inputs in {time.time() - t0:.1f}s "
        f"(M={case.M} N={case.N} K={case.K} G={case.G} {case.dtype})")
    dev = torch.device("cuda:0")

    def dev_tensor(a):
        if case.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    gy, w = dev_tensor(case.grad_y), dev_tensor(case.weight)
    eri = torch.from_numpy(case.eri).to(dev)
    gl = torch.from_numpy(case.group_list).to(dev)
    plan = pgg.plan(gy, w, eri, gl, case.batch, case.topk, case.row_idx_type)
    ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device=dev)
    out = torch.empty((case.batch, case.K), dtype=torch.float32, device=dev)

    def step():
        pgg.moe_dx(gy, w, eri, gl, case.batch, case.topk, case.row_idx_type, out=out, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # settle: the GPU's clocks take a few milliseconds of sustained load to
    # reach steady state (kernel durations drift by up to ~15% in the first
    # ~10 ms of back-to-back work), so untimed steps continue until 30 ms of
    # work have run
    t_settle = time.time()
    while time.time() - t_settle < SETTLE_S:
        for _ in range(4):
            step()
        torch.cuda.synchronize()
    code, detail = pgg.read_device_error(ws)
    if code != 0:
        raise RuntimeError(f"device error {code} ({detail})")

    # timed region 1: the calls alone -> value
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    # timed region 2: the producer (the dominant kernel) and the consumer, each
    # launched back to back between two HIP events on the stream the calls use
    # (after one full call that fills the workspace tables) -> roofline
    p_ms, p_launches = pgg.kernel_time(gy, w, eri, gl, case.batch, case.topk, case.row_idx_type,
                                       which="produce", repeats=steps, out=out, workspace=ws)
    c_ms, c_launches = pgg.kernel_time(gy, w, eri, gl, case.batch, case.topk, case.row_idx_type,
                                       which="consume", repeats=steps, out=out, workspace=ws)
    # per-kernel breakdown with an event pair around every launch (each pair
    # adds the launch's dispatch latency; informative only)
    launches_per_call = 4 + 2 * plan["max_chunks"] * plan["n_panels"]
    with pgg.KernelTimer(capacity=launches_per_call * steps + 16) as timer:
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
    log(f"[bench] {name}: {ms * 1e3:.1f} us/step; producer {p_ms * 1e3:.1f} us x {p_launches}, "
        f"consumer {c_ms * 1e3:.1f} us x {c_launches} per call (back to back); "
        f"event-bracketed kernels {timer.result}")

    # cold variant (HBM-bound workloads): a 512 MiB scrub read before every
    # call, outside its timing, so the caches hold the scrub instead of the
    # inputs (a read leaves no dirty lines to write back during the call);
    # warm calls timed the same way (an event pair per call) for comparison
    cold = None
    if cold_variant is None:
        cold_variant = plan["regime"] == 1
    if cold_variant:
        scrub = torch.ones(128 << 20, dtype=torch.int32, device=dev)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(2 * steps)]
        for k in range(steps):
            sink = scrub.sum(dtype=torch.int64)
            ev[k][0].record()
            step()
            ev[k][1].record()
        for k in range(steps, 2 * steps):
            ev[k][0].record()
            step()
            ev[k][1].record()
        torch.cuda.synchronize()
        t = [a.elapsed_time(b) * 1e3 for a, b in ev]
        med = lambda xs: sorted(xs)[len(xs) // 2]
        cold = {"cold_us_median": med(t[:steps]), "warm_us_median": med(t[steps:]),
                "method": "event pair around each call; cold = 512 MiB scrub read before each call"}
        del scrub
    sclk = smi_sclk()

    flops, bytes_, producer_bytes = algorithmic(case)
    # the library's launch names: the weight sweep is "produce_stream", the
    # fp32 tiles "produce_f32" whatever their size
    prod_name = ("produce_stream" if plan["regime"] == 1 else
                 "produce_f32" if case.dtype == "f32" else
                 {0: "produce_large", 2: "produce_f32"}[plan["regime"]])
    hbm_bound = plan["regime"] == 1
    if hbm_bound:
        # algorithmic bytes of one launch: d_y and the non-empty experts' weights
        achieved = producer_bytes / p_launches / (p_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None}
        value = bytes_ / (ms * 1e-3) / 1e9
        unit = "GB/s"
    else:
        # algorithmic flops of one launch: 2 M N K over the call's chunks
        peak = PEAK_TFLOPS[case.dtype]
        achieved = flops / p_launches / (p_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": None}
        value = flops / (ms * 1e-3) / 1e12
        unit = "TFLOP/s"
    traffic = measured_traffic(prod_name, name)
    roof["traffic"] = traffic
    roof["traffic_unit"] = "bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    roof["kernel"] = prod_name
    roof["avg_launch_us"] = p_ms * 1e3
    roof["launches_per_step"] = p_launches

    res = {
        "value": value, "unit": unit, "ms_per_step": ms,
        "tflops": flops / (ms * 1e-3) / 1e12, "gbs": bytes_ / (ms * 1e-3) / 1e9,
        "frac_bf16_peak": flops / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"],
        "frac_hbm": bytes_ / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline": roof,
        "kernels_ms_per_step": {prod_name: p_ms * p_launches, "consume": c_ms * c_launches},
        "kernels_event_bracketed_ms_per_step": {k: v[1] / steps for k, v in timer.result.items()},
        "cold_vs_warm": cold, "smi_sclk_after_timing": sclk,
        "workspace_bytes": plan["workspace_bytes"], "ring_bytes": plan["ring_bytes"],
        "d_expanded_x_fp32_bytes": case.M * case.K * 4,
        "workspace_vs_MK4": plan["workspace_bytes"] / (case.M * case.K * 4),
        "plan": plan,
        "dtype": case.dtype,
        "config": {"workload": name, "batch": case.batch, "topk": case.topk, "M": case.M,
                   "G": case.G, "G_nonempty": int(np.count_nonzero(case.group_list)),
                   "K": case.K, "N": case.N, "row_idx_type": case.row_idx_type,
                   "algorithmic_bytes": bytes_, "flops": flops},
    }
    if forward:
        res["forward"] = measure_forward(case, w, eri, gl, steps, log)
        res["dweight"] = measure_dw(case, gy, eri, gl, steps, log)
        res["routing"] = measure_routing(case, steps, log)
        res["unpermute"] = measure_unpermute(case, eri, steps, log)
    if cpu_baseline:
        res["cpu_baseline"] = oracle_baseline(case, unit, log)
    return res


def oracle_baseline(case, unit, log):
    """The oracle, as it stands, on a bounded sample of the workload."""
    import numpy as np

    import oracle
    threads = oracle.default_threads()
    # tokens whose full d_x rows the sample computes: all of a small batch,
    # else a prefix sized for roughly 10-30 s of CPU work
    n_tok = case.batch if case.M * case.N * case.K <= 8e9 else 192
    toks = np.arange(n_tok, dtype=np.int64)
    # a sample shorter than 10 s is repeated until 10 s have run, for a stable rate
    reps = 0
    t0 = time.time()
    while True:
        oracle.case_dx_tokens(case, toks, nthreads=threads)
        reps += 1
        if time.time() - t0 >= 10.0:
            break
    dt = (time.time() - t0) / reps
    rows = n_tok * case.topk
    s = {"f32": 4, "f16": 2, "bf16": 2}[case.dtype]
    if unit == "GB/s":
        # the sample reads the d_y rows of its tokens and the weights of the experts they hit
        experts = set()
        off = np.concatenate([[0], np.cumsum(case.group_list)])
        inv = np.empty(case.M, dtype=np.int64)
        if case.row_idx_type == 0:
            inv[case.eri] = np.arange(case.M)
        else:
            inv = case.eri
        for p in range(n_tok * case.topk):
            experts.add(int(np.searchsorted(off, inv[p], side="right") - 1))
        b = rows * case.N * s + len(experts) * case.K * case.N * s + 4 * n_tok * case.K
        val = b / dt / 1e9
    else:
        val = 2.0 * rows * case.N * case.K / dt / 1e12
    log(f"[bench] oracle sample: {n_tok} tokens, {reps} run(s) of {dt:.2f}s on {threads} threads")
    return {"value": val, "unit": unit, "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "seconds": dt * reps,
            "sample": f"d_x rows of tokens 0..{n_tok - 1} ({rows} expanded rows, all K columns) "
                      f"of the same inputs, computed {reps} time(s)"}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# the other workloads of the headline metric's family, each measured as the
# headline ones are (parity cases too): tiny fp32, mid bf16 (Zipf routing,
# scatter index; cold variant), large fp32 and its K/N-tail variant
EXTRA_WORKLOADS = ("tiny_f32", "mid_bf16", "large_f32", "large_f32_tail")
EXTRA_KEYS = ("value", "unit", "ms_per_step", "tflops", "gbs", "frac_bf16_peak", "frac_hbm",
              "roofline", "kernels_ms_per_step", "cold_vs_warm", "workspace_bytes", "ring_bytes",
              "d_expanded_x_fp32_bytes", "workspace_vs_MK4", "config", "dtype", "plan")


def under_profiler():
    """True when a profiler's tool library is preloaded into this process."""
    pre = os.environ.get("LD_PRELOAD", "")
    return "rocprof" in pre or any(k.startswith("ROCPROF") for k in os.environ)


def smi_sclk():
    """The shader clock rocm-smi reports right after the timed steps (or None).

    Skipped under a profiler: its preloaded library would initialise the GPU in
    every child process, and a script launched through a shebang hop would then
    replace such a process.  rocm-smi is a Python script, so it is started with
    this interpreter directly rather than through its `#!/usr/bin/env` line.
    """
    import shutil
    import subprocess
    if under_profiler():
        return None
    try:
        path = shutil.which("rocm-smi")
        if path is None:
            return None
        path = os.path.realpath(path)
        with open(path, "rb") as f:
            first = f.readline()
        cmd = [sys.executable, path] if b"python" in first else [path]
        r = subprocess.run(cmd + ["--showclocks", "--json"], capture_output=True, text=True,
                           timeout=15)
        data = json.loads(r.stdout)
        card = next(iter(data.values()))
        for k, v in card.items():
            if "sclk" in k.lower():
                return v
    except Exception:
        return None
    return None


def calibrate_copy(log, mib=1024, reps=5):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {reps} copies of {n} bytes")
    print(json.dumps({"copy_bytes": n, "reps": reps}), flush=True)


def vendor_gemm(log, reps=100):
    """Reference point: hipBLASLt (torch.mm) on one chunk of the large fp16
    workload as a plain dense GEMM, [9216 x 2048] x [2048 x 7168] -- the
    producer's shape without grouping or routing -- with fp16 and fp32
    output.  Not part of the path; printed as its own JSON line."""
    import torch
    torch.manual_seed(0)
    M, R, C = 9216, 2048, 7168
    a = torch.randn(M, R, device="cuda", dtype=torch.float16)
    wt = torch.randn(C, R, device="cuda", dtype=torch.float16).t()
    flops = 2.0 * M * R * C
    res = {}
    for name, fn in (("fp16_out", lambda: torch.mm(a, wt)),
                     ("fp32_out", lambda: torch.mm(a, wt, out_dtype=torch.float32))):
        t_end = time.time() + 0.2
        while time.time() < t_end:
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        res[name] = {"us": us, "tflops": flops / us / 1e6}
        log(f"[bench] vendor dense GEMM {M}x{R}x{C} {name}: {us:.1f} us, {flops / us / 1e6:.0f} TFLOP/s")
    print(json.dumps({"vendor_dense_gemm": res, "shape": [M, R, C], "library": "torch.mm (hipBLASLt)"}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_bf16")
    ap.add_argument("--no-large", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the tiny, mid and large fp32 workloads (the \"workloads\" object)")
    ap.add_argument("--no-forward", action="store_true",
                    help="skip the forward, weight-gradient, routing and unpermute measurements")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only time hipBLASLt (torch.mm) on the large workload's per-chunk dense GEMM")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on exactly one GPU; --gpus {args.gpus} is not supported",
              file=sys.stderr)
        return 2

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        calibrate_copy(log)
        return 0
    if args.vendor_gemm:
        vendor_gemm(log)
        return 0
    primary = measure(args.workload, args.steps, args.warmup, not args.no_cpu_baseline, log,
                      forward=not args.no_forward)
    line = {
        "metric": METRIC,
        "value": primary["value"], "unit": primary["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": primary["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": primary["dtype"], "data": "synthetic",
        "config": primary["config"],
        "roofline": primary["roofline"],
    }
    if "cpu_baseline" in primary:
        line["cpu_baseline"] = primary["cpu_baseline"]
    line["detail"] = {k: primary[k] for k in ("tflops", "gbs", "frac_bf16_peak", "frac_hbm",
                                              "cold_vs_warm", "smi_sclk_after_timing",
                                              "kernels_ms_per_step",
                                              "kernels_event_bracketed_ms_per_step",
                                              "workspace_bytes", "ring_bytes",
                                              "d_expanded_x_fp32_bytes", "workspace_vs_MK4",
                                              "plan")}
    for k in ("forward", "dweight", "routing", "unpermute"):
        if k in primary:
            line[k] = primary[k]
    if not args.no_large and args.workload != "large_f16":
        large = measure("large_f16", max(5, args.steps // 2), args.warmup,
                        not args.no_cpu_baseline, log, forward=not args.no_forward)
        line["large"] = {k: large[k] for k in ("value", "unit", "ms_per_step", "tflops", "gbs",
                                               "smi_sclk_after_timing",
                                               "frac_bf16_peak", "roofline", "kernels_ms_per_step",
                                               "kernels_event_bracketed_ms_per_step",
                                               "workspace_bytes", "ring_bytes",
                                               "d_expanded_x_fp32_bytes", "workspace_vs_MK4",
                                               "config", "dtype", "plan")}
        if "cpu_baseline" in large:
            line["large"]["cpu_baseline"] = large["cpu_baseline"]
        for k in ("forward", "dweight", "routing", "unpermute"):
            if k in large:
                line["large"][k] = large[k]
    if not args.no_extra:
        extra = {}
        for name in EXTRA_WORKLOADS:
            if name == args.workload:
                continue
            r = measure(name, max(5, args.steps // 2), args.warmup, not args.no_cpu_baseline, log,
                        forward=False, cold_variant=(name == "mid_bf16"))
            extra[name] = {k: r[k] for k in EXTRA_KEYS if k in r}
            if "cpu_baseline" in r:
                extra[name]["cpu_baseline"] = r["cpu_baseline"]
        line["workloads"] = extra
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
