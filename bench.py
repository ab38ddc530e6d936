"""Benchmark of the zero-computation-expert MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill]
                    [--no-decode] [--no-extra] [--no-backward] [--no-cpu-baseline] [--no-packed]
                    [--no-overlap] [--calib-copy]

One step = one lc_moe_forward (router, permutation, grouped SwiGLU FFN, combine) over the
workload's resident inputs.  Prints ONE JSON line.  value = tokens/s of the whole layer
(inputs and weights already in HBM).  Per-stage times come from HIP events recorded by
lc_moe_forward_staged on the launch stream inside the timed region; step_ms_percentiles
gives p10/p50/p90 of the timed steps' spans (first to last stage event of each step).

roofline: the dominant kernel is the gate/up grouped GEMM (ffn_bf16_pipe_kernel<0>: two
thirds of the FFN FLOPs and weight bytes).  Its algorithmic work per launch: 4*d*I FLOPs
per FFN pick, and as bytes the gate and up weights of every touched expert (2*I*d*2 each)
plus x read once (T*d*2); the per-pick row gathers and the H rows it writes are the
implementation's (implementation_bytes).  The bound is the larger of the two floors
(bytes / 8 TB/s, FLOPs / 2.5 PFLOP/s): HBM at the prefill shape, MFMA for the skewed
layer.  achieved = algorithmic bytes (or FLOPs) per launch over the mean event-timed
launch duration; profile_frac is the same over the mean duration of the committed
rocprofv3 kernel trace of that workload, while the kernel source still matches it.
traffic = HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE counters (scaled by
a plain-copy calibration), read from the committed profile summary and dropped (null)
when the kernel source no longer matches the one the counters were taken on.
small, skewed: the other two bf16 layers, each with its own stage times and roofline.
decode: the decode-shaped layer (T in 64/128/256, zero-expert share 0/33/66%); the FFN
(gate/up + down) is bound by streaming the weights of the experts that received at least
one token; reported against the HBM peak.  Each decode layer is also captured into a HIP
graph and replayed (graph_ms_per_step), run on packed bf16 expert weights (packed_*), and
run on block-FP8 expert weights (fp8_*).
prefill_packed: the prefill layer on packed bf16 expert weights (lc_moe_pack_weights; at
this size the same bits as the row-major weights).
prefill_fp8: the prefill layer on block-FP8 expert weights (lc_moe_quantize_weights).
prefill_fp8_mfma, skewed.fp8_mfma: the layer on block-FP8 weights and block-FP8 activations
(lc_moe_weights.fp8_act), both projections on the FP8 matrix cores, against the FP8 peak.
overlap: a dense SwiGLU FFN (width 2d) over the same tokens beside the layer, serial on one
stream against concurrent on two streams.
backward: lc_moe_ffn_backward (dx and every expert's dW) for the forward's picks and a
seeded dy, timed over its 8 grouped GEMMs' FLOPs.
cpu_baseline: the CPU oracle timed on this host on a bounded sample of the same workload.
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

MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_FP8_PEAK_TFLOPS = 5000.0
HBM_PEAK_GBS = 8000.0
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "ffn_bf16_pipe_kernel_gate_up_prefill_T16384_hbm_traffic.txt")
TRACE_PROFILES = {"prefill": os.path.join(ROOT, "profiles", "ffn_bf16_pipe_kernel_prefill_T16384_kernel_trace.txt"),
                  "skewed": os.path.join(ROOT, "profiles", "ffn_bf16_pipe_kernel_skewed_T32768_kernel_trace.txt")}
GATE_UP_KERNEL = "lcm::ffn_bf16_pipe_kernel<0, false, false>"
KERNEL_SOURCES = [os.path.join(ROOT, "mixture_experts_layer_router_amd", "csrc", f)
                  for f in ("ffn.hip", "common.h", "lds_dma.h")]
METRIC = "MoE-layer tokens/s and % of bf16 MFMA peak (prefill) / % HBM peak (decode)"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profile_fields(path):
    """The machine-read `key: value` lines of a committed profile summary ({} if absent)."""
    kv = {}
    try:
        with open(path) as fh:
            for line in fh:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
    except OSError:
        pass
    return kv


def measured_traffic(workload):
    """HBM bytes per gate/up launch from the committed counter summary, or None when the
    summary is for another workload or another version of the kernel source."""
    kv = profile_fields(TRAFFIC_PROFILE)
    try:
        if kv.get("workload") != workload or kv.get("source_sha256") != kernel_source_hash():
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def profiled_gate_up_us(workload):
    """Mean gate/up launch duration (us) in the committed rocprofv3 kernel trace of this
    workload, or None when there is none or the kernel source has changed since."""
    kv = profile_fields(TRACE_PROFILES.get(workload, ""))
    try:
        if kv.get("workload") != workload or kv.get("source_sha256") != kernel_source_hash():
            return None
        return float(kv["gate_up_avg_us"])
    except (KeyError, ValueError):
        return None


def layer_measures(wl, st, total, stages, steps):
    """Stage times, FFN rates and the gate/up roofline of one timed run of a layer."""
    load = st["outs"]["load"].cpu().numpy()
    nnz = int(load[:wl.N].sum())
    touched = int((load[:wl.N] > 0).sum())
    st_ms = {k: float(np.mean(v)) for k, v in stages.items()}
    gu_flops = 4.0 * wl.d * wl.I * nnz
    dn_flops = 2.0 * wl.d * wl.I * nnz
    gu_bytes = touched * 2.0 * wl.I * wl.d * 2 + wl.T * wl.d * 2.0
    impl_bytes = nnz * (wl.d + wl.I) * 2.0 - wl.T * wl.d * 2.0
    hbm_floor = gu_bytes / (HBM_PEAK_GBS * 1e9) * 1e3
    mfma_floor = gu_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e3
    launch = st_ms["gate_up"]
    gu_gbs = gu_bytes / (launch * 1e-3) / 1e9
    gu_tflops = gu_flops / (launch * 1e-3) / 1e12
    bound = "hbm" if hbm_floor >= mfma_floor else "mfma"
    if bound == "hbm":
        ach, peak, unit = gu_gbs, HBM_PEAK_GBS, "GB/s"
    else:
        ach, peak, unit = gu_tflops, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    prof_us = profiled_gate_up_us(wl.name)
    prof_frac = None
    if prof_us:
        work = gu_bytes / 1e9 if bound == "hbm" else gu_flops / 1e12
        prof_frac = work / (prof_us * 1e-6) / peak
    ffn_ms = st_ms["gate_up"] + st_ms["down"]
    ffn_tflops = (gu_flops + dn_flops) / (ffn_ms * 1e-3) / 1e12
    wbytes = touched * 3 * wl.I * wl.d * 2
    roof = {"bound": bound, "kernel": GATE_UP_KERNEL + " (gate/up + SwiGLU)", "achieved": ach, "peak": peak,
            "unit": unit, "frac": ach / peak, "traffic": measured_traffic(wl.name),
            "algorithmic_bytes": gu_bytes, "implementation_bytes": impl_bytes, "flops_per_launch": gu_flops,
            "hbm_GBps": gu_gbs, "hbm_frac": gu_gbs / HBM_PEAK_GBS,
            "mfma_tflops": gu_tflops, "mfma_frac": gu_tflops / MFMA_BF16_PEAK_TFLOPS,
            "hbm_floor_ms": hbm_floor, "mfma_floor_ms": mfma_floor, "launch_ms": launch,
            "profile_launch_us": prof_us, "profile_frac": prof_frac}
    ffn = {"rows": nnz, "touched_experts": touched, "ms": ffn_ms, "TFLOPs": ffn_tflops,
           "mfma_frac": ffn_tflops / MFMA_BF16_PEAK_TFLOPS, "weight_GBps": wbytes / (ffn_ms * 1e-3) / 1e9}
    return {"ms_per_step": total / steps, "tokens_per_s": wl.T * steps / (total * 1e-3), "stages_ms": st_ms,
            "roofline": roof, "ffn": ffn}


def setup(wl, dev):
    import torch
    import mixture_experts_layer_router_amd as lm
    from inputs.generate import expert_weights, routing_inputs
    ri = routing_inputs(wl)
    w = expert_weights(wl, dev)
    x = ri.x_torch(dev)
    wr, b = ri.w_router_torch(dev), ri.bias_torch(dev)
    shape = lm.make_shape(wl.T, wl.d, wl.N, wl.Z, wl.K, wl.I, lm.BF16 if wl.dtype == "bf16" else lm.F32)
    ws = lm.workspace_for(shape, dev)
    outs = dict(y=torch.empty_like(x),
                idx=torch.empty((wl.T, wl.K), dtype=torch.int32, device=dev),
                gate=torch.empty((wl.T, wl.K), dtype=torch.float32, device=dev),
                load=torch.empty(wl.E, dtype=torch.int32, device=dev))
    wts = lm._weights(wr, b, w["gate"], w["up"], w["down"])
    torch.cuda.synchronize()
    return dict(ri=ri, w=w, x=x, wr=wr, b=b, shape=shape, ws=ws, outs=outs, wts=wts)


def use_fp8(lm, st):
    """Quantize the layer's expert weights to block FP8 and point the forward at them."""
    import torch
    st["fp8"] = lm.quantize_weights(st["w"]["gate"], st["w"]["up"], st["w"]["down"])
    st["wts"] = lm._weights(st["wr"], st["b"], st["w"]["gate"], st["w"]["up"], st["w"]["down"], st["fp8"])
    torch.cuda.synchronize()


def use_packed(lm, st):
    """Re-lay the layer's bf16 expert weights in the packed tile layout and point the
    forward at them (the same values)."""
    import torch
    st["packed"] = lm.pack_weights(st["w"]["gate"], st["w"]["up"], st["w"]["down"])
    st["wts"] = lm._weights(st["wr"], st["b"], st["w"]["gate"], st["w"]["up"], st["w"]["down"], None,
                            st["packed"])
    torch.cuda.synchronize()


def drop_packed(lm, st):
    st.pop("packed", None)
    st["wts"] = lm._weights(st["wr"], st["b"], st["w"]["gate"], st["w"]["up"], st["w"]["down"])


def fp8_mfma_ok(wl):
    """Shapes the FP8 MFMA layer takes (bf16, d and I multiples of 64, up to 16384)."""
    return (wl.dtype == "bf16" and wl.d % 64 == 0 and wl.I % 64 == 0 and wl.d <= 16384 and wl.I <= 16384
            and wl.T * wl.K * wl.I < 2 ** 31)


def fp8_mfma_run(lm, st, wl, steps, warmup, gu_flops, touched):
    """The layer on block-FP8 weights with FP8 activations (lc_moe_weights.fp8_act): x and H
    quantized in 1 x 128 blocks, both projections on the FP8 matrix cores.  The gate_up stage
    includes x's quantization.  Rates against the dense FP8 MFMA peak (5.0 PFLOP/s) and, for
    comparison with the bf16 layer, the bf16 peak."""
    st["wts"] = lm._weights(st["wr"], st["b"], st["w"]["gate"], st["w"]["up"], st["w"]["down"], st["fp8"],
                            None, True)
    total, stages = run_steps(lm, st, steps, warmup)
    sm = {k: float(np.mean(v)) for k, v in stages.items()}
    ffn_ms = sm["gate_up"] + sm["down"]
    gu_tf = gu_flops / (sm["gate_up"] * 1e-3) / 1e12
    ffn_tf = 1.5 * gu_flops / (ffn_ms * 1e-3) / 1e12
    w8 = touched * 3.0 * wl.I * wl.d  # one byte per weight
    out = {"ms_per_step": total / steps, "tokens_per_s": wl.T * steps / (total * 1e-3), "stages_ms": sm,
           "gate_up_tflops": gu_tf, "gate_up_fp8_frac": gu_tf / MFMA_FP8_PEAK_TFLOPS,
           "ffn_ms": ffn_ms, "ffn_tflops": ffn_tf, "ffn_fp8_frac": ffn_tf / MFMA_FP8_PEAK_TFLOPS,
           "ffn_bf16_frac": ffn_tf / MFMA_BF16_PEAK_TFLOPS, "ffn_weight_GBps": w8 / (ffn_ms * 1e-3) / 1e9}
    log(f"{wl.name} FP8 MFMA (FP8 weights and activations): {out['ms_per_step']:.3f} ms/step; gate_up "
        f"{gu_tf:.0f} TFLOP/s ({out['gate_up_fp8_frac']:.1%} of FP8 peak); FFN {ffn_tf:.0f} TFLOP/s "
        f"({out['ffn_fp8_frac']:.1%} of FP8, {out['ffn_bf16_frac']:.1%} of bf16 peak); stages "
        f"{json.dumps({k: round(v, 4) for k, v in sm.items()})}")
    return out


def run_steps(lm, st, steps, warmup):
    """Warm up, then time exactly `steps` forwards; returns (total_ms, per-stage ms lists).
    Each step's span (first to last stage event) is left in st["step_ms"]."""
    import torch
    o = st["outs"]

    def fwd(events=None):
        lm.lc_moe_forward_staged(st["shape"], st["x"], st["wts"], o["y"], o["idx"], o["gate"],
                                 o["load"], st["ws"], stage_events=events)

    for _ in range(warmup):
        fwd()
    nst = lm.NUM_STAGES
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for row in evs:             # torch creates the hipEvent_t on the first record
        for e in row:
            e.record()
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        fwd(evs[i])
    stop.record()
    torch.cuda.synchronize()
    total = start.elapsed_time(stop)
    stages = {lm.stage_name(s): [evs[i][s].elapsed_time(evs[i][s + 1]) for i in range(steps)]
              for s in range(nst)}
    st["step_ms"] = [evs[i][0].elapsed_time(evs[i][nst]) for i in range(steps)]
    return total, stages


def cpu_baseline(st, wl, ffn_budget_s=6.0):
    """Oracle timed on the host: route, permute and combine over all T tokens; the SwiGLU
    FFN on the rows of the first FFN experts, expert by expert until their timed FFN work
    reaches ffn_budget_s (about 10 s of oracle work in all at the prefill layer), scaled to
    nnz.  Copying each expert's weights to the host is not timed."""
    from inputs.generate import weights_f64
    from oracle import moe as orc
    blas_lib = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        blas_threads = max([i.get("num_threads", 1) for i in info] or [1])
        if info:
            blas_lib = f"{info[0].get('internal_api', '?')} {info[0].get('version', '')}".strip()
    except Exception:  # pragma: no cover
        blas_threads = len(os.sched_getaffinity(0))
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), cpu_model)
    except OSError:  # pragma: no cover
        pass
    ri = st["ri"]
    x = ri.x_f64()
    wr = ri.w_router.astype(np.float64)
    t0 = time.perf_counter()
    idx, gate, _ = orc.route(x, wr, ri.bias, wl.K)
    t_route = time.perf_counter() - t0
    t0 = time.perf_counter()
    offsets, perm_token, slot_row = orc.permute(idx, wl.N)
    t_perm = time.perf_counter() - t0
    nnz = int(offsets[-1])
    t_ffn, rows, experts = 0.0, 0, 0
    y_perm = np.zeros((nnz, wl.d))
    for e in range(wl.N):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        wg, wu, wd = (weights_f64(st["w"][k][e]) for k in ("gate", "up", "down"))
        t0 = time.perf_counter()
        y_perm[r0:r1] = orc.swiglu_expert(x[perm_token[r0:r1]], wg, wu, wd)
        t_ffn += time.perf_counter() - t0
        rows += r1 - r0
        experts += 1
        if t_ffn >= ffn_budget_s:
            break
    t0 = time.perf_counter()
    orc.combine(x, y_perm, idx, gate, slot_row, wl.N)
    t_comb = time.perf_counter() - t0
    t_ffn_scaled = t_ffn * nnz / max(rows, 1)
    total = t_route + t_perm + t_ffn_scaled + t_comb
    return {"value": wl.T / total, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "cpu": cpu_model, "blas": blas_lib,
            "sample": (f"fp64 numpy oracle; routing, permutation and combine over all {wl.T} tokens; "
                       f"SwiGLU FFN on the {rows} rows of the first {experts} FFN experts "
                       f"(of {nnz} FFN rows), FFN time scaled by {nnz}/{rows}; "
                       f"route {t_route:.2f}s permute {t_perm:.2f}s ffn {t_ffn:.2f}s "
                       f"(scaled {t_ffn_scaled:.1f}s) combine {t_comb:.2f}s; "
                       f"elementwise numpy on 1 thread, BLAS on {blas_threads}")}


def graph_ms(lm, st, steps):
    """Capture one lc_moe_forward into a HIP graph (torch.cuda.CUDAGraph) and time `steps`
    back-to-back replays with events; returns ms per replay."""
    import torch
    o = st["outs"]

    def fwd():
        lm.lc_moe_forward(st["shape"], st["x"], st["wts"], o["y"], o["idx"], o["gate"], o["load"], st["ws"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    g.replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    del g
    return ms


def backward_run(lm, st, wl, steps, warmup):
    """lc_moe_ffn_backward for the layer's own picks and gates (from the timed forward) and a
    seeded dy; returns ms per call and the rate of its 8 grouped GEMMs (16*d*I FLOPs per FFN
    pick: G and U recomputed, dH, dX (two), dW_down, dW_gate, dW_up)."""
    import torch
    from inputs.generate import upstream_grad
    dev = st["x"].device
    o = st["outs"]
    dy = torch.from_numpy(upstream_grad(wl).view(np.int16)).view(torch.bfloat16).to(dev)
    w = st["w"]
    shape = lm.make_shape(wl.T, wl.d, wl.N, wl.Z, wl.K, wl.I, lm.BF16)
    ws = torch.empty(lm.lc_moe_backward_workspace_size(shape), dtype=torch.uint8, device=dev)
    out = dict(dx=torch.empty_like(st["x"]), dw_gate=torch.empty_like(w["gate"]), dw_up=torch.empty_like(w["up"]),
               dw_down=torch.empty_like(w["down"]))
    wts = lm._weights(None, None, w["gate"], w["up"], w["down"])

    def call():
        lm.lc_moe_ffn_backward(shape, st["x"], wts, o["idx"], o["gate"], dy, out["dx"], out["dw_gate"],
                               out["dw_up"], out["dw_down"], ws)

    for _ in range(warmup):
        call()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        call()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    nnz = int(o["load"][:wl.N].sum())
    flops = 16.0 * wl.d * wl.I * nnz
    res = {"ms": ms, "flops": flops, "TFLOPs": flops / (ms * 1e-3) / 1e12,
           "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    del out, ws
    torch.cuda.empty_cache()
    return res


def dense_ffn_setup(lm, wl, dev, i_dense):
    """A dense SwiGLU FFN over all T tokens (width i_dense), expressed as the layer with one
    FFN expert, no zero experts and K = 1: the router over one expert gives gate 1 exactly,
    so y = FFN(x).  Returns (shape, weights, workspace, outputs)."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    std = 1.0 / np.sqrt(wl.d)
    w = {k: (torch.randn(sh, generator=g, device=dev) * std).to(torch.bfloat16)
         for k, sh in (("gate", (1, i_dense, wl.d)), ("up", (1, i_dense, wl.d)), ("down", (1, wl.d, i_dense)))}
    wr = torch.zeros((1, wl.d), dtype=torch.float32, device=dev)
    b = torch.zeros(1, dtype=torch.float32, device=dev)
    shape = lm.make_shape(wl.T, wl.d, 1, 0, 1, i_dense, lm.BF16)
    ws = lm.workspace_for(shape, dev)
    outs = dict(y=torch.empty((wl.T, wl.d), dtype=torch.bfloat16, device=dev),
                idx=torch.empty((wl.T, 1), dtype=torch.int32, device=dev),
                gate=torch.empty((wl.T, 1), dtype=torch.float32, device=dev),
                load=torch.empty(1, dtype=torch.int32, device=dev))
    return shape, lm._weights(wr, b, w["gate"], w["up"], w["down"]), ws, outs, w


def overlap_run(lm, st, wl, steps, i_dense, stage_ms):
    """The MoE layer and a dense FFN over the same tokens, one after the other on one
    stream, then concurrently on two streams (default priority).  Returns ms per step."""
    import torch
    dev = st["x"].device
    dshape, dwts, dws, douts, _keep = dense_ffn_setup(lm, wl, dev, i_dense)
    o = st["outs"]

    def moe(stream):
        lm.lc_moe_forward(st["shape"], st["x"], st["wts"], o["y"], o["idx"], o["gate"], o["load"], st["ws"],
                          stream=stream)

    def dense(stream):
        lm.lc_moe_forward(dshape, st["x"], dwts, douts["y"], douts["idx"], douts["gate"], douts["load"], dws,
                          stream=stream)

    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(s0)
        for _ in range(steps):
            fn()
        b.record(s0)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    t_moe = timed(lambda: moe(s0))
    t_dense = timed(lambda: dense(s0))
    t_serial = timed(lambda: (moe(s0), dense(s0)))

    def both():
        s1.wait_stream(s0)
        moe(s0)
        dense(s1)
        s0.wait_stream(s1)

    t_conc = timed(both)
    # What one GPU can hide at most: the layer's stages that leave the CUs' load paths free
    # for the dense FFN (route, permute, combine; the grouped FFN kernels already hold every
    # CU's load path), measured in the timed run of the layer.
    ceiling = sum(stage_ms[k] for k in ("route", "permute", "combine"))
    saved = t_serial - t_conc
    return {"dense_I": i_dense, "moe_ms": t_moe, "dense_ms": t_dense, "serial_ms": t_serial,
            "concurrent_ms": t_conc, "saved_frac": 1.0 - t_conc / t_serial, "saved_ms": saved,
            "ceiling_ms": ceiling, "saved_of_ceiling": saved / ceiling if ceiling > 0 else None}


def decode_runs(lm, dev, steps, warmup):
    import torch
    from inputs import configs
    res = []
    for T in configs.DECODE_T:
        for share in configs.DECODE_SHARES:
            wl = configs.decode(T, share)
            st = setup(wl, dev)
            total, stages = run_steps(lm, st, steps, warmup)
            load = st["outs"]["load"].cpu().numpy()
            touched = int((load[:wl.N] > 0).sum())
            wbytes = touched * 3 * wl.I * wl.d * 2
            ffn_ms = float(np.mean(stages["gate_up"]) + np.mean(stages["down"]))
            gbs = wbytes / (ffn_ms * 1e-3) / 1e9
            gms = graph_ms(lm, st, steps)
            use_packed(lm, st)
            totalp, stagesp = run_steps(lm, st, steps, warmup)
            ffnp = float(np.mean(stagesp["gate_up"]) + np.mean(stagesp["down"]))
            gbsp = wbytes / (ffnp * 1e-3) / 1e9
            drop_packed(lm, st)
            use_fp8(lm, st)
            total8, stages8 = run_steps(lm, st, steps, warmup)
            ffn8 = float(np.mean(stages8["gate_up"]) + np.mean(stages8["down"]))
            gbs8 = wbytes / 2 / (ffn8 * 1e-3) / 1e9  # FP8 codes: half the bytes (scales < 0.02%)
            res.append({"T": T, "zero_share_pct": share, "ms_per_step": total / steps,
                        "graph_ms_per_step": gms, "packed_ms_per_step": totalp / steps, "packed_ffn_ms": ffnp,
                        "packed_ffn_weight_GBps": gbsp, "packed_hbm_frac": gbsp / HBM_PEAK_GBS,
                        "fp8_ms_per_step": total8 / steps, "fp8_ffn_ms": ffn8,
                        "fp8_ffn_weight_GBps": gbs8, "fp8_hbm_frac": gbs8 / HBM_PEAK_GBS,
                        "tokens_per_s": T * steps / (total * 1e-3), "touched_experts": touched,
                        "ffn_rows": int(load[:wl.N].sum()), "ffn_ms": ffn_ms,
                        "ffn_weight_GBps": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                        "stages_ms": {k: float(np.mean(v)) for k, v in stages.items()}})
            log(f"decode T={T} share={share}%: {total / steps:.3f} ms/step ({gms:.3f} from a graph), "
                f"FFN {ffn_ms:.3f} ms, {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of HBM peak); "
                f"packed weights FFN {ffnp:.3f} ms, {gbsp:.0f} GB/s ({gbsp / HBM_PEAK_GBS:.1%}); "
                f"FP8 weights {total8 / steps:.3f} ms/step, FFN {ffn8:.3f} ms, {gbs8:.0f} GB/s "
                f"({gbs8 / HBM_PEAK_GBS:.1%})")
            del st
            torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-packed", action="store_true",
                    help="skip the packed-weight runs (they launch the same kernel names as the "
                         "row-major runs, which a per-kernel profile would then mix)")
    ap.add_argument("--no-overlap", action="store_true",
                    help="skip the dense-FFN-beside-the-layer two-stream measurement")
    ap.add_argument("--no-extra", action="store_true", help="skip the small and skewed layers")
    ap.add_argument("--no-backward", action="store_true", help="skip the FFN backward timing")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 4 GiB device copy (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the layer runs on a single MI355X and has no "
              f"multi-GPU path; --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    import mixture_experts_layer_router_amd as lm
    from inputs import configs

    dev = torch.device("cuda:0")
    wl = configs.get(args.workload)
    log(f"workload: {wl.description}")
    st = setup(wl, dev)
    log("inputs resident")
    total, stages = run_steps(lm, st, args.steps, args.warmup)
    ms = total / args.steps
    step_pct = {f"p{q}": float(np.percentile(st["step_ms"], q)) for q in (10, 50, 90)}
    m = layer_measures(wl, st, total, stages, args.steps)
    st_ms, roof, ffn = m["stages_ms"], m["roofline"], m["ffn"]
    touched, nnz = ffn["touched_experts"], ffn["rows"]
    gu_flops, gu_bytes = roof["flops_per_launch"], roof["algorithmic_bytes"]
    log(f"{ms:.3f} ms/step; stages {json.dumps({k: round(v, 4) for k, v in st_ms.items()})}")
    log(f"gate_up {roof['mfma_tflops']:.0f} TFLOP/s ({roof['mfma_frac']:.1%}), {roof['hbm_GBps']:.0f} GB/s "
        f"({roof['hbm_frac']:.1%}); FFN {ffn['TFLOPs']:.0f} TFLOP/s ({ffn['mfma_frac']:.1%}); "
        f"weights {ffn['weight_GBps']:.0f} GB/s")

    if args.calib_copy:
        a = torch.empty(1 << 31, dtype=torch.int16, device=dev)
        bcp = torch.empty_like(a)
        for _ in range(3):
            bcp.copy_(a)
        torch.cuda.synchronize()
        del a, bcp

    result = {
        "metric": METRIC, "value": wl.T * args.steps / (total * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic (seeded; random-init expert weights)",
        "config": {"workload": wl.description, "T": wl.T, "d": wl.d, "N": wl.N, "Z": wl.Z,
                   "K": wl.K, "I": wl.I, "parallelism": "single GPU"},
        "roofline": roof,
        "ffn": ffn,
        "stages_ms": st_ms,
        "step_ms_percentiles": step_pct,
    }
    if not args.no_packed:
        use_packed(lm, st)
        totalp, stagesp = run_steps(lm, st, args.steps, args.warmup)
        stp = {k: float(np.mean(v)) for k, v in stagesp.items()}
        result["prefill_packed"] = {"ms_per_step": totalp / args.steps,
                                    "tokens_per_s": wl.T * args.steps / (totalp * 1e-3), "stages_ms": stp,
                                    "gate_up_GBps": gu_bytes / (stp["gate_up"] * 1e-3) / 1e9,
                                    "gate_up_frac": gu_bytes / (stp["gate_up"] * 1e-3) / 1e9 / HBM_PEAK_GBS}
        log(f"packed weights: {totalp / args.steps:.3f} ms/step; stages "
            f"{json.dumps({k: round(v, 4) for k, v in stp.items()})}")
        drop_packed(lm, st)
        torch.cuda.empty_cache()
    use_fp8(lm, st)
    total8, stages8 = run_steps(lm, st, args.steps, args.warmup)
    st8 = {k: float(np.mean(v)) for k, v in stages8.items()}
    gu8_bytes = touched * 2.0 * wl.I * wl.d + wl.T * wl.d * 2.0  # FP8 codes: one byte per weight
    result["prefill_fp8"] = {"ms_per_step": total8 / args.steps, "tokens_per_s": wl.T * args.steps / (total8 * 1e-3),
                             "stages_ms": st8,
                             "gate_up_GBps": gu8_bytes / (st8["gate_up"] * 1e-3) / 1e9,
                             "gate_up_tflops": gu_flops / (st8["gate_up"] * 1e-3) / 1e12}
    log(f"FP8 weights: {total8 / args.steps:.3f} ms/step; stages "
        f"{json.dumps({k: round(v, 4) for k, v in st8.items()})}")
    if fp8_mfma_ok(wl):
        result["prefill_fp8_mfma"] = fp8_mfma_run(lm, st, wl, args.steps, args.warmup, gu_flops, touched)
    st["wts"] = lm._weights(st["wr"], st["b"], st["w"]["gate"], st["w"]["up"], st["w"]["down"])
    if not args.no_backward and wl.dtype == "bf16":
        run_steps(lm, st, 1, 0)  # the row-major forward's picks and gates
        result["backward"] = backward_run(lm, st, wl, max(3, args.steps // 4), 1)
        bw = result["backward"]
        log(f"backward (dx, dW_gate, dW_up, dW_down): {bw['ms']:.3f} ms, {bw['TFLOPs']:.0f} TFLOP/s "
            f"({bw['mfma_frac']:.1%} of the bf16 peak)")
    if not args.no_overlap:
        result["overlap"] = overlap_run(lm, st, wl, max(3, args.steps // 2), 2 * wl.d, st_ms)
        ov = result["overlap"]
        log(f"dense FFN (I={ov['dense_I']}) beside the layer: moe {ov['moe_ms']:.3f} + dense {ov['dense_ms']:.3f} ms; "
            f"serial {ov['serial_ms']:.3f} ms, two streams {ov['concurrent_ms']:.3f} ms ({ov['saved_frac']:.1%} saved, "
            f"{ov['saved_ms']:.3f} of a {ov['ceiling_ms']:.3f} ms ceiling)")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(st, wl)
        log(f"cpu baseline: {result['cpu_baseline']['value']:.1f} tokens/s")
    del st
    torch.cuda.empty_cache()
    if not args.no_extra:
        for name in ("small", "skewed"):
            if name == wl.name:
                continue
            xw = configs.get(name)
            xst = setup(xw, dev)
            xtotal, xstages = run_steps(lm, xst, args.steps, args.warmup)
            xm = layer_measures(xw, xst, xtotal, xstages, args.steps)
            xm["config"] = {"workload": xw.description, "T": xw.T, "d": xw.d, "N": xw.N, "Z": xw.Z,
                            "K": xw.K, "I": xw.I}
            result[name] = xm
            xr = xm["roofline"]
            log(f"{name}: {xm['ms_per_step']:.3f} ms/step; gate_up {xr['mfma_tflops']:.0f} TFLOP/s "
                f"({xr['mfma_frac']:.1%}), {xr['hbm_GBps']:.0f} GB/s; FFN {xm['ffn']['TFLOPs']:.0f} TFLOP/s "
                f"({xm['ffn']['mfma_frac']:.1%}); bound {xr['bound']} at {xr['frac']:.1%}")
            if fp8_mfma_ok(xw):
                use_fp8(lm, xst)
                xm["fp8_mfma"] = fp8_mfma_run(lm, xst, xw, args.steps, args.warmup, xr["flops_per_launch"],
                                              xm["ffn"]["touched_experts"])
            del xst
            torch.cuda.empty_cache()
    if not args.no_decode:
        result["decode"] = decode_runs(lm, dev, max(5, args.steps), args.warmup)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
