"""Benchmark of the W4A4 microscaling linear layer on one MI355X.

Headline (the JSON line's `value`): MXFP4 W4A4 GEMM throughput in TFLOP/s at
M = 8192 on the MLP prefill pair -- up projection K=5120 -> N=17408 and down
projection K=17408 -> N=5120.  One step is one pass of the serving hot path
over one batch for both projections: per-token CEIL activation quantization
(mx_quantize_act) followed by the block-scaled FP4 GEMM (mx_gemm).  Weights
are packed once beforehand (mx_pack_weights, EVEN rule): packing is the
offline exporter step, and its own time is reported under `rows`.

Also reported under `rows`: the fused-quantization GEMM, decode-shaped GEMMs
(M = 1, 8, 32) in GB/s with weight copies rotated so the 256 MB last-level
cache cannot serve them, the standalone quantizer in GB/s, NVFP4, MXFP8 and
the vocab-sized projection.

`roofline` covers the dominant kernel (mx_gemm) with HIP-event durations of
its launches inside the timed steps; `cpu_baseline` is the CPU oracle timed
on a bounded row sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import platform
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP4 W4A4 GEMM TFLOP/s (M=8192) + GB/s (M<=32) and % of MI355X roofline"
PEAK_TFLOPS = {"fp4": 10100.0, "fp8": 5000.0, "f16": 2500.0}
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--quick", action="store_true", help="headline only (skip the other rows)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time")
    p.add_argument("--kernel-set", action="store_true",
                   help="only run each main kernel a few times on its workload (for rocprofv3 counter passes) "
                        "and exit")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain elementwise copy of known size (the reference point that "
                        "scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings to bytes) and exit")
    return p.parse_args()


COPY_BYTES = 1 << 30


def copy_calibration(torch):
    """Three launches of torch's elementwise negate over a 1 GiB fp32 tensor:
    each reads exactly COPY_BYTES and writes exactly COPY_BYTES."""
    dev = torch.device("cuda:0")
    src = torch.randn(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"read_bytes": COPY_BYTES, "write_bytes": COPY_BYTES,
                                           "launches": 3}}))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this build runs on one GPU only: the hot path is data-parallel "
                          "over tokens with no communication, and multi-GPU runs are not part of it; "
                          "run with --gpus 1"}))
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(torch)
        return

    import fp8_quantized_linear_amd as mxl
    import workloads as W

    if args.kernel_set:
        kernel_set(torch, mxl, W)
        return

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # ------------------------------------------------------------ headline inputs
    t0 = time.time()
    up, down = W.PREFILL_UP, W.PREFILL_DOWN
    host_inputs = {"a_up": up.activations(), "w_up": up.weights(), "a_down": down.activations(),
                   "w_down": down.weights()}
    # SHA-256 of each bf16 input's bytes (row-major), so that another run can
    # show it timed the same data
    input_sha = {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest() for k, v in host_inputs.items()}
    a_up, w_up = to_dev(host_inputs["a_up"]), to_dev(host_inputs["w_up"])
    a_dn, w_dn = to_dev(host_inputs["a_down"]), to_dev(host_inputs["w_down"])
    del host_inputs
    log(f"inputs generated in {time.time() - t0:.1f}s")

    # offline weight packing (timed separately)
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record()
    wq_up, ws_up = mxl.mx_pack_weights(w_up, "mxfp4", "even")
    wq_dn, ws_dn = mxl.mx_pack_weights(w_dn, "mxfp4", "even")
    e1.record()
    torch.cuda.synchronize()
    pack_ms = e0.elapsed_time(e1)

    aq_up = torch.empty((up.m, up.k // 2), dtype=torch.uint8, device=dev)
    as_up = torch.empty((up.m, up.k // 32), dtype=torch.uint8, device=dev)
    aq_dn = torch.empty((down.m, down.k // 2), dtype=torch.uint8, device=dev)
    as_dn = torch.empty((down.m, down.k // 32), dtype=torch.uint8, device=dev)
    y_up = torch.empty((up.m, up.n), dtype=torch.bfloat16, device=dev)
    y_dn = torch.empty((down.m, down.n), dtype=torch.bfloat16, device=dev)

    def step(events=None):
        mxl.mx_quantize_act(a_up, "mxfp4", "ceil", out=(aq_up, as_up))
        if events is not None:
            events[0].record()
        mxl.mx_gemm(aq_up, as_up, wq_up, ws_up, up.k, y=y_up)
        if events is not None:
            events[1].record()
        mxl.mx_quantize_act(a_dn, "mxfp4", "ceil", out=(aq_dn, as_dn))
        if events is not None:
            events[2].record()
        mxl.mx_gemm(aq_dn, as_dn, wq_dn, ws_dn, down.k, y=y_dn)
        if events is not None:
            events[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[ev() for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / args.steps
    step_flops = up.flops + down.flops
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    gemm_up_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    gemm_dn_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    achieved = step_flops / ((gemm_up_ms + gemm_dn_ms) * 1e-3) / 1e12
    log(f"step {ms_per_step:.3f} ms -> {value:.1f} TFLOP/s; gemm up {gemm_up_ms * 1e3:.1f} us, "
        f"down {gemm_dn_ms * 1e3:.1f} us")

    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_TFLOPS["fp4"],
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["fp4"], 4),
                "traffic": traffic_from_profiles(),
                "kernel": mxl.mx_gemm_plan("mxfp4", "mxfp4", up.m, up.n, up.k),
                "per_launch_us": {"up": round(gemm_up_ms * 1e3, 2), "down": round(gemm_dn_ms * 1e3, 2)},
                "algorithmic_flop_per_launch": up.flops}

    # the graphics clock under this load (power-limited, below the 2.4 GHz of
    # the spec peak), and the peak and fraction at that clock
    clock = measure_gfxclk(lambda: (mxl.mx_gemm(aq_up, as_up, wq_up, ws_up, up.k, y=y_up),
                                    mxl.mx_gemm(aq_dn, as_dn, wq_dn, ws_dn, down.k, y=y_dn)), torch)
    if clock.get("gfxclk_mhz"):
        peak_clk = PEAK_TFLOPS["fp4"] * clock["gfxclk_mhz"] / 2400.0
        roofline["peak_at_measured_clock"] = round(peak_clk, 1)
        roofline["frac_at_measured_clock"] = round(achieved / peak_clk, 4)
    roofline["clock"] = clock

    rows = {"pack_weights_ms": round(pack_ms, 3)}
    if not args.quick:
        rows.update(extra_rows(torch, mxl, W, dev, to_dev, a_up, wq_up, ws_up, a_dn, wq_dn, ws_dn))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(up, args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "mxfp4",
        "data": "synthetic (seeded N(0,1) activations with 1% x20 outliers, N(0,0.02) weights)",
        "config": {"workload": "mxfp4 MLP prefill pair: up 8192x5120x17408 + down 8192x17408x5120, "
                               "per-token CEIL quantize + block-scaled FP4 GEMM, bf16 out",
                   "m": up.m, "k_up": up.k, "n_up": up.n, "k_down": down.k, "n_down": down.n,
                   "step_flop": step_flops},
        "inputs_sha256": input_sha,
        "host": host_info(torch),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(out))


def kernel_set(torch, mxl, W, reps: int = 3):
    """Each main kernel `reps` times on its workload, launch order fixed, for
    per-kernel rocprofv3 counter passes (one kernel name per workload)."""
    dev = torch.device("cuda:0")

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def run(name, fn):
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        log(f"kernel-set: {name}")

    up, down = W.PREFILL_UP, W.PREFILL_DOWN
    for cfg in (up, down):
        a, w = to_dev(cfg.activations()), to_dev(cfg.weights())
        wq, ws = mxl.mx_pack_weights(w, "mxfp4", "even")
        aq, as_ = mxl.mx_quantize_act(a, "mxfp4", "ceil")
        y = torch.empty((cfg.m, cfg.n), dtype=torch.bfloat16, device=dev)
        run(f"quantize {cfg.name}", lambda: mxl.mx_quantize_act(a, "mxfp4", "ceil", out=(aq, as_)))
        run(f"gemm {cfg.name}", lambda: mxl.mx_gemm(aq, as_, wq, ws, cfg.k, y=y))
        run(f"fused in-GEMM {cfg.name}", lambda: mxl.mx_gemm_fused(a, wq, ws, y=y, in_gemm=True))
        del a, w, wq, ws, aq, as_, y
    c8 = W.MXFP8_ATTN
    a = to_dev(c8.activations())
    wq, ws = mxl.mx_pack_weights(to_dev(c8.weights()), "mxfp8", "floor")
    aq, as_ = mxl.mx_quantize_act(a, "mxfp8", "ceil")
    y = torch.empty((c8.m, c8.n), dtype=torch.bfloat16, device=dev)
    run(c8.name, lambda: mxl.mx_gemm(aq, as_, wq, ws, c8.k, "mxfp8", "mxfp8", y=y))
    nv = W.NVFP4
    a, w = to_dev(nv.activations()), to_dev(nv.weights())
    g_a = mxl.mx_nv_global_scale(float(mxl.mx_tensor_amax(a).item()))
    g_w = mxl.mx_nv_global_scale(float(mxl.mx_tensor_amax(w).item()))
    aq, as_ = mxl.mx_quantize_act(a, "nvfp4", global_scale=g_a)
    wq, ws = mxl.mx_pack_weights(w, "nvfp4", global_scale=g_w)
    y = torch.empty((nv.m, nv.n), dtype=torch.bfloat16, device=dev)
    run(f"quantize {nv.name}", lambda: mxl.mx_quantize_act(a, "nvfp4", global_scale=g_a, out=(aq, as_)))
    run(nv.name, lambda: mxl.nv_gemm(aq, as_, wq, ws, nv.k, 1.0 / (g_a * g_w), y=y))
    dec = W.DECODE[0]
    wq, ws = mxl.mx_pack_weights(to_dev(dec.weights()), "mxfp4", "even")
    for cfg in W.DECODE:
        a = to_dev(cfg.activations())
        aq, as_ = mxl.mx_quantize_act(a)
        y = torch.empty((cfg.m, cfg.n), dtype=torch.bfloat16, device=dev)
        run(cfg.name, lambda: mxl.mx_gemm(aq, as_, wq, ws, cfg.k, y=y))
        if cfg.m <= 16:
            run(f"w4a16 {cfg.name}", lambda: mxl.mx_gemm_w4a16(a, wq, ws, "mxfp4", y=y))
    # NVFP4 W4A4 and W8A8 MXFP8 decode, M = 1
    cfg = W.DECODE[0]
    w, a = to_dev(cfg.weights()), to_dev(cfg.activations())
    g_w = mxl.mx_nv_global_scale(float(mxl.mx_tensor_amax(w).item()))
    g_a = mxl.mx_nv_global_scale(float(mxl.mx_tensor_amax(a).item()))
    wq, ws = mxl.mx_pack_weights(w, "nvfp4", global_scale=g_w)
    aq, as_ = mxl.mx_quantize_act(a, "nvfp4", global_scale=g_a)
    y = torch.empty((cfg.m, cfg.n), dtype=torch.bfloat16, device=dev)
    run(f"nvfp4 {cfg.name}", lambda: mxl.nv_gemm(aq, as_, wq, ws, cfg.k, 1.0 / (g_a * g_w), y=y))
    wq, ws = mxl.mx_pack_weights(w, "mxfp8", "floor")
    aq, as_ = mxl.mx_quantize_act(a, "mxfp8", "ceil")
    run(f"mxfp8 {cfg.name}", lambda: mxl.mx_gemm(aq, as_, wq, ws, cfg.k, "mxfp8", "mxfp8", y=y))
    print(json.dumps({"kernel_set": "done", "reps": reps}))


def measure_gfxclk(step, torch, seconds: float = 2.5):
    """Median graphics clock (MHz) reported by amdsmi (current_gfxclk, which
    the driver refreshes about once a second) while `step` runs back to back
    for `seconds`; samples from the first second are dropped."""
    import threading
    import time
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
        amdsmi.amdsmi_get_gpu_metrics_info(handle)
    except Exception as e:   # no amdsmi or no access on this machine
        return {"gfxclk_mhz": None, "error": repr(e)[:200]}
    samples, stop = [], [False]
    t0 = time.time()

    def sampler():
        while not stop[0]:
            try:
                mhz = amdsmi.amdsmi_get_gpu_metrics_info(handle).get("current_gfxclk")
                if isinstance(mhz, (int, float)) and time.time() - t0 > 1.0:
                    samples.append(float(mhz))
            except Exception:
                pass
            time.sleep(0.01)

    th = threading.Thread(target=sampler)
    th.start()
    while time.time() - t0 < seconds:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    stop[0] = True
    th.join()
    if not samples:
        return {"gfxclk_mhz": None, "error": "no samples"}
    return {"gfxclk_mhz": float(np.median(samples)), "samples": len(samples),
            "source": "amdsmi current_gfxclk during back-to-back headline GEMMs"}


def traffic_from_profiles():
    """HBM bytes per mx_gemm launch from the committed rocprofv3 PMC summary, if
    it was taken on the current kernel source (else null)."""
    path = os.path.join(ROOT, "profiles", "mx_gemm_prefill_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_sha():
        return None
    return rec.get("traffic_bytes_per_launch")


# the sources of mx_gemm_prefill_kernel (the kernel the traffic record covers)
PREFILL_SOURCES = ("mx_device.h", "gemm_prefill.hip", "gemm_prefill_tile.inc", "gemm_tile_epilogue.inc")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in PREFILL_SOURCES:
        h.update(open(os.path.join(ROOT, "fp8_quantized_linear_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def _median_ms(torch, fn, iters, warmup=3):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for i, (a, b) in enumerate(evs):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    return float(np.median(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90))


def _median_interleaved_ms(torch, fns, iters, warmup=2):
    """Median event time of each call in fns, the calls alternating (fns[0],
    fns[1], ..., fns[0], ...), so that all of them see the same clock: the
    graphics clock of this chip drifts with power from call to call."""
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
           for _ in range(iters)]
    for row in evs:
        for f, (a, b) in zip(fns, row):
            a.record()
            f()
            b.record()
    torch.cuda.synchronize()
    return [float(np.median([row[j][0].elapsed_time(row[j][1]) for row in evs])) for j in range(len(fns))]


def extra_rows(torch, mxl, W, dev, to_dev, a_up, wq_up, ws_up, a_dn, wq_dn, ws_dn):
    rows = {}
    up, down = W.PREFILL_UP, W.PREFILL_DOWN
    # fused quantization prologue (the quantizer into the workspace, then the
    # GEMM; and the one-launch form) against the standalone pair, interleaved
    fused = {}
    for name, cfg, a, wq, ws in (("up", up, a_up, wq_up, ws_up), ("down", down, a_dn, wq_dn, ws_dn)):
        y = torch.empty((cfg.m, cfg.n), dtype=torch.bfloat16, device=dev)
        aq = torch.empty((cfg.m, cfg.k // 2), dtype=torch.uint8, device=dev)
        as_ = torch.empty((cfg.m, cfg.k // 32), dtype=torch.uint8, device=dev)

        def pair(a=a, wq=wq, ws=ws, y=y, aq=aq, as_=as_, k=cfg.k):
            mxl.mx_quantize_act(a, "mxfp4", "ceil", out=(aq, as_))
            mxl.mx_gemm(aq, as_, wq, ws, k, y=y)
        t_f, t_p, t_g = _median_interleaved_ms(
            torch, [lambda: mxl.mx_gemm_fused(a, wq, ws, y=y), pair,
                    lambda: mxl.mx_gemm_fused(a, wq, ws, y=y, in_gemm=True)], 10)
        fused[name] = (t_f, t_p, t_g)
        del y, aq, as_
    (fu, pu, gu), (fd, pd, gd) = fused["up"], fused["down"]
    rows["fused_prefill"] = {"up_us": round(fu * 1e3, 1), "down_us": round(fd * 1e3, 1),
                             "tflops": round((up.flops + down.flops) / ((fu + fd) * 1e-3) / 1e12, 1),
                             "pair_up_us": round(pu * 1e3, 1), "pair_down_us": round(pd * 1e3, 1),
                             "in_gemm_up_us": round(gu * 1e3, 1), "in_gemm_down_us": round(gd * 1e3, 1),
                             "timing": "median of 10 interleaved calls each: mx_gemm_fused (default), "
                                       "mx_quantize_act + mx_gemm (pair), mx_gemm_fused one-launch form"}
    log(f"fused: up {fu * 1e3:.1f} us (pair {pu * 1e3:.1f}, one launch {gu * 1e3:.1f}); "
        f"down {fd * 1e3:.1f} us (pair {pd * 1e3:.1f}, one launch {gd * 1e3:.1f})")

    # standalone quantizer GB/s (inputs rotated through 4 copies: > 256 MB)
    for name, cfg, a in (("up", up, a_up), ("down", down, a_dn)):
        copies = [a] + [a.clone() for _ in range(3)]
        q = torch.empty((cfg.m, cfg.k // 2), dtype=torch.uint8, device=dev)
        s = torch.empty((cfg.m, cfg.k // 32), dtype=torch.uint8, device=dev)
        med, p10, p90 = _median_ms(torch, lambda i: mxl.mx_quantize_act(copies[i % 4], out=(q, s)), 20)
        nbytes = cfg.m * cfg.k * 2 + cfg.m * cfg.k // 2 + cfg.m * cfg.k // 32
        rows[f"quantizer_{name}"] = {"us": round(med * 1e3, 2), "GBps": round(nbytes / (med * 1e-3) / 1e9, 1),
                                     "frac_hbm": round(nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
                                     "bytes": nbytes}
        del copies

    # the gated MLP block: gate_up projection (8192 x 5120 x 34816) with the
    # SwiGLU + CEIL MXFP4 epilogue fused, then the down projection; against
    # the unfused chain (bf16 gate_up output, standalone SwiGLU quantization)
    mlp = W.MLP_GATE_UP
    inter = mlp.n // 2
    w_gu = to_dev(mlp.weights())
    wq_gu, ws_gu = mxl.mx_pack_weights(w_gu, "mxfp4", "even")
    del w_gu
    wq_il, ws_il = mxl.interleave_gate_up(wq_gu), mxl.interleave_gate_up(ws_gu)
    aq_m, as_m = mxl.mx_quantize_act(a_up, "mxfp4", "ceil")
    hq = torch.empty((mlp.m, inter // 2), dtype=torch.uint8, device=dev)
    hs = torch.empty((mlp.m, inter // 32), dtype=torch.uint8, device=dev)
    y_gu = torch.empty((mlp.m, mlp.n), dtype=torch.bfloat16, device=dev)
    y_dn = torch.empty((down.m, down.n), dtype=torch.bfloat16, device=dev)
    t_fused, _, _ = _median_ms(torch, lambda i: mxl.mx_gemm_swiglu_quant(aq_m, as_m, wq_il, ws_il, mlp.k,
                                                                         out=(hq, hs)), 10)
    t_gemm, _, _ = _median_ms(torch, lambda i: mxl.mx_gemm(aq_m, as_m, wq_gu, ws_gu, mlp.k, y=y_gu), 10)
    t_act, _, _ = _median_ms(torch, lambda i: mxl.mx_swiglu_quant(y_gu, out=(hq, hs)), 10)
    t_down, _, _ = _median_ms(torch, lambda i: mxl.mx_gemm(hq, hs, wq_dn, ws_dn, down.k, y=y_dn), 10)
    block_flops = mlp.flops + down.flops
    rows["mlp_block"] = {
        "gate_up_swiglu_fused_us": round(t_fused * 1e3, 1),
        "gate_up_gemm_us": round(t_gemm * 1e3, 1), "swiglu_quant_us": round(t_act * 1e3, 1),
        "down_us": round(t_down * 1e3, 1),
        "fused_block_tflops": round(block_flops / ((t_fused + t_down) * 1e-3) / 1e12, 1),
        "unfused_block_tflops": round(block_flops / ((t_gemm + t_act + t_down) * 1e-3) / 1e12, 1)}
    log(f"mlp block: fused gate_up+swiglu {t_fused * 1e3:.1f} us vs gemm {t_gemm * 1e3:.1f} + act "
        f"{t_act * 1e3:.1f} us; down {t_down * 1e3:.1f} us")
    del wq_gu, ws_gu, wq_il, ws_il, y_gu, y_dn, hq, hs

    # fake quantization (training forward: quantize -> dequantize -> bf16),
    # GB/s over bf16 in + bf16 out, inputs rotated through 4 copies
    cfg = up
    copies = [a_up] + [a_up.clone() for _ in range(3)]
    yq = torch.empty_like(a_up)
    g_fq = mxl.mx_nv_global_scale(float(mxl.mx_tensor_amax(a_up).item()))
    for name, fmt, rule, g in (("mxfp4_ceil", "mxfp4", "ceil", 1.0), ("mxfp8_ceil", "mxfp8", "ceil", 1.0),
                               ("nvfp4", "nvfp4", None, g_fq)):
        med, _, _ = _median_ms(torch, lambda i: mxl.mx_fake_quant(copies[i % 4], fmt, rule, g, out=yq), 20)
        nbytes = cfg.m * cfg.k * 4
        rows[f"fake_quant_{name}"] = {"us": round(med * 1e3, 2), "GBps": round(nbytes / (med * 1e-3) / 1e9, 1),
                                      "frac_hbm": round(nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
                                      "bytes": nbytes}
        log(f"fake_quant {name}: {med * 1e3:.2f} us {nbytes / (med * 1e-3) / 1e9:.0f} GB/s")
    del copies, yq

    # decode-shaped GEMMs, weights rotated through 11 copies (> 512 MB).  A
    # call takes a few microseconds, less than the host needs to submit one,
    # so the 11 calls are captured once in a HIP graph and the graph is
    # replayed; the output of every timed replay is checked against the eager
    # result of the same call.
    dec = W.DECODE[0]
    w_bits = to_dev(dec.weights())
    wq0, ws0 = mxl.mx_pack_weights(w_bits, "mxfp4", "even")
    del w_bits
    wcopies = [(wq0, ws0)] + [(wq0.clone(), ws0.clone()) for _ in range(10)]
    for cfg in W.DECODE:
        a = to_dev(cfg.activations())
        aq, as_ = mxl.mx_quantize_act(a)
        yd = torch.empty((cfg.m, cfg.n), dtype=torch.bfloat16, device=dev)
        ref = mxl.mx_gemm(aq, as_, wcopies[10][0], wcopies[10][1], cfg.k).clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(3):
                mxl.mx_gemm(aq, as_, wcopies[i][0], wcopies[i][1], cfg.k, y=yd)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(11):
                mxl.mx_gemm(aq, as_, wcopies[i][0], wcopies[i][1], cfg.k, y=yd)
        torch.cuda.synchronize()
        times = []
        for rep in range(25):
            yd.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            if not torch.equal(yd, ref):
                raise RuntimeError(f"decode m={cfg.m}: graph replay {rep} differs from the eager result")
            times.append(e0.elapsed_time(e1) / 11)
        t = np.array(times[3:])
        med, p10, p90 = float(np.median(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90))
        nbytes = (cfg.m + cfg.n) * (cfg.k // 2 + cfg.k // 32) + cfg.m * cfg.n * 2
        gbs = nbytes / (med * 1e-3) / 1e9
        rows[f"decode_m{cfg.m}"] = {"us": round(med * 1e3, 2), "p10_us": round(p10 * 1e3, 2),
                                    "p90_us": round(p90 * 1e3, 2), "GBps": round(gbs, 1),
                                    "frac_hbm": round(gbs / PEAK_HBM_GBS, 3), "bytes": nbytes,
                                    "timing": "HIP graph of 11 back-to-back calls (one per weight copy), replayed",
                                    "kernel": mxl.mx_gemm_plan("mxfp4", "mxfp4", cfg.m, cfg.n, cfg.k)}
        log(f"decode m={cfg.m}: {med * 1e3:.2f} us {gbs:.0f} GB/s")
        del graph

    # W4A16 (weight-only) decode on the same shapes: bf16 activations times
    # the MXFP4 copies above, then times NVFP4 packings of the same weights
    def graph_rows(call, name, nbytes, plan, m):
        yd = call(10).clone()
        ref = yd.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(3):
                call(i, yd)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(11):
                call(i, yd)
        torch.cuda.synchronize()
        times = []
        for rep in range(25):
            yd.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            if not torch.equal(yd, ref):
                raise RuntimeError(f"{name}: graph replay {rep} differs from the eager result")
            times.append(e0.elapsed_time(e1) / 11)
        t = np.array(times[3:])
        med, p10, p90 = float(np.median(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90))
        gbs = nbytes / (med * 1e-3) / 1e9
        rows[name] = {"us": round(med * 1e3, 2), "p10_us": round(p10 * 1e3, 2), "p90_us": round(p90 * 1e3, 2),
                      "GBps": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 3), "bytes": nbytes,
                      "timing": "HIP graph of 11 back-to-back calls (one per weight copy), replayed",
                      "kernel": plan}
        log(f"{name}: {med * 1e3:.2f} us {gbs:.0f} GB/s")

    w_bits_dev = to_dev(dec.weights())
    g_w = mxl.mx_nv_global_scale(float(mxl.mx_tensor_amax(w_bits_dev).item()))
    nq0, ns0 = mxl.mx_pack_weights(w_bits_dev, "nvfp4", global_scale=g_w)
    del w_bits_dev
    ncopies = [(nq0, ns0)] + [(nq0.clone(), ns0.clone()) for _ in range(10)]
    alpha_nv = float(np.float32(1.0) / np.float32(g_w))
    for cfg in [c for c in W.DECODE if c.m <= 16]:
        a = to_dev(cfg.activations())
        for fmt, copies, alpha in (("mxfp4", wcopies, 1.0), ("nvfp4", ncopies, alpha_nv)):
            def call(i, y=None, fmt=fmt, copies=copies, alpha=alpha, a=a):
                return mxl.mx_gemm_w4a16(a, copies[i][0], copies[i][1], fmt, alpha, y=y)
            kb = cfg.k // (16 if fmt == "nvfp4" else 32)
            nbytes = cfg.n * (cfg.k // 2 + kb) + cfg.m * cfg.k * 2 + cfg.m * cfg.n * 2
            graph_rows(call, f"w4a16_{fmt}_decode_m{cfg.m}", nbytes,
                       mxl.mx_gemm_w4a16_plan(fmt, cfg.m, cfg.n, cfg.k), cfg.m)
    del wcopies

    # W4A4 NVFP4 (the NVFP4 copies above) and W8A8 MXFP8 (FLOOR packings of
    # the same weights) decode on the same shapes
    w_bits_dev = to_dev(dec.weights())
    fq0, fs0 = mxl.mx_pack_weights(w_bits_dev, "mxfp8", "floor")
    del w_bits_dev
    fcopies = [(fq0, fs0)] + [(fq0.clone(), fs0.clone()) for _ in range(10)]
    for cfg in [c for c in W.DECODE if c.m <= 16]:
        a = to_dev(cfg.activations())
        g_a = mxl.mx_nv_global_scale(float(mxl.mx_tensor_amax(a).item()))
        naq, nas = mxl.mx_quantize_act(a, "nvfp4", global_scale=g_a)
        alpha = float(np.float32(1.0) / (np.float32(g_a) * np.float32(g_w)))

        def call_nv(i, y=None, naq=naq, nas=nas, alpha=alpha, k=cfg.k):
            return mxl.nv_gemm(naq, nas, ncopies[i][0], ncopies[i][1], k, alpha, y=y)
        nbytes = (cfg.m + cfg.n) * (cfg.k // 2 + cfg.k // 16) + cfg.m * cfg.n * 2
        graph_rows(call_nv, f"nvfp4_decode_m{cfg.m}", nbytes,
                   mxl.mx_gemm_plan("nvfp4", "nvfp4", cfg.m, cfg.n, cfg.k), cfg.m)
        faq, fas = mxl.mx_quantize_act(a, "mxfp8", "ceil")

        def call_f8(i, y=None, faq=faq, fas=fas, k=cfg.k):
            return mxl.mx_gemm(faq, fas, fcopies[i][0], fcopies[i][1], k, "mxfp8", "mxfp8", y=y)
        nbytes = (cfg.m + cfg.n) * (cfg.k + cfg.k // 32) + cfg.m * cfg.n * 2
        graph_rows(call_f8, f"mxfp8_decode_m{cfg.m}", nbytes,
                   mxl.mx_gemm_plan("mxfp8", "mxfp8", cfg.m, cfg.n, cfg.k), cfg.m)
    del ncopies, fcopies

    # NVFP4 W4A4
    nv = W.NVFP4
    run = 0.0
    for b in nv.calibration_batches():
        run = max(run, float(mxl.mx_tensor_amax(to_dev(b)).item()))
    g_a = mxl.mx_nv_global_scale(run)
    a = to_dev(nv.activations())
    w = to_dev(nv.weights())
    g_w = mxl.mx_nv_global_scale(float(mxl.mx_tensor_amax(w).item()))
    wq, ws = mxl.mx_pack_weights(w, "nvfp4", global_scale=g_w)
    aq, as_ = mxl.mx_quantize_act(a, "nvfp4", global_scale=g_a)
    alpha = float(np.float32(1.0) / (np.float32(g_a) * np.float32(g_w)))
    yn = torch.empty((nv.m, nv.n), dtype=torch.bfloat16, device=dev)
    med, _, _ = _median_ms(torch, lambda i: mxl.nv_gemm(aq, as_, wq, ws, nv.k, alpha, y=yn), 20)
    tf = nv.flops / (med * 1e-3) / 1e12
    rows["nvfp4"] = {"us": round(med * 1e3, 1), "tflops": round(tf, 1),
                     "frac_f16_peak": round(tf / PEAK_TFLOPS["f16"], 3),
                     "frac_fp4_peak": round(tf / PEAK_TFLOPS["fp4"], 4)}
    log(f"nvfp4: {med * 1e3:.1f} us {tf:.0f} TFLOP/s")
    del a, w, wq, ws, aq, as_, yn

    # MXFP8 attention projection and the vocab-sized MXFP4 projection on the same A
    c8, cv = W.MXFP8_ATTN, W.MXFP4_VOCAB
    a = to_dev(c8.activations())
    w8 = to_dev(c8.weights())
    wq8, ws8 = mxl.mx_pack_weights(w8, "mxfp8", "floor")
    del w8
    aq8, as8 = mxl.mx_quantize_act(a, "mxfp8", "ceil")
    y8 = torch.empty((c8.m, c8.n), dtype=torch.bfloat16, device=dev)
    med, _, _ = _median_ms(torch, lambda i: mxl.mx_gemm(aq8, as8, wq8, ws8, c8.k, "mxfp8", "mxfp8", y=y8), 20)
    tf8 = c8.flops / (med * 1e-3) / 1e12
    rows["mxfp8_attn"] = {"us": round(med * 1e3, 1), "tflops": round(tf8, 1),
                          "frac_fp8_peak": round(tf8 / PEAK_TFLOPS["fp8"], 3)}
    log(f"mxfp8: {med * 1e3:.1f} us {tf8:.0f} TFLOP/s")
    del wq8, ws8, y8, aq8, as8
    wv = to_dev(cv.weights())
    wqv, wsv = mxl.mx_pack_weights(wv, "mxfp4", "even")
    del wv
    aqv, asv = mxl.mx_quantize_act(a)
    yv = torch.empty((cv.m, cv.n), dtype=torch.bfloat16, device=dev)
    med, _, _ = _median_ms(torch, lambda i: mxl.mx_gemm(aqv, asv, wqv, wsv, cv.k, y=yv), 10, warmup=2)
    tfv = cv.flops / (med * 1e-3) / 1e12
    rows["mxfp4_vocab"] = {"us": round(med * 1e3, 1), "tflops": round(tfv, 1),
                           "frac_fp4_peak": round(tfv / PEAK_TFLOPS["fp4"], 3)}
    log(f"vocab: {med * 1e3:.1f} us {tfv:.0f} TFLOP/s")
    del wqv, wsv, aqv, asv, yv

    # small-N projections (the 96-wide fused in_proj_ba, MXFP8 and MXFP4) and
    # a 512-token chunk: too few output tiles to fill the GPU, so the library
    # splits K (workspace) -- timed with and without the split, per call from
    # a HIP graph of 10 back-to-back calls
    def graph_us(fn, reps=10):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=side):
                for _ in range(reps):
                    fn()
        torch.cuda.current_stream().wait_stream(side)
        graph.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(15):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / reps)
        return float(np.median(ts[3:]))

    # c1, the small 16 x 256 x 256 configuration: launch-bound; one quantize +
    # GEMM pair per call
    c1 = W.SMALL
    a1 = to_dev(c1.activations())
    wq1, ws1 = mxl.mx_pack_weights(to_dev(c1.weights()), "mxfp4", "even")
    aq1 = torch.empty((c1.m, c1.k // 2), dtype=torch.uint8, device=dev)
    as1 = torch.empty((c1.m, c1.k // 32), dtype=torch.uint8, device=dev)
    y1 = torch.empty((c1.m, c1.n), dtype=torch.bfloat16, device=dev)
    t_q = graph_us(lambda: mxl.mx_quantize_act(a1, out=(aq1, as1)))
    t_g = graph_us(lambda: mxl.mx_gemm(aq1, as1, wq1, ws1, c1.k, y=y1))
    rows["small_c1_16x256x256"] = {"quantize_us": round(t_q, 2), "gemm_us": round(t_g, 2),
                                   "kernel": mxl.mx_gemm_plan("mxfp4", "mxfp4", c1.m, c1.n, c1.k),
                                   "timing": "HIP graph of 10 back-to-back calls, replayed"}
    log(f"c1 16x256x256: quantize {t_q:.2f} us, gemm {t_g:.2f} us")

    for name, fmt, m, n in (("mxfp8_n96_m4096", "mxfp8", 4096, 96), ("mxfp8_n96_m1", "mxfp8", 1, 96),
                            ("mxfp4_n96_m4096", "mxfp4", 4096, 96), ("mxfp4_n2048_m512", "mxfp4", 512, 2048)):
        k = 5120
        ws_ = to_dev(W.normal_bf16(n, k, 0.02, 1))
        wq_, wsc_ = mxl.mx_pack_weights(ws_, fmt, "floor" if fmt == "mxfp8" else "even")
        a_ = to_dev(W.activations_entry_outliers(m, k))
        aq_, as_ = mxl.mx_quantize_act(a_, fmt, "ceil")
        y_ = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        t_split = graph_us(lambda: mxl.mx_gemm(aq_, as_, wq_, wsc_, k, fmt, fmt, y=y_))
        t_one = graph_us(lambda: mxl.mx_gemm(aq_, as_, wq_, wsc_, k, fmt, fmt, y=y_, split_k=False))
        rows[f"small_{name}"] = {"us": round(t_split, 2), "unsplit_us": round(t_one, 2),
                                 "tflops": round(2 * m * n * k / (t_split * 1e-6) / 1e12, 1),
                                 "kernel": mxl.mx_gemm_plan(fmt, fmt, m, n, k),
                                 "timing": "HIP graph of 10 back-to-back calls, replayed"}
        log(f"small {name}: {t_split:.1f} us (unsplit {t_one:.1f} us)")
        del ws_, wq_, wsc_, a_, aq_, as_, y_
    return rows


def host_info(torch):
    """CPU model and logical CPU count of the host, and the GPU's name."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model or platform.processor() or "unknown", "logical_cpus": os.cpu_count(),
            "gpu": torch.cuda.get_device_name(0)}


def cpu_baseline(cfg, target_s):
    """The CPU oracle on a contiguous sample of activation rows of the up
    projection: CEIL quantization of those rows plus their full output rows
    from codes (weights packed by the oracle beforehand, untimed like the
    GPU's packing).  Rows are doubled until the run takes ~target_s."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    a_bits = cfg.activations(m=512)
    w_bits = cfg.weights()
    wq, ws = oracle.mx_quantize("e2m1", "even", w_bits, nthreads=threads)
    rows, took = 2, 0.0
    while True:
        t = time.perf_counter()
        aq, as_ = oracle.mx_quantize("e2m1", "ceil", np.ascontiguousarray(a_bits[:rows]), nthreads=threads)
        oracle.mx_gemm("e2m1", aq, as_, "e2m1", wq, ws, rows, cfg.n, cfg.k, nthreads=threads)
        took = time.perf_counter() - t
        if took >= target_s / 2 or rows >= 512:
            break
        rows *= 2
    flops = 2 * rows * cfg.n * cfg.k
    return {"value": round(flops / took / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of 8192 activation rows of the up projection (K=5120, N=17408): oracle CEIL "
                      f"quantization + fp64 GEMM from codes, {took:.1f} s"}


if __name__ == "__main__":
    main()
