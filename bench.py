"""Throughput bench of the quantized-attention forward pass on one MI355X.

A step is one sage_attn_fwd call (K mean, quantization of Q and K, V layout or
V quantization, fused attention kernel) over one synthetic workload whose
inputs are already resident in HBM. `value` is attention TOPS: 4*B*H*N^2*d
per step (halved when causal) divided by the step time.

Default workload: LLM prefill, B=4, H=32, N=4096, d=128, non-causal, INT8
Q/K with Q scale blocks of 128 tokens and K blocks of 64, FP16 P.V.
--workload picks another: n16k (B=1, H=32, N=16384, d=128, the kernel
throughput target shape), long_causal, video_dit, mxfp4, tiny.

Also on the JSON line:
  roofline      the fused attention kernel alone (sage_attn_compute), timed
                with HIP events on the stream it runs on, against the dense
                MFMA peak of its input type (INT8, or MXFP4); `traffic` comes
                from committed rocprofv3 counter summaries taken on the
                current kernel source, else null.
  torch_sdpa_fp16  PyTorch's fused FP16 scaled_dot_product_attention on the
                same inputs (context for the quantized path's speedup; not
                vs_baseline).
  cpu_baseline  the CPU oracle (oracle.int8_attention / mxfp4_attention in
                float64) timed on a bounded sample of the same workload
                (whole heads) on one host thread.
  median_ms_per_step  median of per-step times (separate pass, an event
                between steps).
  shader_clock_mhz  the shader clock measured by a probe wave (cycle counter
                against the device wall clock) on a second stream during the
                last warm-up steps, and on an idle GPU (throttling shows as
                under_load < idle). The warm-up (default 50 steps) also covers
                the clock transient that follows an idle GPU: the first ~25
                launches of the attention kernel after idling run up to 35%
                slower.
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published dense MFMA peaks (TOPS) and HBM bandwidth (GB/s)
PEAK = {"int8": 5000.0, "fp16": 2500.0, "mxfp4": 10100.0, "fp8": 5000.0}
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(name: str) -> str:
    path = os.path.join(ROOT, "bit_quantized_attention_mean_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(tag: str, source: str):
    """HBM bytes per launch from profiles/<tag>_traffic.json, if taken on this kernel source."""
    path = os.path.join(PROFILES, f"{tag}_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != kernel_source_hash(source):
        return None
    return rec.get("hbm_bytes_per_launch")


def timed(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return e0.elapsed_time(e1) / steps, wall


def warmup_with_clock_probe(fn, warmup, sa, torch):
    """Runs `warmup` steps; a clock-probe wave on a second stream starts after
    3/5 of them (past the clock transient that follows an idle GPU) and spans at
    most ~60% of the rest. Returns the shader clock in MHz over that window."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fn()
    e1.record()
    torch.cuda.synchronize()
    est_ms = e0.elapsed_time(e1)
    k0 = max(1, (3 * warmup) // 5)
    rest_ms = max(1, warmup - k0) * est_ms
    cycles = int(min(12e6, max(2.4e5, rest_ms * 0.6 * 2.4e6)))
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    ev = torch.cuda.Event()
    for i in range(max(warmup, 1)):
        fn()
        if i == k0 - 1:
            ev.record()
            side.wait_event(ev)
            sa.sage_clock_probe(cycles, out, side)
    torch.cuda.synchronize()
    c, w = (int(x) for x in out.cpu())
    return c / w * sa.sage_wall_clock_khz() / 1000.0


def median_step_ms(fn, steps, torch):
    """Median of per-step durations (an event between consecutive steps; separate pass)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    d = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return d[len(d) // 2] if len(d) % 2 else 0.5 * (d[len(d) // 2 - 1] + d[len(d) // 2])


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(name: str, mode_name: str, budget_s: float = 12.0):
    """The oracle on whole heads of the workload until ~budget_s of CPU time (1 thread)."""
    from threadpoolctl import threadpool_limits

    import oracle as O
    from synthetic import WORKLOADS, make_inputs

    w = WORKLOADS[name]
    ops = 0.0
    t_total = 0.0
    heads = 0
    with threadpool_limits(limits=1):
        while t_total < budget_s and heads < w.B * w.H:
            q, k, v = make_inputs(name, B=1, H=1, seed=1000 + heads)   # one head, same recipe
            t0 = time.perf_counter()
            if mode_name in ("mxfp4", "mxfp4_fp8pv"):
                O.mxfp4_attention(q, k, v, causal=w.causal, sm_scale=w.sm_scale, pv_fp8=mode_name == "mxfp4_fp8pv")
            elif mode_name == "fp16":
                O.fp16_attention(q, k, v, causal=w.causal, sm_scale=w.sm_scale)
            elif mode_name in ("int8_pv", "int8_pv_per_token"):
                b = 1 if mode_name == "int8_pv_per_token" else None
                O.int8_pv_attention(q, k, v, causal=w.causal, sm_scale=w.sm_scale, blk_q=b or 128, blk_k=b or 64)
            else:
                bq, bk = {"int8_q128_k64": (128, 64), "int8_q64_k64": (64, 64), "int8_per_token": (1, 1)}[mode_name]
                O.int8_attention(q, k, v, causal=w.causal, sm_scale=w.sm_scale, blk_q=bq, blk_k=bk)
            t_total += time.perf_counter() - t0
            ops += 4.0 * w.N * w.N * w.d / (2 if w.causal else 1)
            heads += 1
    return {"value": ops / t_total / 1e12, "unit": "TOPS", "cores": 1, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cores_available": len(os.sched_getaffinity(0)),
            "sample": f"{heads} whole head(s) of the {name} workload (N={w.N}, d={w.d}): "
                      f"quantization + tiled fp64 emulation, {t_total:.1f} s on 1 thread"}


def select_layers(names, torch, sa):
    """Each synthetic workload stands for one attention layer: calibrate it with the
    selector and print one JSON line per layer (measured cos and time per mode)."""
    from bit_quantized_attention_mean_amd import selector as S
    from synthetic import WORKLOADS, make_inputs

    for name in names:
        w = WORKLOADS[name]
        q, k, v = make_inputs(name)
        qd, kd, vd = (torch.from_numpy(x).to("cuda:0") for x in (q, k, v))
        del q, k, v
        mode, meas = S.calibrate(qd, kd, vd, causal=w.causal, sm_scale=w.sm_scale, reps=10)
        print(json.dumps({"layer": name, "chosen_mode": mode, "threshold": S.COS_THRESHOLD,
                          "candidates": [{"mode": m.mode, "cos": round(m.cos, 6), "ms": round(m.ms, 4)}
                                         for m in meas]}), flush=True)
        del qd, kd, vd
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-sdpa", action="store_true", help="skip timing torch's FP16 SDPA for context")
    ap.add_argument("--mode", default=None,
                    choices=["int8_q128_k64", "int8_q64_k64", "int8_per_token", "mxfp4", "fp16", "mxfp4_fp8pv",
                             "int8_pv", "int8_pv_per_token"],
                    help="override the workload's quantization mode (ablations; fp16 = unquantized baseline; "
                         "int8_pv* = P and V in INT8 as well)")
    ap.add_argument("--no-smooth", action="store_true", help="skip the K mean subtraction (ablation)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (HBM counter calibration)")
    ap.add_argument("--select", nargs="*", default=None, metavar="WORKLOAD",
                    help="only run the per-layer kernel selection (cos >= 99.8%% vs the FP16 mode, fastest "
                         "wins) on the named synthetic workloads (default: all but mxfp4)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the whole hot path runs on a single MI355X "
              f"(--gpus {args.gpus} is not supported).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        # A plain copy of 1 GiB (read 1 GiB, write 1 GiB per launch): the reference
        # against which rocprofv3's FETCH_SIZE / WRITE_SIZE are scaled to bytes.
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(7)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": args.steps}), flush=True)
        return

    import bit_quantized_attention_mean_amd as sa
    from synthetic import WORKLOADS, make_inputs

    if args.select is not None:
        select_layers(args.select or ["tiny", "prefill", "long_causal", "video_dit", "n16k"], torch, sa)
        return

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    w = WORKLOADS[args.workload]
    mode_name = args.mode or w.mode
    mode = {"int8_q128_k64": 0, "int8_q64_k64": 1, "mxfp4": 2, "int8_per_token": 3, "fp16": 4,
            "mxfp4_fp8pv": 5, "int8_pv": 6, "int8_pv_per_token": 7}[mode_name]
    flags = sa.SAGE_FLAG_NO_SMOOTH if args.no_smooth else 0
    t0 = time.perf_counter()
    q, k, v = make_inputs(w.name)
    qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    del q, k, v
    ws = sa.make_workspace(w.B, w.H, w.N, w.d, mode | flags, dev)
    out = torch.empty_like(qd)
    log(f"[bench] {w.name}: inputs ready in {time.perf_counter() - t0:.1f} s")

    # whole step
    step = lambda: sa.sage_attn_fwd(qd, kd, vd, out, causal=w.causal, sm_scale=w.sm_scale, mode=mode | flags,
                                    workspace=ws)
    clk_load = warmup_with_clock_probe(step, args.warmup, sa, torch)
    ms_step, wall_step = timed(step, args.steps, 0, torch)
    # the two phases separately
    prep = lambda: sa.sage_attn_prepare(qd, kd, vd, ws, mode=mode | flags)
    ms_prep, _ = timed(prep, args.steps, args.warmup, torch)
    comp = lambda: sa.sage_attn_compute(out, ws, causal=w.causal, sm_scale=w.sm_scale, mode=mode | flags, q=qd, k=kd, v=vd)
    ms_attn, _ = timed(comp, args.steps, args.warmup, torch)
    log(f"[bench] {w.name}: step {ms_step:.4f} ms (wall {wall_step:.4f}), attention kernel {ms_attn:.4f} ms, "
        f"quantization phase {ms_prep:.4f} ms")
    med_step = median_step_ms(step, args.steps, torch)
    # shader clock of the idle GPU, for comparison with the one under load
    clk_idle = sa.measure_clock_mhz(12_000_000)
    log(f"[bench] median step {med_step:.4f} ms; shader clock {clk_load:.0f} MHz under load, {clk_idle:.0f} MHz idle")

    ops = w.attention_ops()
    tops_step = ops / (ms_step * 1e-3) / 1e12
    tops_attn = ops / (ms_attn * 1e-3) / 1e12
    n_el = w.B * w.H * w.N * w.d
    if mode in (2, 5):
        # read K (mean), Q, K, V (2 B each); write packed codes (0.5 B) + exponents (1/32 B)
        # for Q and K, and for V 0.5 B (E2M1) or 1 B (E4M3) + exponents
        quant_bytes = n_el * 8 + 2 * n_el * (0.5 + 1 / 32) + n_el * ((1.0 if mode == 5 else 0.5) + 1 / 32)
        # mode 5: half the work (Q K^T) on FP4, half (P V) on FP8
        peak = PEAK["mxfp4"] if mode == 2 else round(2 / (1 / PEAK["mxfp4"] + 1 / PEAK["fp8"]), 1)
        kernel = f"attn_mxfp4_kernel<{w.d},{str(w.causal).lower()},{str(mode == 5).lower()}>"
        src = "attn_mxfp4.hip"
    elif mode == 4:
        # unquantized baseline: nothing to prepare (the kernel reads Q, K, V as given)
        quant_bytes = 0
        peak, src = PEAK["fp16"], "attn_int8.hip"
        kernel = f"attn_int8_kernel<{w.d},{str(w.causal).lower()},2,false>"
    elif mode in (6, 7):
        # read K (mean), Q, K, V (channel maxima), V (codes) (2 B each); write Q/K/V^T codes (1 B each)
        quant_bytes = n_el * 10 + n_el * 3
        peak, src = PEAK["int8"], "attn_int8.hip"
        kernel = f"attn_int8_kernel<{w.d},{str(w.causal).lower()},{1 if mode == 7 else 0},true>"
    else:
        # read K (mean), Q, K (2 B each); write Q/K codes (1 B each); V is read as given by the kernel
        quant_bytes = n_el * 6 + n_el * 2
        peak, src = PEAK["int8"], "attn_int8.hip"
        kernel = f"attn_int8_kernel<{w.d},{str(w.causal).lower()},{1 if mode == 3 else 0},false>"
    roofline = {"bound": "mfma", "achieved": round(tops_attn, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(tops_attn / peak, 4),
                "traffic": load_traffic(f"{src[:-4]}_{w.name}", src) if (mode_name == w.mode and not flags) else None,
                "kernel": kernel, "kernel_ms": round(ms_attn, 4)}
    if mode in (0, 1, 3):
        # half the work (Q K^T) at the INT8 rate, half (P V) at the FP16 rate
        mixed = 2 / (1 / PEAK["int8"] + 1 / PEAK["fp16"])
        roofline["mixed_int8_fp16_peak"] = round(mixed, 1)
        roofline["frac_of_mixed"] = round(tops_attn / mixed, 4)
    # context: PyTorch's own fused FP16 attention (scaled_dot_product_attention,
    # the flash backend of this ROCm build) on the same resident inputs
    sdpa = None
    if not args.no_sdpa:
        import torch.nn.functional as F
        sdpa_fn = lambda: F.scaled_dot_product_attention(qd, kd, vd, is_causal=w.causal, scale=w.sm_scale)
        ms_sdpa, _ = timed(sdpa_fn, max(5, args.steps // 5), 3, torch)
        sdpa = {"ms": round(ms_sdpa, 4), "tflops": round(ops / (ms_sdpa * 1e-3) / 1e12, 2),
                "step_speedup": round(ms_sdpa / ms_step, 3), "kernel_speedup": round(ms_sdpa / ms_attn, 3)}
        log(f"[bench] torch SDPA fp16: {ms_sdpa:.4f} ms; this step is {ms_sdpa / ms_step:.2f}x faster")
    del qd, kd, vd, ws, out
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(w.name, mode_name)
        log(f"[bench] cpu oracle: {cpu['value']:.3e} TOPS")

    line = {
        "metric": "attention TOPS (4*B*H*N^2*d per step / step time, halved if causal)",
        "value": round(tops_step, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "median_ms_per_step": round(med_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {2: "mxfp4", 4: "f16", 5: "mxfp4+mxfp8", 6: "int8", 7: "int8"}.get(mode, "int8+f16"),
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "mode": mode_name, "k_smoothing": not args.no_smooth, "global_batch": w.B, "seq_len": w.N},
        "attn_kernel_ms": round(ms_attn, 4),
        "attn_kernel_tops": round(tops_attn, 2),
        "quant_phase_ms": round(ms_prep, 4),
        "quant_phase_gbs": round(quant_bytes / (ms_prep * 1e-3) / 1e9, 1) if quant_bytes else None,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "torch_sdpa_fp16": sdpa,
        "shader_clock_mhz": {"under_load": round(clk_load), "idle": round(clk_idle)},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
