"""Throughput bench of the quantized-attention forward pass on one MI355X.

A step is one sage_attn_fwd call (K mean, quantization of Q and K, V
quantization where the mode has it, fused attention kernel; in the per-block
INT8 modes from 65536 token rows on the kernel quantizes Q in its prologue) over
one synthetic workload whose inputs are already resident in HBM. `value` is attention TOPS: 4*B*H*N^2*d
per step (halved when causal) divided by the step time.

Default workload: n16k, B=1, H=32, N=16384, d=128, non-causal, INT8 Q/K
with Q scale blocks of 128 tokens and K blocks of 64, FP16 P.V (the shape the
kernel throughput target is set at). --workload picks another: prefill
(B=4, H=32, N=4096, d=128, outlier K channels), long_causal, video_dit,
mxfp4, tiny.

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
                float64, as it stands) on the same workload, spread over every
                host core available to the process (one worker process per
                core, one BLAS thread each, blocks of query rows of whole
                heads as work units), for a bounded wall time; run before the
                GPU is touched. `cores` is the number of workers.
  median_ms_per_step  median of per-step times (separate pass, an event
                between steps).
  backward      (INT8 per-block modes) the 8-bit backward pass on the same
                workload: sage_attn_bwd (quantization of Q, K, V and dO, row
                terms, transposed codes, the dK/dV and dQ kernels) timed with
                HIP events, its throughput as 10*B*H*N^2*d (five products,
                halved if causal) per call, against the INT8 peak; the
                training forward (sage_attn_fwd_lse) and torch's FP16 SDPA
                backward on the same inputs for context.
  shader_clock_mhz  the shader clock measured by a probe wave (cycle counter
                against the device wall clock) on a second stream during the
                last warm-up steps, and on an idle GPU (throttling shows as
                under_load < idle). The warm-up (default 50 steps) also covers
                the clock transient that follows an idle GPU: the first ~25
                launches of the attention kernel after idling run up to 35%
                slower.
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
       python bench.py --sweep   (kernel TOPS against sequence length, one JSON line per point)
"""
import argparse
import hashlib
import json
import re
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published dense MFMA peaks (TOPS) and HBM bandwidth (GB/s)
PEAK = {"int8": 5000.0, "fp16": 2500.0, "mxfp4": 10100.0, "fp8": 5000.0}
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(name: str) -> str:
    """sha256[:16] of a kernel source's code: comments dropped and whitespace runs
    collapsed, so an edit to comments alone keeps counters taken on that code."""
    path = os.path.join(ROOT, "bit_quantized_attention_mean_amd", "csrc", name)
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    code = " ".join(text.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


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


_CPU = {}   # inputs shared with the forked oracle workers (copy-on-write)


def _cpu_unit(unit):
    """One work unit of the CPU baseline: the oracle on query rows r0:r1 of head (b, h)."""
    import oracle as O
    from synthetic import WORKLOADS

    b, h, r0, r1 = unit
    w, mode_name = WORKLOADS[_CPU["name"]], _CPU["mode"]
    q, k, v = (x[b:b + 1, h:h + 1] for x in _CPU["qkv"])
    rows = np.arange(r0, r1)
    t0 = time.perf_counter()
    if mode_name in ("mxfp4", "mxfp4_fp8pv"):
        O.mxfp4_attention(q, k, v, causal=w.causal, sm_scale=w.sm_scale, rows=rows, pv_fp8=mode_name == "mxfp4_fp8pv")
    elif mode_name == "fp16":
        O.fp16_attention(q, k, v, causal=w.causal, sm_scale=w.sm_scale, rows=rows)
    elif mode_name in ("int8_pv", "int8_pv_per_token"):
        bl = 1 if mode_name == "int8_pv_per_token" else None
        O.int8_pv_attention(q, k, v, causal=w.causal, sm_scale=w.sm_scale, blk_q=bl or 128, blk_k=bl or 64, rows=rows)
    else:
        bq, bk = {"int8_q128_k64": (128, 64), "int8_q64_k64": (64, 64), "int8_per_token": (1, 1)}[mode_name]
        O.int8_attention(q, k, v, causal=w.causal, sm_scale=w.sm_scale, blk_q=bq, blk_k=bk, rows=rows)
    # ops by the metric's convention: 4 d per visible (query, key) pair
    pairs = (np.minimum(rows + 1, w.N).sum() if w.causal else rows.size * w.N)
    return 4.0 * w.d * float(pairs), time.perf_counter() - t0


def cpu_baseline(name: str, mode_name: str, budget_s: float = 20.0):
    """The oracle on the workload, one forked worker per available host core.

    Work units are blocks of query rows of one head (rows are independent given
    the head's keys; each unit quantizes its head and runs the tiled fp64
    emulation on its rows). Units are handed out in a seeded shuffled order
    until `budget_s` of wall time has passed; the value is the metric's ops of
    the finished units over the wall time. Must run before the process touches
    the GPU (the workers are plain forks)."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits

    from synthetic import WORKLOADS, make_inputs

    w = WORKLOADS[name]
    cores = len(os.sched_getaffinity(0))
    _CPU.update(name=name, mode=mode_name, qkv=make_inputs(name))
    rb = min(w.N, 512)
    units = [(b, h, r0, min(r0 + rb, w.N)) for b in range(w.B) for h in range(w.H) for r0 in range(0, w.N, rb)]
    np.random.default_rng(0).shuffle(units)
    ops, busy, done = 0.0, 0.0, 0
    with threadpool_limits(limits=1):
        ctx = mp.get_context("fork")
        t0 = time.perf_counter()
        with ctx.Pool(cores) as pool:
            for o, t in pool.imap_unordered(_cpu_unit, units, chunksize=1):
                ops += o
                busy += t
                done += 1
                if time.perf_counter() - t0 > budget_s:
                    break
            wall = time.perf_counter() - t0
            pool.terminate()
    _CPU.clear()
    return {"value": ops / wall / 1e12, "unit": "TOPS", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cores_available": cores,
            "sample": f"{done} of {len(units)} work units (blocks of {rb} query rows of one head) of the {name} "
                      f"workload (B={w.B}, H={w.H}, N={w.N}, d={w.d}, mode {mode_name}): per-head quantization + "
                      f"tiled fp64 emulation, {wall:.1f} s wall on {cores} worker processes "
                      f"({busy:.1f} s of worker time), ops of the finished units / wall time"}


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


def backward_bench(w, mode, qd, kd, vd, args, sa, torch, sdpa=True):
    """Times the INT8 backward pass (sage_attn_bwd) on the workload's resident inputs."""
    from synthetic import make_grad
    dev = qd.device
    gd = torch.from_numpy(make_grad(w.B, w.H, w.N, w.d, seed=w.seed)).to(dev)
    wsb = sa.make_bwd_workspace(w.B, w.H, w.N, w.d, mode, dev)
    out = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    shape = (w.B, w.H, w.N, w.d)
    dq, dk, dv = (torch.empty(shape, dtype=torch.float32, device=dev) for _ in range(3))
    fwd = lambda: sa.sage_attn_fwd_lse(qd, kd, vd, out, lse, causal=w.causal, sm_scale=w.sm_scale, mode=mode,
                                       workspace=wsb)
    ms_fwd, _ = timed(fwd, args.steps, args.warmup, torch)
    bwd = lambda: sa.sage_attn_bwd(qd, kd, vd, out, gd, lse, dq, dk, dv, causal=w.causal, sm_scale=w.sm_scale,
                                   mode=mode, workspace=wsb)
    ms_bwd, _ = timed(bwd, args.steps, args.warmup, torch)
    ops = 2.5 * w.attention_ops()    # five products of 2 N^2 d each against the forward's two
    tops = ops / (ms_bwd * 1e-3) / 1e12
    log(f"[bench] {w.name}: INT8 backward {ms_bwd:.4f} ms ({tops:.1f} TOPS), training forward {ms_fwd:.4f} ms")
    rec = {"ms": round(ms_bwd, 4), "tops": round(tops, 2), "ops_per_call": ops, "peak": PEAK["int8"],
           "frac": round(tops / PEAK["int8"], 4), "fwd_lse_ms": round(ms_fwd, 4),
           "grad_dtype": "f32", "dout": "standard normal, synthetic"}
    if sdpa:
        import torch.nn.functional as F
        qg, kg, vg = (x.detach().clone().requires_grad_(True) for x in (qd, kd, vd))
        o = F.scaled_dot_product_attention(qg, kg, vg, is_causal=w.causal, scale=w.sm_scale)
        g16 = gd
        tb = lambda: torch.autograd.grad(o, (qg, kg, vg), g16, retain_graph=True)
        ms_t, _ = timed(tb, max(5, args.steps // 5), 3, torch)
        rec["torch_sdpa_fp16_bwd_ms"] = round(ms_t, 4)
        rec["speedup_vs_torch_sdpa_bwd"] = round(ms_t / ms_bwd, 3)
        log(f"[bench] torch SDPA fp16 backward: {ms_t:.4f} ms")
        del qg, kg, vg, o
    del gd, wsb, out, lse, dq, dk, dv
    torch.cuda.empty_cache()
    return rec


def sweep(torch, sa, steps):
    """Kernel throughput against sequence length, as in the pages' speed plots: N
    from 1K to 32K tokens with B*N = 32K tokens per head slot (H = 32), d = 64 and
    128, causal or not, for the INT8 kernel (mode 0), the in-repo FP16 kernel
    (mode 4), the MXFP4 kernel (mode 2) and torch's FP16 SDPA on the same inputs.
    Inputs are the prefill recipe without outlier channels (N(0, 1), K offset
    N(0, 3^2)). One JSON line per point, the attention kernel alone (HIP events
    on its stream, after a warm-up), its TOPS against the INT8 peak. The INT8
    kernel runs as sage_attn_fwd runs it: every point has B*H*N >= 65536 token
    rows, so it quantizes Q in its prologue (SAGE_FLAG_FUSED_Q)."""
    import torch.nn.functional as F
    from synthetic import make_custom
    rows = []
    for d in (128, 64):
        for causal in (False, True):
            for N in (1024, 2048, 4096, 8192, 16384, 32768):
                B, H = max(1, 32768 // N), 32
                q, k, v = make_custom(B, H, N, d, seed=7 + N + d)
                qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
                del q, k, v
                sm = 1.0 / np.sqrt(d)
                ops = 4.0 * B * H * N * N * d / (2.0 if causal else 1.0)
                rec = {"sweep": "attention kernel TOPS", "B": B, "H": H, "N": N, "d": d, "causal": causal}
                out = torch.empty_like(qd)
                fq = sa.SAGE_FLAG_FUSED_Q if B * H * N >= 65536 else 0
                for name, mode in (("int8", 0 | fq), ("fp16", 4), ("mxfp4", 2)):
                    ws = sa.make_workspace(B, H, N, d, mode & 0xff, qd.device)
                    sa.sage_attn_prepare(qd, kd, vd, ws, mode=mode)
                    comp = lambda: sa.sage_attn_compute(out, ws, causal=causal, sm_scale=sm, mode=mode, q=qd, k=kd, v=vd)
                    ms, _ = timed(comp, steps, steps, torch)
                    rec[f"{name}_ms"] = round(ms, 4)
                    rec[f"{name}_tops"] = round(ops / (ms * 1e-3) / 1e12, 1)
                    del ws
                sdpa = lambda: F.scaled_dot_product_attention(qd, kd, vd, is_causal=causal, scale=sm)
                ms, _ = timed(sdpa, steps, steps, torch)
                rec["torch_sdpa_fp16_ms"] = round(ms, 4)
                rec["torch_sdpa_fp16_tops"] = round(ops / (ms * 1e-3) / 1e12, 1)
                rec["int8_frac_of_int8_peak"] = round(rec["int8_tops"] / PEAK["int8"], 4)
                print(json.dumps(rec), flush=True)
                rows.append(rec)
                del qd, kd, vd, out
                torch.cuda.empty_cache()
    log("| d | causal | N | B | INT8 TOPS | % INT8 peak | FP16 kernel TOPS | MXFP4 TOPS | torch SDPA TOPS | INT8 / SDPA |")
    log("|---:|---|---:|---:|---:|---:|---:|---:|---:|---:|")
    for r in rows:
        log(f"| {r['d']} | {r['causal']} | {r['N']} | {r['B']} | {r['int8_tops']} | {100 * r['int8_frac_of_int8_peak']:.1f}% | "
            f"{r['fp16_tops']} | {r['mxfp4_tops']} | {r['torch_sdpa_fp16_tops']} | "
            f"{r['int8_tops'] / r['torch_sdpa_fp16_tops']:.2f}x |")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="n16k")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-sdpa", action="store_true", help="skip timing torch's FP16 SDPA for context")
    ap.add_argument("--mode", default=None,
                    choices=["int8_q128_k64", "int8_q64_k64", "int8_per_token", "mxfp4", "fp16", "mxfp4_fp8pv",
                             "int8_pv", "int8_pv_per_token"],
                    help="override the workload's quantization mode (ablations; fp16 = unquantized baseline; "
                         "int8_pv* = P and V in INT8 as well)")
    ap.add_argument("--no-smooth", action="store_true", help="skip the K mean subtraction (ablation)")
    ap.add_argument("--no-bwd", action="store_true", help="skip timing the INT8 backward pass")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (HBM counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="only time the attention kernels against sequence length (d 64 and 128, causal or "
                         "not; INT8, FP16, MXFP4 and torch SDPA), one JSON line per point")
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

    if args.sweep:
        import bit_quantized_attention_mean_amd as sa
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        sweep(torch, sa, max(5, min(args.steps, 20)))
        return

    from synthetic import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    mode_name = args.mode or w.mode
    # the CPU oracle baseline first: its workers are forks of this process, which
    # has neither touched the GPU nor loaded the HIP library yet
    cpu = None
    if not args.no_cpu and args.select is None:
        log(f"[bench] timing the CPU oracle on {len(os.sched_getaffinity(0))} host cores ...")
        cpu = cpu_baseline(w.name, mode_name)
        log(f"[bench] cpu oracle: {cpu['value']:.3e} TOPS ({cpu['sample']})")

    import bit_quantized_attention_mean_amd as sa

    if args.select is not None:
        select_layers(args.select or ["tiny", "prefill", "long_causal", "video_dit", "n16k"], torch, sa)
        return

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
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
    # the two phases separately, as sage_attn_fwd runs them: in the per-block
    # INT8 modes from 65536 token rows on, Q is quantized inside the attention
    # kernel (SAGE_FLAG_FUSED_Q) and the prepare phase covers K only
    fused_q = mode in (0, 1) and w.B * w.H * w.N >= 65536
    pflags = flags | (sa.SAGE_FLAG_FUSED_Q if fused_q else 0)
    prep = lambda: sa.sage_attn_prepare(qd, kd, vd, ws, mode=mode | pflags)
    ms_prep, _ = timed(prep, args.steps, args.warmup, torch)
    comp = lambda: sa.sage_attn_compute(out, ws, causal=w.causal, sm_scale=w.sm_scale, mode=mode | pflags, q=qd, k=kd, v=vd)
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
    smooth = not args.no_smooth
    # Algorithmic bytes of the prepare phase: each tensor it quantizes is read once
    # (2 B per element) and its codes written once, plus the scales; K's second read
    # (the channel-mean pass) and V's (the INT8 V channel maxima) are not counted,
    # they are reported separately as `quant_phase_rereads_bytes`.
    n_rows = w.B * w.H * w.N
    if mode in (2, 5):
        # Q, K, V: 2 B read; E2M1 codes 0.5 B (V in mode 5: E4M3, 1 B) + one E8M0 byte per 32 elements
        quant_bytes = 3 * n_el * 2 + 2 * n_el * (0.5 + 1 / 32) + n_el * ((1.0 if mode == 5 else 0.5) + 1 / 32)
        rereads = n_el * 2 if smooth else 0
        # mode 5: half the work (Q K^T) on FP4, half (P V) on FP8
        peak = PEAK["mxfp4"] if mode == 2 else round(2 / (1 / PEAK["mxfp4"] + 1 / PEAK["fp8"]), 1)
        kernel = f"attn_mxfp4_kernel<{w.d},{str(w.causal).lower()},{str(mode == 5).lower()}>"
        src = "attn_mxfp4.hip"
    elif mode == 4:
        # unquantized baseline: nothing to prepare (the kernel reads Q, K, V as given)
        quant_bytes, rereads = 0, 0
        peak, src = PEAK["fp16"], "attn_int8.hip"
        kernel = f"attn_int8_kernel<{w.d},{str(w.causal).lower()},2,false>"
    else:
        qblk = 1 if mode in (3, 7) else (64 if mode == 1 else 128)
        kblk = 1 if mode in (3, 7) else 64
        # Q and K: 2 B read + 1 B code per element, 4 B per scale (K only when
        # the attention kernel quantizes Q itself)
        quant_bytes = (n_el * 3 + 4 * (n_rows // kblk)) if fused_q else (n_el * 6 + 4 * (n_rows // qblk + n_rows // kblk))
        rereads = n_el * 2 if smooth else 0
        if mode in (6, 7):
            # V: 2 B read + 1 B code per element, one 4 B scale per channel; the
            # channel-maxima pass reads V a second time
            quant_bytes += n_el * 3 + 4 * w.B * w.H * w.d
            rereads += n_el * 2
        peak, src = PEAK["int8"], "attn_int8.hip"
        kernel = f"attn_int8_kernel<{w.d},{str(w.causal).lower()},{1 if mode in (3, 7) else 0},{str(mode in (6, 7)).lower()}>"
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
    bwd = None
    if mode in (0, 1) and not args.no_bwd:
        bwd = backward_bench(w, mode | flags, qd, kd, vd, args, sa, torch, sdpa=not args.no_sdpa)
    del qd, kd, vd, ws, out
    torch.cuda.empty_cache()


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
        "quant_phase_bytes": int(quant_bytes),
        "quant_phase_rereads_bytes": int(rereads),
        "q_quantized_in_kernel": bool(fused_q),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "torch_sdpa_fp16": sdpa,
        "shader_clock_mhz": {"under_load": round(clk_load), "idle": round(clk_idle)},
        "backward": bwd,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
