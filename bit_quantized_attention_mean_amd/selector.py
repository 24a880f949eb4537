"""Per-layer kernel selection.

The SageAttention page ("Approach") picks, for every attention layer, the
fastest of its kernels whose output keeps cosine similarity above 99.8%
against full-precision attention; its "Measured effects" table reports that
choosing the INT8 P,V kernel where it is accurate enough raised throughput
(and that quantizing P and V costs accuracy).

A layer here is one attention call site with its own input statistics.
calibrate() runs each candidate mode of the library on a calibration batch of
the layer, and the unquantized FP16 mode (the same kernel with fp16 Q K^T, fp16
P and fp32 accumulation) as the full-precision reference; it times every
candidate with HIP events on the current stream. choose() keeps the fastest
candidate at or above the threshold, and the FP16 mode when none qualifies.
The cosine is taken over the whole flattened output, in float64.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

from . import (SAGE_MODE_FP16, SAGE_MODE_INT8_PER_TOKEN, SAGE_MODE_INT8_PV, SAGE_MODE_INT8_PV_PER_TOKEN,
               SAGE_MODE_INT8_Q128_K64, make_workspace, sage_attn_fwd, sage_attn_workspace_size)

COS_THRESHOLD = 0.998
# SAGEAttn-B, -vB, -T, -vT in the page's naming: per-block or per-token Q, K scales,
# with P and V in FP16 or in INT8.
DEFAULT_CANDIDATES = (SAGE_MODE_INT8_Q128_K64, SAGE_MODE_INT8_PV, SAGE_MODE_INT8_PER_TOKEN,
                      SAGE_MODE_INT8_PV_PER_TOKEN)


@dataclass(frozen=True)
class Measurement:
    mode: int
    cos: float   # cosine similarity of the output with the FP16 reference
    ms: float    # mean time of one sage_attn_fwd call


def choose(measurements, threshold: float = COS_THRESHOLD, fallback: int = SAGE_MODE_FP16) -> int:
    """The mode of the fastest measurement with cos >= threshold; `fallback` if none."""
    ok = [m for m in measurements if m.cos >= threshold]
    if not ok:
        return fallback
    return min(ok, key=lambda m: (m.ms, m.mode)).mode


def cosine(a, b) -> float:
    """Cosine similarity of two tensors over all elements, in float64."""
    x = a.reshape(-1).double()
    y = b.reshape(-1).double()
    den = math.sqrt(float((x * x).sum()) * float((y * y).sum()))
    return float((x * y).sum()) / den if den > 0 else (1.0 if float((x - y).abs().max()) == 0 else 0.0)


def _time_ms(fn, reps: int, torch) -> float:
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def calibrate(q, k, v, *, causal: bool = False, sm_scale: float | None = None,
              candidates=DEFAULT_CANDIDATES, threshold: float = COS_THRESHOLD, reps: int = 5):
    """Measures every candidate mode on (q, k, v) and returns (chosen mode, measurements).

    Candidates the library does not accept for this shape (sage_attn_workspace_size
    returns 0, e.g. the INT8 P.V modes beyond their sequence-length limit) are skipped.
    """
    import torch
    B, H, N, d = (int(x) for x in q.shape)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    ref = sage_attn_fwd(q, k, v, causal=causal, sm_scale=sm_scale, mode=SAGE_MODE_FP16)
    out = torch.empty_like(q)
    results = []
    for mode in candidates:
        if sage_attn_workspace_size(B, H, N, d, mode) == 0:
            continue
        ws = make_workspace(B, H, N, d, mode, q.device)
        run = lambda: sage_attn_fwd(q, k, v, out, causal=causal, sm_scale=sm_scale, mode=mode, workspace=ws)
        ms = _time_ms(run, reps, torch)
        results.append(Measurement(mode=mode, cos=cosine(out, ref), ms=ms))
        del ws
    return choose(results, threshold), results


class LayerSelector:
    """Keeps one chosen mode per layer name; a layer's first call calibrates it."""

    def __init__(self, candidates=DEFAULT_CANDIDATES, threshold: float = COS_THRESHOLD, reps: int = 5):
        self.candidates = tuple(candidates)
        self.threshold = threshold
        self.reps = reps
        self.modes: dict = {}
        self.measurements: dict = {}

    def __call__(self, layer, q, k, v, *, causal: bool = False, sm_scale: float | None = None, out=None):
        if layer not in self.modes:
            mode, meas = calibrate(q, k, v, causal=causal, sm_scale=sm_scale, candidates=self.candidates,
                                   threshold=self.threshold, reps=self.reps)
            self.modes[layer] = mode
            self.measurements[layer] = meas
        return sage_attn_fwd(q, k, v, out, causal=causal, sm_scale=sm_scale, mode=self.modes[layer])
