"""Accuracy of the method itself on the synthetic workloads (CPU oracle only).

For each workload, on sampled heads and query rows, compares the
quantization-emulating oracle with fp64 exact attention (cosine similarity,
relative L1, RMSE, max abs) for the INT8 per-block path as configured, and the
ablations the SageAttention page's "Measured effects" table reports the
direction of: K smoothing on and off at per-block, per-token (blocks of 1
token) and per-tensor granularity, and INT8 P and V (per-block and per-token
Q, K).
MXFP4 runs the microscaled-FP4 emulation (and its variant with MX-FP8 P and
V). Test infrastructure: the numbers
describe the method (what any faithful kernel computes), not a kernel.
Usage: python oracle/method_accuracy.py [workload ...] > table.md
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from synthetic import WORKLOADS, make_inputs  # noqa: E402

ROWS = 256  # sampled query rows per head


def sample_rows(N, rng):
    """First and last 64 rows (the ragged tail) plus random rows in between."""
    fixed = np.unique(np.concatenate([np.arange(min(64, N)), np.arange(max(0, N - 64), N)]))
    rest = np.setdiff1d(np.arange(N), fixed)
    extra = rng.choice(rest, size=min(len(rest), ROWS - len(fixed)), replace=False) if len(rest) else []
    return np.sort(np.concatenate([fixed, extra])).astype(np.int64)


def per_tensor(qs, ks, vs, w, rows, scales, smooth):
    """INT8 attention of one head with per-tensor Q and K scales (taken over the whole
    workload tensors): the per-block emulation with one block per head holding the
    tensor scale."""
    N = qs.shape[2]
    sq, sk = scales
    kf = O.smooth_k(ks, O.k_mean(ks)) if smooth else ks.astype(np.float32)
    quant = dict(q_codes=O.int8_quant_with_scale(qs.astype(np.float32), sq), q_scales=np.full((1, 1, 1), sq),
                 k_codes=O.int8_quant_with_scale(kf, sk), k_scales=np.full((1, 1, 1), sk), k_mean=None)
    return O.int8_attention(qs, ks, vs, causal=w.causal, sm_scale=w.sm_scale, blk_q=N, blk_k=N, rows=rows,
                            quant=quant)


def main(names):
    rng = np.random.default_rng(123)
    print("| workload | variant | cos vs fp64 | rel L1 | RMSE | max abs | sample |")
    print("|---|---|---:|---:|---:|---:|---|")
    for name in names:
        w = WORKLOADS[name]
        t0 = time.time()
        q, k, v = make_inputs(name)
        heads = [(0, 0), (w.B - 1, w.H - 1)] if w.B * w.H > 1 else [(0, 0)]
        results = {}
        if w.mode != "mxfp4":
            # per-tensor scales of the whole Q and (smoothed or raw) K tensors
            ks_full = O.smooth_k(k, O.k_mean(k))
            tensor_scales = {True: (O.int8_tensor_scale(q.astype(np.float32)), O.int8_tensor_scale(ks_full)),
                             False: (O.int8_tensor_scale(q.astype(np.float32)),
                                     O.int8_tensor_scale(k.astype(np.float32)))}
            del ks_full
        for (b, h) in heads:
            qs, ks, vs = (x[b:b + 1, h:h + 1] for x in (q, k, v))
            rows = sample_rows(w.N, rng)
            ex = O.exact_attention(qs, ks, vs, causal=w.causal, sm_scale=w.sm_scale, rows=rows)
            if w.mode == "mxfp4":
                variants = {"MXFP4 (Q, K_s, V, P)": O.mxfp4_attention(qs, ks, vs, causal=w.causal,
                                                                      sm_scale=w.sm_scale, rows=rows),
                            "MXFP4, no K smoothing": O.mxfp4_attention(qs, ks, vs, causal=w.causal,
                                                                       sm_scale=w.sm_scale, rows=rows, smooth=False),
                            "MXFP4 Q, K_s; MX-FP8 P, V": O.mxfp4_attention(qs, ks, vs, causal=w.causal,
                                                                          sm_scale=w.sm_scale, rows=rows,
                                                                          pv_fp8=True)}
            else:
                bq = 128 if w.mode == "int8_q128_k64" else 64
                variants = {
                    f"INT8 per-block Q{bq}/K64": O.int8_attention(qs, ks, vs, causal=w.causal, sm_scale=w.sm_scale,
                                                                  blk_q=bq, blk_k=64, rows=rows),
                    "INT8 per-block, no K smoothing": O.int8_attention(qs, ks, vs, causal=w.causal,
                                                                       sm_scale=w.sm_scale, blk_q=bq, blk_k=64,
                                                                       rows=rows, smooth=False),
                    "INT8 per-token": O.int8_attention(qs, ks, vs, causal=w.causal, sm_scale=w.sm_scale,
                                                       blk_q=1, blk_k=1, rows=rows),
                    "INT8 per-token, no K smoothing": O.int8_attention(qs, ks, vs, causal=w.causal,
                                                                       sm_scale=w.sm_scale, blk_q=1, blk_k=1,
                                                                       rows=rows, smooth=False),
                    "INT8 per-tensor": per_tensor(qs, ks, vs, w, rows, tensor_scales[True], True),
                    "INT8 per-tensor, no K smoothing": per_tensor(qs, ks, vs, w, rows, tensor_scales[False], False),
                    "INT8 per-block, INT8 P and V": O.int8_pv_attention(qs, ks, vs, causal=w.causal,
                                                                        sm_scale=w.sm_scale, blk_q=bq, blk_k=64,
                                                                        rows=rows),
                    "INT8 per-token, INT8 P and V": O.int8_pv_attention(qs, ks, vs, causal=w.causal,
                                                                        sm_scale=w.sm_scale, blk_q=1, blk_k=1,
                                                                        rows=rows),
                }
            for key, val in variants.items():
                results.setdefault(key, []).append((val, ex))
        for key, pairs in results.items():
            got = np.concatenate([p[0].ravel() for p in pairs])
            ref = np.concatenate([p[1].ravel() for p in pairs])
            m = O.metrics(got, ref)
            print(f"| {name} | {key} | {m['cos']:.6f} | {m['rel_l1']:.4f} | {m['rmse']:.3e} | {m['max_abs']:.3e} "
                  f"| heads {heads}, {ROWS} rows each |", flush=True)
        print(f"<!-- {name}: {time.time() - t0:.0f} s -->", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["tiny", "prefill", "long_causal", "video_dit", "mxfp4", "n16k"])
