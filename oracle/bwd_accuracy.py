"""Accuracy of the INT8 backward pass itself on the synthetic workloads (CPU oracle only).

For each workload, on two heads cut to at most 2048 tokens (the exact float64
backward holds N x N matrices), compares the gradients of the INT8 emulation
(oracle.int8_forward_for_training, then oracle.int8_attention_backward; readings
Rb1-Rb7) with the exact float64 gradients (oracle.exact_attention_backward):
cosine similarity and relative L1 of dQ, dK and dV. dO is the synthetic
standard-normal output gradient (synthetic.make_grad). Test infrastructure: the
numbers describe the method, not a kernel.
Usage: python oracle/bwd_accuracy.py [workload ...] > table.md
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from synthetic import WORKLOADS, make_grad, make_inputs  # noqa: E402

NMAX = 2048


def metrics(a, b):
    a, b = a.ravel(), b.ravel()
    return a @ b / np.linalg.norm(a) / np.linalg.norm(b), np.abs(a - b).sum() / np.abs(b).sum()


def main(names):
    print("| workload (heads cut to N tokens) | dQ cos | dK cos | dV cos | dQ rel L1 | dK rel L1 | dV rel L1 |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    for name in names:
        w = WORKLOADS[name]
        t0 = time.time()
        N = min(w.N, NMAX)
        q, k, v = make_inputs(name, N=N)
        do = make_grad(w.B, w.H, N, w.d, seed=w.seed)
        heads = [(0, 0), (w.B - 1, w.H - 1)] if w.B * w.H > 1 else [(0, 0)]
        blk_q = 64 if w.mode == "int8_q64_k64" else 128
        got = {g: [] for g in ("dq", "dk", "dv")}
        ref = {g: [] for g in ("dq", "dk", "dv")}
        for b, h in heads:
            sl = (slice(b, b + 1), slice(h, h + 1))
            fw = O.int8_forward_for_training(q[sl], k[sl], v[sl], causal=w.causal, sm_scale=w.sm_scale, blk_q=blk_q)
            r = O.int8_attention_backward(q[sl], k[sl], v[sl], do[sl], fw["o16"], fw["lse"], causal=w.causal,
                                          sm_scale=w.sm_scale, blk_q=blk_q)
            ex = O.exact_attention_backward(q[sl], k[sl], v[sl], do[sl], causal=w.causal, sm_scale=w.sm_scale)
            for g in got:
                got[g].append(r[g])
                ref[g].append(ex[g])
        m = {g: metrics(np.concatenate(got[g]), np.concatenate(ref[g])) for g in got}
        print(f"| {name} (N={N}) | {m['dq'][0]:.6f} | {m['dk'][0]:.6f} | {m['dv'][0]:.6f} | "
              f"{m['dq'][1]:.4f} | {m['dk'][1]:.4f} | {m['dv'][1]:.4f} |", flush=True)
        print(f"  ({name}: {time.time() - t0:.1f} s)", file=sys.stderr)


if __name__ == "__main__":
    main(sys.argv[1:] or ["tiny", "prefill", "long_causal", "video_dit", "n16k"])
