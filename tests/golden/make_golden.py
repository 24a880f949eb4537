"""Writes tests/golden/tiny_oracle.json from the CPU oracle alone.

The pages print no worked example, so this fixture is a regression guard for
the oracle itself: any later change to the oracle's arithmetic that moves these
numbers must regenerate the file and name, in its commit message, the passage
or reading that justifies the change. Inputs: the 'tiny' synthetic workload
(B=1, H=2, N=256, d=64, Q/K blocks of 64). Floats are stored as hex strings.
Run: python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from synthetic import make_inputs, WORKLOADS  # noqa: E402


def build():
    w = WORKLOADS["tiny"]
    q, k, v = make_inputs("tiny")
    qd = O.quant_qk_int8(q, k, blk_q=64, blk_k=64)
    o = O.int8_attention(q, k, v, causal=False, sm_scale=w.sm_scale, blk_q=64, blk_k=64, quant=qd)
    mx = O.quant_mxfp4(q, k, v)
    om = O.mxfp4_attention(q, k, v, causal=False, sm_scale=w.sm_scale, quant=mx)
    return {
        "source": "oracle/sage_oracle.py on synthetic workload 'tiny' (seed 0)",
        "k_mean": [float(x).hex() for x in qd["k_mean"].ravel()],
        "q_scales": [float(x).hex() for x in qd["q_scales"].ravel()],
        "k_scales": [float(x).hex() for x in qd["k_scales"].ravel()],
        "q_codes_sum": int(qd["q_codes"].astype(np.int64).sum()),
        "k_codes_abs_sum": int(np.abs(qd["k_codes"].astype(np.int64)).sum()),
        "k_codes_weighted": int((qd["k_codes"].astype(np.int64).ravel() * (np.arange(qd["k_codes"].size) % 97)).sum()),
        "o_int8_head0_rows0_3": [float(x).hex() for x in o[0, 0, :4].ravel()],
        "mx_k_e8m0_sum": int(mx["k_e8m0"].astype(np.int64).sum()),
        "mx_v_codes_weighted": int((mx["v_codes"].astype(np.int64).ravel() * (np.arange(mx["v_codes"].size) % 89)).sum()),
        "o_mxfp4_head1_rows0_3": [float(x).hex() for x in om[0, 1, :4].ravel()],
    }


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(out, "w") as f:
        json.dump(build(), f, indent=0)
    print("wrote", out)
