"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

Per workload: the whole quantization (K mean, codes, scales / MX codes and
exponents) is compared with the oracle bit for bit over every element; the
attention output is compared element by element on sampled query rows of two
heads (first and last), which the oracle computes from that head alone (every
quantity is per head). Rows: the first and last 64 (the ragged tail) and random
rows in between.
"""
import numpy as np
import pytest

import oracle as O
from synthetic import WORKLOADS, make_inputs
from _parity import assert_output_parity, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MODES = {"int8_q128_k64": 0, "int8_q64_k64": 1, "mxfp4": 2}
# relative difference between the kernel's fp32 P and the oracle's exact P within
# which an MX code of P may round either way (a few ulps of the score accumulation,
# the exponent argument and exp2, with a wide margin)
FLIP_DELTA = 2.0 ** -16


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_attention_mean_amd as m
    return m


def _rows(N, rng, n=256):
    fixed = np.unique(np.concatenate([np.arange(min(64, N)), np.arange(max(0, N - 64), N)]))
    rest = np.setdiff1d(np.arange(N), fixed)
    extra = rng.choice(rest, size=min(len(rest), n - len(fixed)), replace=False)
    return np.sort(np.concatenate([fixed, extra])).astype(np.int64)


@pytest.mark.parametrize("name", ["prefill", "long_causal", "video_dit", "n16k", "mxfp4"])
def test_full_size_workload(sa, name):
    w = WORKLOADS[name]
    mode = MODES[w.mode]
    say(f"full-size {name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal} mode={w.mode}")
    q, k, v = make_inputs(name)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))

    # quantization: INT8 every element; MXFP4 every element of six sampled heads
    # (quantization is per head; the oracle's brute-force E2M1 search over all
    # 128 Mi elements per tensor would take minutes)
    if mode == 2:
        got = sa.sage_quant_mxfp4(qd, kd, vd)
        torch.cuda.synchronize()
        got = {key: val.cpu().numpy() for key, val in got.items()}
        for (b, h) in [(0, 0), (0, w.H - 1), (1, 7), (2, 16), (w.B - 1, 3), (w.B - 1, w.H - 1)]:
            sl = (slice(b, b + 1), slice(h, h + 1))
            ref = O.quant_mxfp4(q[sl], k[sl], v[sl])
            assert np.array_equal(got["q_fp4"][sl], O.pack_fp4(ref["q_codes"]))
            assert np.array_equal(got["k_fp4"][sl], O.pack_fp4(ref["k_codes"]))
            assert np.array_equal(got["q_e8m0"][sl], ref["q_e8m0"])
            assert np.array_equal(got["k_e8m0"][sl], ref["k_e8m0"])
            assert np.array_equal(got["vt_e8m0"][sl], np.swapaxes(ref["v_e8m0"], 2, 3))
            assert np.array_equal(got["vt_fp4"][sl], O.pack_fp4(np.swapaxes(ref["v_codes"], 2, 3)))
            assert np.array_equal(got["k_mean"][sl], ref["k_mean"])
        del ref
    else:
        bq = 128 if mode == 0 else 64
        got = sa.sage_quant_qk(qd, kd, blk_q=bq, blk_k=64)
        torch.cuda.synchronize()
        ref = O.quant_qk_int8(q, k, blk_q=bq, blk_k=64)
        assert np.array_equal(got["k_mean"].cpu().numpy().view(np.uint32), ref["k_mean"].view(np.uint32))
        assert np.array_equal(got["q_scales"].cpu().numpy().view(np.uint32), ref["q_scales"].view(np.uint32))
        assert np.array_equal(got["k_scales"].cpu().numpy().view(np.uint32), ref["k_scales"].view(np.uint32))
        assert np.array_equal(got["q_codes"].cpu().numpy(), ref["q_codes"])
        assert np.array_equal(got["k_codes"].cpu().numpy(), ref["k_codes"])
        del ref
    del got
    say(f"  quantization bit-exact")

    # attention, as bench.py runs it (workspace + current stream)
    ws = sa.make_workspace(w.B, w.H, w.N, w.d, mode)
    out = torch.empty_like(qd)
    sa.sage_attn_fwd(qd, kd, vd, out, causal=w.causal, sm_scale=w.sm_scale, mode=mode, workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(99)
    for (b, h) in [(0, 0), (w.B - 1, w.H - 1)]:
        rows = _rows(w.N, rng)
        qs, ks, vs = (x[b:b + 1, h:h + 1] for x in (q, k, v))
        extra = None
        if mode == 2:
            ref, extra = O.mxfp4_attention(qs, ks, vs, causal=w.causal, sm_scale=w.sm_scale, rows=rows,
                                           flip_delta=FLIP_DELTA)
            extra = extra[0, 0]
        else:
            bq = 128 if mode == 0 else 64
            ref = O.int8_attention(qs, ks, vs, causal=w.causal, sm_scale=w.sm_scale, blk_q=bq, blk_k=64, rows=rows)
        err = assert_output_parity(got[b, h, rows], ref[0, 0], what=f"{name} head ({b},{h})", extra=extra)
        say(f"  head ({b},{h}): {rows.size} rows, max |gpu - oracle| = {err:.2e}")


@pytest.mark.parametrize("name,mode", [("n16k", 6), ("prefill", 7), ("mxfp4", 5), ("video_dit", 6), ("video_dit", 7)])
def test_full_size_variant_modes(sa, name, mode):
    # The INT8 P,V modes and the MX-FP8 P,V mode at full workload sizes, as bench.py --mode
    # runs them: V codes and scales bit for bit on two heads (INT8 V), attention on sampled
    # rows of two heads against the oracle.
    w = WORKLOADS[name]
    say(f"full-size {name} in mode {mode}: B={w.B} H={w.H} N={w.N} d={w.d}")
    q, k, v = make_inputs(name)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    if mode in (6, 7):
        got = sa.sage_quant_v_int8(vd)
        torch.cuda.synchronize()
        for (b, h) in heads:
            codes, scales = O.int8_quant_v_channels(v[b:b + 1, h:h + 1])
            assert np.array_equal(got["vt_codes"][b, h, :, :w.N].cpu().numpy(), codes[0, 0].T)
            assert np.array_equal(got["v_scales"][b, h].cpu().numpy().view(np.uint32), scales[0, 0].view(np.uint32))
        del got
        say("  INT8 V bit-exact")
    ws = sa.make_workspace(w.B, w.H, w.N, w.d, mode)
    out = torch.empty_like(qd)
    sa.sage_attn_fwd(qd, kd, vd, out, causal=w.causal, sm_scale=w.sm_scale, mode=mode, workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(7)
    for (b, h) in heads:
        rows = _rows(w.N, rng, n=128)
        qs, ks, vs = (x[b:b + 1, h:h + 1] for x in (q, k, v))
        extra = None
        if mode == 5:
            ref, extra = O.mxfp4_attention(qs, ks, vs, causal=w.causal, sm_scale=w.sm_scale, rows=rows, pv_fp8=True,
                                           flip_delta=FLIP_DELTA)
            extra = extra[0, 0]
        else:
            blk = 1 if mode == 7 else None
            ref, extra = O.int8_pv_attention(qs, ks, vs, causal=w.causal, sm_scale=w.sm_scale, blk_q=blk or 128,
                                             blk_k=blk or 64, rows=rows, flip_delta=FLIP_DELTA)
            extra = extra[0, 0]
        err = assert_output_parity(got[b, h, rows], ref[0, 0], what=f"{name} mode {mode} head ({b},{h})", extra=extra)
        say(f"  head ({b},{h}): {rows.size} rows, max |gpu - oracle| = {err:.2e}")
