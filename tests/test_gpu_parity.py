"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Quantization outputs (K mean, INT8 codes and scales, MXFP4 codes and
exponents) must match bit for bit; attention outputs must be within
2e-3 + half an fp16 ulp of the quantization-emulating oracle, element by
element. Inputs are seeded synthetic tensors (synthetic.make_custom).
"""
import numpy as np
import pytest

import oracle as O
from synthetic import make_custom
from _parity import assert_output_parity, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_attention_mean_amd as m
    return m


# relative difference between the kernel's fp32 P and the oracle's exact P within
# which an MX or INT8 code of P may round either way (see oracle.mxfp4_attention
# and oracle.int8_pv_attention)
FLIP_DELTA = 2.0 ** -16


def _dev(*arrs):
    return [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrs]


QUANT_CASES = [
    # B, H, N, d, blk_q, blk_k, flags, dist
    (1, 2, 256, 64, 64, 64, 0, "normal"),
    (2, 3, 1000, 128, 128, 64, 0, "normal"),
    (1, 2, 777, 64, 128, 64, 0, "student_t"),
    (1, 1, 1, 128, 128, 64, 0, "normal"),
    (1, 2, 63, 64, 64, 64, 0, "normal"),
    (1, 2, 65, 128, 16, 32, 0, "normal"),
    (1, 2, 300, 128, 1, 1, 0, "normal"),
    (1, 2, 300, 64, 128, 64, 0x100, "normal"),
    (1, 2, 64, 128, 64, 64, 0, "normal"),
    (1, 3, 127, 64, 128, 64, 0, "student_t"),
]


@pytest.mark.parametrize("case", QUANT_CASES, ids=lambda c: "x".join(map(str, c[:4])) + f"-b{c[4]}-{c[5]}-f{c[6]}")
def test_int8_quant_bitexact(sa, case):
    B, H, N, d, bq, bk, flags, dist = case
    say("int8 quant", case)
    q, k, _ = make_custom(B, H, N, d, seed=N + d, dist=dist)
    ref = O.quant_qk_int8(q, k, blk_q=bq, blk_k=bk, smooth=not flags)
    qd, kd = _dev(q, k)
    got = sa.sage_quant_qk(qd, kd, blk_q=bq, blk_k=bk, flags=flags)
    torch.cuda.synchronize()
    assert np.array_equal(got["q_codes"].cpu().numpy(), ref["q_codes"])
    assert np.array_equal(got["k_codes"].cpu().numpy(), ref["k_codes"])
    assert np.array_equal(got["q_scales"].cpu().numpy().view(np.uint32), ref["q_scales"].view(np.uint32))
    assert np.array_equal(got["k_scales"].cpu().numpy().view(np.uint32), ref["k_scales"].view(np.uint32))
    if not flags:
        assert np.array_equal(got["k_mean"].cpu().numpy().view(np.uint32), ref["k_mean"].view(np.uint32))


@pytest.mark.parametrize("N,d", [(300000, 128), (70001, 64)])
def test_k_mean_exact_over_the_fp16_range(sa, N, d):
    """The K mean is the exact rational mean rounded once (reading R1), whatever
    the values: K is drawn uniformly over all finite fp16 bit patterns
    (subnormals up to +-65504), with enough tokens that each thread of the
    column-sum blocks adds a few hundred of them."""
    say("k mean fp16 range", (1, 2, N, d))
    rng = np.random.default_rng(N + d)
    bits = rng.integers(0, 0x7C00, size=(1, 2, N, d), dtype=np.uint16)
    bits |= rng.integers(0, 2, size=bits.shape, dtype=np.uint16) << 15
    k = bits.view(np.float16)
    want = O.k_mean(k)
    kd, = _dev(k)
    got = sa.sage_quant_qk(kd, kd, blk_q=128, blk_k=64)
    torch.cuda.synchronize()
    assert np.array_equal(got["k_mean"].cpu().numpy().view(np.uint32), want.view(np.uint32))


MX_CASES = [(1, 2, 256, 64, 0), (2, 2, 1000, 128, 0), (1, 1, 33, 128, 0), (1, 2, 96, 64, 0x100),
            (1, 2, 300, 128, 0x200), (1, 1, 33, 64, 0x300)]   # 0x200: V in MX-FP8 (E4M3)


@pytest.mark.parametrize("case", MX_CASES, ids=lambda c: "x".join(map(str, c)))
def test_mxfp4_quant_bitexact(sa, case):
    B, H, N, d, flags = case
    say("mxfp4 quant", case)
    fp8v = bool(flags & 0x200)
    q, k, v = make_custom(B, H, N, d, seed=7 * N + d)
    ref = O.quant_mxfp4(q, k, v, smooth=not (flags & 0x100), v_fp8=fp8v)
    qd, kd, vd = _dev(q, k, v)
    got = sa.sage_quant_mxfp4(qd, kd, vd, flags=flags)
    torch.cuda.synchronize()
    assert np.array_equal(got["q_fp4"].cpu().numpy(), O.pack_fp4(ref["q_codes"]))
    assert np.array_equal(got["k_fp4"].cpu().numpy(), O.pack_fp4(ref["k_codes"]))
    assert np.array_equal(got["q_e8m0"].cpu().numpy(), ref["q_e8m0"])
    assert np.array_equal(got["k_e8m0"].cpu().numpy(), ref["k_e8m0"])
    Nv = -(-N // 32) * 32
    vcodes = np.zeros((B, H, Nv, d), np.uint8)
    vcodes[:, :, :N] = ref["v_codes"]
    vt = np.swapaxes(vcodes, 2, 3)
    assert np.array_equal(got["vt_fp4"].cpu().numpy(), vt if fp8v else O.pack_fp4(vt))
    assert np.array_equal(got["vt_e8m0"].cpu().numpy(), np.swapaxes(ref["v_e8m0"], 2, 3))


ATTN_CASES = [
    # B, H, N, d, causal, mode, dist
    (1, 2, 256, 64, False, 1, "normal"),       # the tiny workload's shape
    (1, 2, 1000, 128, False, 0, "normal"),
    (1, 2, 1000, 128, True, 0, "normal"),
    (2, 2, 777, 64, False, 0, "student_t"),
    (1, 2, 777, 64, True, 1, "normal"),
    (1, 1, 1, 128, False, 0, "normal"),
    (1, 1, 1, 64, True, 0, "normal"),
    (1, 2, 300, 128, False, 3, "normal"),      # per-token scales
    (1, 2, 300, 64, True, 3, "normal"),
    # odd tile counts (11 and 13 key tiles): the period loop's single-tile tail
    (1, 2, 700, 128, False, 0, "normal"),
    (1, 2, 777, 128, True, 0, "normal"),
]


def _int8_blocks(mode):
    return {0: (128, 64), 1: (64, 64), 3: (1, 1)}[mode]


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: "x".join(map(str, c[:4])) + f"-c{int(c[4])}-m{c[5]}")
def test_int8_attention_matches_oracle(sa, case):
    B, H, N, d, causal, mode, dist = case
    say("int8 attention", case)
    q, k, v = make_custom(B, H, N, d, seed=3 * N + d + mode, dist=dist)
    sm = 1.0 / np.sqrt(d)
    bq, bk = _int8_blocks(mode)
    ref = O.int8_attention(q, k, v, causal=causal, sm_scale=sm, blk_q=bq, blk_k=bk)
    qd, kd, vd = _dev(q, k, v)
    out = sa.sage_attn_fwd(qd, kd, vd, causal=causal, sm_scale=sm, mode=mode)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    err = assert_output_parity(got, ref, what=f"int8 {case}")
    ex = O.exact_attention(q, k, v, causal=causal, sm_scale=sm)
    say(f"  max err vs oracle {err:.2e}; cos vs fp64 gpu {O.metrics(got, ex)['cos']:.6f} "
        f"oracle {O.metrics(ref, ex)['cos']:.6f}")


F16_CASES = [
    # B, H, N, d, causal, dist: the unquantized FP16 baseline of the same kernel
    (1, 2, 256, 64, False, "normal"),
    (1, 2, 1000, 128, False, "normal"),
    (1, 2, 1000, 128, True, "normal"),
    (2, 1, 777, 64, True, "student_t"),
    (1, 1, 1, 128, False, "normal"),
    (1, 1, 777, 128, True, "normal"),
]


@pytest.mark.parametrize("case", F16_CASES, ids=lambda c: "x".join(map(str, c[:4])) + f"-c{int(c[4])}")
def test_fp16_baseline_attention_matches_oracle(sa, case):
    B, H, N, d, causal, dist = case
    say("fp16 baseline attention", case)
    q, k, v = make_custom(B, H, N, d, seed=11 * N + d, dist=dist)
    sm = 1.0 / np.sqrt(d)
    ref = O.fp16_attention(q, k, v, causal=causal, sm_scale=sm)
    qd, kd, vd = _dev(q, k, v)
    out = sa.sage_attn_fwd(qd, kd, vd, causal=causal, sm_scale=sm, mode=sa.SAGE_MODE_FP16)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    err = assert_output_parity(got, ref, what=f"fp16 {case}")
    say(f"  max err vs oracle {err:.2e}")


MXATTN_CASES = [
    (1, 2, 256, 64, False),
    (1, 2, 1000, 128, False),
    (1, 2, 1000, 128, True),
    (1, 2, 333, 64, True),
    (1, 2, 700, 128, False),
]


MX8ATTN_CASES = [
    (1, 2, 256, 64, False),
    (1, 2, 1000, 128, False),
    (1, 2, 777, 128, True),
    (1, 1, 1, 128, False),
]


@pytest.mark.parametrize("case", MX8ATTN_CASES, ids=lambda c: "x".join(map(str, c[:4])) + f"-c{int(c[4])}")
def test_mxfp4_fp8pv_attention_matches_oracle(sa, case):
    B, H, N, d, causal = case
    say("mxfp4 + fp8 P,V attention", case)
    q, k, v = make_custom(B, H, N, d, seed=13 * N + d)
    sm = 1.0 / np.sqrt(d)
    ref, extra = O.mxfp4_attention(q, k, v, causal=causal, sm_scale=sm, pv_fp8=True, flip_delta=FLIP_DELTA)
    qd, kd, vd = _dev(q, k, v)
    out = sa.sage_attn_fwd(qd, kd, vd, causal=causal, sm_scale=sm, mode=sa.SAGE_MODE_MXFP4_FP8PV)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    err = assert_output_parity(got, ref, what=f"mxfp4-fp8pv {case}", extra=extra)
    ex = O.exact_attention(q, k, v, causal=causal, sm_scale=sm)
    say(f"  max err vs oracle {err:.2e}; cos vs fp64 gpu {O.metrics(got, ex)['cos']:.6f} "
        f"oracle {O.metrics(ref, ex)['cos']:.6f}")


@pytest.mark.parametrize("case", MXATTN_CASES, ids=lambda c: "x".join(map(str, c[:4])) + f"-c{int(c[4])}")
def test_mxfp4_attention_matches_oracle(sa, case):
    B, H, N, d, causal = case
    say("mxfp4 attention", case)
    q, k, v = make_custom(B, H, N, d, seed=5 * N + d)
    sm = 1.0 / np.sqrt(d)
    ref, extra = O.mxfp4_attention(q, k, v, causal=causal, sm_scale=sm, flip_delta=FLIP_DELTA)
    qd, kd, vd = _dev(q, k, v)
    out = sa.sage_attn_fwd(qd, kd, vd, causal=causal, sm_scale=sm, mode=2)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    err = assert_output_parity(got, ref, what=f"mxfp4 {case}", extra=extra)
    ex = O.exact_attention(q, k, v, causal=causal, sm_scale=sm)
    say(f"  max err vs oracle {err:.2e}; cos vs fp64 gpu {O.metrics(got, ex)['cos']:.6f} "
        f"oracle {O.metrics(ref, ex)['cos']:.6f}")


SINT_CASES = [
    # B, H, N, d, mode, [(bh, q_tile, k_tile), ...]
    (1, 2, 1000, 128, 0, [(0, 0, 0), (1, 3, 15), (1, 1, 7)]),   # q tile 3 and k tile 15 hold the ragged tail
    (2, 1, 333, 64, 1, [(1, 1, 5), (0, 0, 2)]),
    (1, 2, 300, 128, 3, [(1, 1, 4), (0, 0, 0)]),
]


@pytest.mark.parametrize("case", SINT_CASES, ids=lambda c: "x".join(map(str, c[:4])) + f"-m{c[4]}")
def test_int8_scores_are_the_exact_integer_products(sa, case):
    # The scores the kernel's INT8 matrix op produces, dumped from inside the attention
    # kernel, equal q_codes . k_codes^T computed in int64 from the oracle's codes, bit for bit.
    B, H, N, d, mode, tiles = case
    say("int8 scores", case)
    q, k, v = make_custom(B, H, N, d, seed=23 * N + d)
    bq, bk = _int8_blocks(mode)
    ref = O.quant_qk_int8(q, k, blk_q=bq, blk_k=bk)
    qd, kd, vd = _dev(q, k, v)
    ws = sa.make_workspace(B, H, N, d, mode)
    sa.sage_attn_prepare(qd, kd, vd, ws, mode=mode)
    out = torch.empty_like(qd)
    for (bh, qt, kt) in tiles:
        got = sa.sage_attn_dump_scores(out, ws, v=vd, bh=bh, q_tile=qt, k_tile=kt, mode=mode)
        torch.cuda.synchronize()
        b, h = divmod(bh, H)
        qc = np.zeros((256, d), np.int64)
        kc = np.zeros((64, d), np.int64)
        rows = np.arange(256 * qt, min(256 * qt + 256, N))
        keys = np.arange(64 * kt, min(64 * kt + 64, N))
        qc[:rows.size] = ref["q_codes"][b, h, rows]
        kc[:keys.size] = ref["k_codes"][b, h, keys]
        want = qc @ kc.T
        assert np.array_equal(got.cpu().numpy().astype(np.int64), want), (bh, qt, kt)
    # the dump instance also computes the attention itself
    ex = O.int8_attention(q, k, v, causal=False, sm_scale=1.0 / np.sqrt(d), blk_q=bq, blk_k=bk)
    assert_output_parity(out.cpu().numpy(), ex, what=f"int8 scores {case}")


VQ_CASES = [(1, 2, 256, 64, "normal"), (2, 3, 1000, 128, "normal"), (1, 2, 777, 64, "student_t"),
            (1, 1, 1, 128, "normal"), (1, 2, 70, 128, "zero_channel")]


@pytest.mark.parametrize("case", VQ_CASES, ids=lambda c: "x".join(map(str, c[:4])) + f"-{c[4]}")
def test_int8_v_quant_bitexact(sa, case):
    B, H, N, d, dist = case
    say("int8 V quant", case)
    _, _, v = make_custom(B, H, N, d, seed=17 * N + d, dist="normal" if dist == "zero_channel" else dist)
    if dist == "zero_channel":
        v[:, :, :, 5] = 0
    codes, scales = O.int8_quant_v_channels(v)
    (vd,) = _dev(v)
    got = sa.sage_quant_v_int8(vd)
    torch.cuda.synchronize()
    Nv = -(-N // 16) * 16
    want = np.zeros((B, H, Nv, d), np.int8)
    want[:, :, :N] = codes
    assert np.array_equal(got["vt_codes"].cpu().numpy(), np.swapaxes(want, 2, 3))
    assert np.array_equal(got["v_scales"].cpu().numpy().view(np.uint32), scales.view(np.uint32))


PV8_CASES = [
    # B, H, N, d, causal, mode (6: per-block Q128/K64, 7: per token), dist
    (1, 2, 256, 64, False, 6, "normal"),
    (1, 2, 1000, 128, False, 6, "normal"),
    (1, 2, 1000, 128, True, 6, "normal"),
    (2, 2, 777, 64, False, 6, "student_t"),
    (1, 2, 777, 64, True, 7, "normal"),
    (1, 2, 300, 128, False, 7, "normal"),
    (1, 1, 1, 128, False, 6, "normal"),
    (1, 1, 1, 64, True, 7, "normal"),
    (1, 2, 777, 128, True, 6, "normal"),
]


@pytest.mark.parametrize("case", PV8_CASES, ids=lambda c: "x".join(map(str, c[:4])) + f"-c{int(c[4])}-m{c[5]}")
def test_int8_pv_attention_matches_oracle(sa, case):
    B, H, N, d, causal, mode, dist = case
    say("int8 P,V attention", case)
    q, k, v = make_custom(B, H, N, d, seed=19 * N + d + mode, dist=dist)
    sm = 1.0 / np.sqrt(d)
    blk = 1 if mode == 7 else None
    ref, flips = O.int8_pv_attention(q, k, v, causal=causal, sm_scale=sm, blk_q=blk or 128, blk_k=blk or 64,
                                     flip_delta=FLIP_DELTA)
    qd, kd, vd = _dev(q, k, v)
    out = sa.sage_attn_fwd(qd, kd, vd, causal=causal, sm_scale=sm, mode=mode)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    err = assert_output_parity(got, ref, what=f"int8-pv {case}", extra=flips)
    ex = O.exact_attention(q, k, v, causal=causal, sm_scale=sm)
    say(f"  max err vs oracle {err:.2e}; cos vs fp64 gpu {O.metrics(got, ex)['cos']:.6f} "
        f"oracle {O.metrics(ref, ex)['cos']:.6f}")


def test_int8_pv_weights_stay_in_range_for_large_logits(sa):
    # Logits near 10^5 (log2 units): the rounding of the reference max could push
    # round(127 P) of a row's maximum past 127 (an int8 wrap) without the exponent cap.
    # Constant V rows per channel make every output equal to the dequantized channel value.
    say("int8 P,V large logits")
    rng = np.random.default_rng(41)
    B, H, N, d = 1, 2, 300, 64
    q = (rng.standard_normal((B, H, N, d)) * 100).astype(np.float16)
    k = (rng.standard_normal((B, H, N, d)) * 100).astype(np.float16)
    v = np.broadcast_to(rng.standard_normal((1, 1, 1, d)).astype(np.float16), (B, H, N, d)).copy()
    ref = O.int8_pv_attention(q, k, v, causal=False, sm_scale=1.0, blk_q=128, blk_k=64)
    qd, kd, vd = _dev(q, k, v)
    out = sa.sage_attn_fwd(qd, kd, vd, causal=False, sm_scale=1.0, mode=sa.SAGE_MODE_INT8_PV)
    torch.cuda.synchronize()
    assert_output_parity(out.cpu().numpy(), ref, what="int8-pv large logits")


@pytest.mark.parametrize("mode", [0, 2, 4, 5, 6, 7])
def test_prepare_compute_equals_fwd_and_is_deterministic(sa, mode):
    say("determinism mode", mode)
    q, k, v = make_custom(1, 2, 700, 128, seed=11)
    qd, kd, vd = _dev(q, k, v)
    a = sa.sage_attn_fwd(qd, kd, vd, causal=True, mode=mode)
    b = sa.sage_attn_fwd(qd, kd, vd, causal=True, mode=mode)
    ws = sa.make_workspace(1, 2, 700, 128, mode)
    c = torch.empty_like(qd)
    sa.sage_attn_prepare(qd, kd, vd, ws, mode=mode)
    sa.sage_attn_compute(c, ws, causal=True, mode=mode, q=qd, k=kd, v=vd)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)
    # another stream, and the phases launched with an unrelated call in between
    st = torch.cuda.Stream()
    other = _dev(*make_custom(1, 1, 300, 128, seed=12))
    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        ws2 = sa.make_workspace(1, 2, 700, 128, mode)
        d2 = torch.empty_like(qd)
        sa.sage_attn_prepare(qd, kd, vd, ws2, mode=mode)
        sa.sage_attn_fwd(*other, causal=False, mode=mode)
        sa.sage_attn_compute(d2, ws2, causal=True, mode=mode, q=qd, k=kd, v=vd)
    st.synchronize()
    assert torch.equal(a, d2)


def test_clock_probe_reads_a_plausible_shader_clock(sa):
    say("clock probe")
    idle = sa.measure_clock_mhz(2_400_000)
    qd, kd, vd = _dev(*make_custom(1, 32, 2048, 128, seed=5))
    out = torch.empty_like(qd)
    ws = sa.make_workspace(1, 32, 2048, 128, 0)
    run = lambda: [sa.sage_attn_fwd(qd, kd, vd, out, mode=0, workspace=ws) for _ in range(20)]
    loaded = sa.measure_clock_mhz(2_400_000, during=run)
    say(f"  shader clock idle {idle:.0f} MHz, under load {loaded:.0f} MHz, wall clock {sa.sage_wall_clock_khz()} kHz")
    assert 300 < idle < 3500 and 300 < loaded < 3500


def test_layer_selector_on_synthetic_layers(sa):
    # Two synthetic "layers": Gaussian inputs, where every INT8 variant clears 99.8%, and
    # heavy-tailed ones (Student-t, nu = 3) where per-block scales fall short. The cosine the
    # selector measures against the FP16 mode must agree with the oracle's method accuracy.
    from bit_quantized_attention_mean_amd import selector as S
    say("layer selector")
    sel = S.LayerSelector(reps=3)
    for name, dist, seed in (("gauss", "normal", 51), ("heavy", "student_t", 52)):
        q, k, v = make_custom(1, 2, 1024, 64, seed=seed, dist=dist, k_offset_std=2.0)
        qd, kd, vd = _dev(q, k, v)
        out = sel(name, qd, kd, vd)
        torch.cuda.synchronize()
        mode, meas = sel.modes[name], sel.measurements[name]
        say(f"  {name}: chose {mode}; " + ", ".join(f"m{m.mode} cos {m.cos:.6f} {m.ms:.3f} ms" for m in meas))
        assert {m.mode for m in meas} == set(S.DEFAULT_CANDIDATES)
        assert mode == S.choose(meas)
        ok = [m for m in meas if m.cos >= S.COS_THRESHOLD]
        assert (mode == sa.SAGE_MODE_FP16) == (not ok)
        if ok:
            assert all(next(m for m in meas if m.mode == mode).ms <= m.ms for m in ok)
        again = sa.sage_attn_fwd(qd, kd, vd, mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(out, again)
        ex = O.exact_attention(q, k, v, causal=False, sm_scale=1 / 8)
        em = O.int8_attention(q, k, v, causal=False, sm_scale=1 / 8, blk_q=128, blk_k=64)
        m0 = next(m for m in meas if m.mode == 0)
        assert abs(m0.cos - O.metrics(em, ex)["cos"]) < 5e-4


@pytest.mark.parametrize("mode,d", [(0, 128), (4, 128), (3, 64), (0, 64)])
def test_ragged_tail_reads_no_row_of_the_next_head(sa, mode, d):
    # fp16 V is read as given, [N, d] per head: the last key tile of head 0
    # (keys 640..703 with N = 700) must read zeros past N, not the first rows
    # of head 1. Head 1's V is all NaN here; head 0 must equal a run on head 0
    # alone, bit for bit.
    say("ragged tail head isolation", mode, d)
    q, k, v = make_custom(1, 2, 700, d, seed=37)
    vn = v.copy()
    vn[0, 1] = np.nan
    out = sa.sage_attn_fwd(*_dev(q, k, vn), mode=mode)
    alone = sa.sage_attn_fwd(*_dev(q[:, :1].copy(), k[:, :1].copy(), v[:, :1].copy()), mode=mode)
    torch.cuda.synchronize()
    assert torch.isfinite(out[:, :1]).all()
    assert torch.equal(out[:, :1], alone)


# Configurations and edge cases of the method run through sage_attn_fwd: K smoothing
# off (the pages' smoothing ablation), per-token scales at d = 64 on heavy-tailed data
# (the per-layer selector's choice there), Q blocks of 64 at d = 128, and the cases
# where a quantization block is all zeros (scale 0, codes 0: a score of exactly 0).
EDGE_CASES = [
    # name, B, H, N, d, causal, mode, dist, edit
    ("nosmooth-int8", 1, 2, 1000, 128, False, 0 | 0x100, "normal", None),
    ("nosmooth-int8-causal", 1, 2, 777, 64, True, 0 | 0x100, "normal", None),
    ("nosmooth-mxfp4", 1, 2, 1000, 128, False, 2 | 0x100, "normal", None),
    ("nosmooth-mxfp4-causal", 1, 2, 333, 64, True, 2 | 0x100, "normal", None),
    ("nosmooth-int8pv", 1, 2, 700, 128, False, 6 | 0x100, "normal", None),
    ("pertoken-d64-t", 2, 2, 777, 64, False, 3, "student_t", None),
    ("q64-d128", 1, 2, 1000, 128, False, 1, "normal", None),
    ("q64-d128-causal", 1, 2, 700, 128, True, 1, "normal", None),
    ("const-k-int8", 1, 2, 300, 64, False, 0, "normal", "const_k"),
    ("const-k-int8-causal", 1, 2, 300, 128, True, 0, "normal", "const_k"),
    ("const-k-mxfp4", 1, 2, 300, 128, False, 2, "normal", "const_k"),
    ("const-k-int8pv", 1, 2, 300, 64, False, 6, "normal", "const_k"),
    ("zero-q-int8", 1, 2, 300, 128, False, 0, "normal", "zero_q"),
    ("zero-q-mxfp4", 1, 2, 300, 64, True, 2, "normal", "zero_q"),
    ("zero-q-pertoken", 1, 2, 300, 64, False, 3, "normal", "zero_q"),
    ("zero-blocks-int8", 1, 2, 700, 128, False, 0 | 0x100, "normal", "zero_blocks"),
    ("zero-blocks-int8-causal", 1, 2, 700, 64, True, 1 | 0x100, "normal", "zero_blocks"),
    ("zero-blocks-mxfp4", 1, 2, 700, 128, False, 2 | 0x100, "normal", "zero_blocks"),
    ("zero-blocks-int8pv", 1, 2, 700, 128, True, 7 | 0x100, "normal", "zero_blocks"),
]


def _edit_inputs(q, k, v, edit):
    if edit == "const_k":        # every token's K equal: smoothing makes K_s exactly 0
        k[:] = k[:, :, :1, :]
    elif edit == "zero_q":       # every score 0: uniform attention over the visible keys
        q[:] = 0
    elif edit == "zero_blocks":  # Q rows 128..255 and K rows 64..127 all zero (no smoothing)
        q[:, :, 128:256] = 0
        k[:, :, 64:128] = 0
    return q, k, v


def _oracle_for_mode(q, k, v, *, causal, sm, mode):
    lo, smooth = mode & 0xFF, not (mode & 0x100)
    if lo in (0, 1, 3):
        bq, bk = _int8_blocks(lo)
        return O.int8_attention(q, k, v, causal=causal, sm_scale=sm, blk_q=bq, blk_k=bk, smooth=smooth), None
    if lo in (6, 7):
        b = 1 if lo == 7 else None
        return O.int8_pv_attention(q, k, v, causal=causal, sm_scale=sm, blk_q=b or 128, blk_k=b or 64,
                                   smooth=smooth, flip_delta=FLIP_DELTA)
    if lo in (2, 5):
        return O.mxfp4_attention(q, k, v, causal=causal, sm_scale=sm, smooth=smooth, pv_fp8=lo == 5,
                                 flip_delta=FLIP_DELTA)
    raise ValueError(mode)


@pytest.mark.parametrize("case", EDGE_CASES, ids=lambda c: c[0])
def test_configuration_and_zero_block_edge_cases(sa, case):
    name, B, H, N, d, causal, mode, dist, edit = case
    say("edge case", case)
    q, k, v = make_custom(B, H, N, d, seed=29 * N + d + (mode & 0xFF), dist=dist)
    q, k, v = _edit_inputs(q, k, v, edit)
    sm = 1.0 / np.sqrt(d)
    ref, extra = _oracle_for_mode(q, k, v, causal=causal, sm=sm, mode=mode)
    qd, kd, vd = _dev(q, k, v)
    out = sa.sage_attn_fwd(qd, kd, vd, causal=causal, sm_scale=sm, mode=mode)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    err = assert_output_parity(got, ref, what=name, extra=extra)
    if edit in ("const_k", "zero_q") and not causal:
        # uniform weights: every output row is the plain mean of V (up to V's own codec)
        vmean = v.astype(np.float64).mean(axis=2, keepdims=True)
        tol = 2e-3 if (mode & 0xFF) in (0, 1, 3) else 0.3 * np.abs(v).max()
        assert np.max(np.abs(got - vmean)) <= tol
    ex = O.exact_attention(q, k, v, causal=causal, sm_scale=sm)
    say(f"  max err vs oracle {err:.2e}; cos vs fp64 gpu {O.metrics(got, ex)['cos']:.6f} "
        f"oracle {O.metrics(ref, ex)['cos']:.6f}")


FUSED_CASES = [
    # B, H, N, d, causal, mode (SAGE_FLAG_FUSED_Q added)
    (1, 2, 700, 128, True, 0),
    (2, 1, 333, 64, False, 1),
    (1, 3, 256, 128, False, 0x100),
    (1, 1, 1, 64, True, 0x101),
    (1, 2, 130, 64, True, 0),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "x".join(map(str, c[:4])) + f"-c{int(c[4])}-m{c[5]:#x}")
def test_fused_q_quantization_is_bit_identical(sa, case):
    """SAGE_FLAG_FUSED_Q: the attention kernel quantizes Q in its prologue (the
    prepare phase skips Q) and must reach the very codes and scales of the
    quantization kernel, so its output equals the two-phase result with Q codes
    from the workspace bit for bit; the oracle bar holds as well."""
    B, H, N, d, causal, mode = case
    say("fused Q", case)
    q, k, v = make_custom(B, H, N, d, seed=77 + N + d, dist="student_t" if N == 333 else "normal")
    qd, kd, vd = _dev(q, k, v)
    sm = 1.0 / np.sqrt(d)
    fused = mode | sa.SAGE_FLAG_FUSED_Q
    ws_a, ws_b = sa.make_workspace(B, H, N, d, mode), sa.make_workspace(B, H, N, d, fused)
    a, b = torch.empty_like(qd), torch.empty_like(qd)
    sa.sage_attn_prepare(qd, kd, vd, ws_a, mode=mode)
    sa.sage_attn_compute(a, ws_a, causal=causal, sm_scale=sm, mode=mode, q=qd, k=kd, v=vd)
    sa.sage_attn_prepare(qd, kd, vd, ws_b, mode=fused)
    sa.sage_attn_compute(b, ws_b, causal=causal, sm_scale=sm, mode=fused, q=qd, k=kd, v=vd)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    bq, bk = _int8_blocks(mode & 0xFF)
    ref = O.int8_attention(q, k, v, causal=causal, sm_scale=sm, blk_q=bq, blk_k=bk, smooth=not (mode & 0x100))
    assert_output_parity(b.cpu().numpy(), ref, what=f"fused Q {case}")


@pytest.mark.parametrize("d,mode", [(128, 0), (64, 1)])
def test_fused_q_special_blocks(sa, d, mode):
    """The prologue quantization on the Q blocks that take its rare branches: an
    all-zero block (scale 0, codes 0), a block of fp16 subnormals only (the
    smallest scales the Markstein quotient sees), and a block mixing +-65504
    with small values; fused and two-phase results equal bit for bit, and the
    oracle bar holds."""
    B, H, N = 1, 2, 600
    blk = 128 if mode == 0 else 64
    say("fused Q special blocks", (B, H, N, d, mode))
    q, k, v = make_custom(B, H, N, d, seed=91 + d)
    rng = np.random.default_rng(92 + d)
    q[:, :, 0:blk] = 0
    sub = rng.integers(1, 1024, size=(B, H, blk, d)).astype(np.float64) * 2.0 ** -24
    q[:, :, blk:2 * blk] = (sub * rng.choice([-1.0, 1.0], size=sub.shape)).astype(np.float16)
    big = rng.standard_normal((B, H, blk, d)).astype(np.float16)
    big[..., ::7] = np.float16(65504.0) * rng.choice([-1, 1], size=big[..., ::7].shape).astype(np.float16)
    q[:, :, 2 * blk:3 * blk] = big
    qd, kd, vd = _dev(q, k, v)
    sm = 1.0 / np.sqrt(d)
    fused = mode | sa.SAGE_FLAG_FUSED_Q
    ws_a, ws_b = sa.make_workspace(B, H, N, d, mode), sa.make_workspace(B, H, N, d, fused)
    a, b = torch.empty_like(qd), torch.empty_like(qd)
    sa.sage_attn_prepare(qd, kd, vd, ws_a, mode=mode)
    sa.sage_attn_compute(a, ws_a, causal=False, sm_scale=sm, mode=mode, q=qd, k=kd, v=vd)
    sa.sage_attn_prepare(qd, kd, vd, ws_b, mode=fused)
    sa.sage_attn_compute(b, ws_b, causal=False, sm_scale=sm, mode=fused, q=qd, k=kd, v=vd)
    torch.cuda.synchronize()
    assert torch.isfinite(b).all()
    assert torch.equal(a, b)
    bq, bk = _int8_blocks(mode)
    ref = O.int8_attention(q, k, v, causal=False, sm_scale=sm, blk_q=bq, blk_k=bk)
    assert_output_parity(b.cpu().numpy(), ref, what=f"fused Q special blocks d={d} mode={mode}")


def test_fwd_fuses_q_on_large_problems(sa):
    """sage_attn_fwd takes the fused pass from 65536 token rows on: its output
    equals the two-phase result with workspace Q codes bit for bit."""
    B, H, N, d = 1, 16, 4096, 64
    q, k, v = make_custom(B, H, N, d, seed=78)
    qd, kd, vd = _dev(q, k, v)
    out = sa.sage_attn_fwd(qd, kd, vd, causal=True)
    ws = sa.make_workspace(B, H, N, d, 0)
    c = torch.empty_like(qd)
    sa.sage_attn_prepare(qd, kd, vd, ws, mode=0)
    sa.sage_attn_compute(c, ws, causal=True, mode=0, q=qd, k=kd, v=vd)
    torch.cuda.synchronize()
    assert torch.equal(out, c)
