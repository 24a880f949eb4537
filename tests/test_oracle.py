"""Pins for the CPU oracle: each test checks it against something other than itself.

Sources of truth used here: a library routine (torch's scaled_dot_product_attention
on CPU in float64), brute-force pure-Python loops, exact rational arithmetic
(fractions.Fraction), closed forms (O = V for one key, mean(V) for flat scores),
and the invariance the SageAttention page states in "Approach" (subtracting
the mean of K across tokens leaves softmax attention unchanged).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from synthetic import make_custom

RNG = np.random.default_rng(1234)


def _rand16(*shape, scale=1.0, rng=RNG):
    return (rng.standard_normal(shape) * scale).astype(np.float16)


# ---------------------------------------------------------------------------
# exact attention (c1)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_exact_matches_torch_sdpa_f64(causal):
    q, k, v = _rand16(2, 3, 37, 16), _rand16(2, 3, 37, 16, scale=2.0), _rand16(2, 3, 37, 16)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64)), torch.from_numpy(k.astype(np.float64)),
        torch.from_numpy(v.astype(np.float64)), is_causal=causal, scale=0.3).numpy()
    got = O.exact_attention(q, k, v, causal=causal, sm_scale=0.3)
    assert np.max(np.abs(got - ref)) < 1e-13


def _brute_attention(q, k, v, causal, scale):
    N, d = len(q), len(q[0])
    out = []
    for i in range(N):
        s = [scale * sum(q[i][c] * k[j][c] for c in range(d)) if (not causal or j <= i) else None
             for j in range(N)]
        mx = max(x for x in s if x is not None)
        w = [math.exp(x - mx) if x is not None else 0.0 for x in s]
        tot = sum(w)
        out.append([sum(w[j] * v[j][c] for j in range(N)) / tot for c in range(d)])
    return np.array(out)


@pytest.mark.parametrize("causal", [False, True])
def test_exact_matches_bruteforce_loops(causal):
    q, k, v = _rand16(1, 1, 6, 3), _rand16(1, 1, 6, 3), _rand16(1, 1, 6, 3)
    ref = _brute_attention(q[0, 0].astype(float).tolist(), k[0, 0].astype(float).tolist(),
                           v[0, 0].astype(float).tolist(), causal, 0.7)
    got = O.exact_attention(q, k, v, causal=causal, sm_scale=0.7)[0, 0]
    assert np.max(np.abs(got - ref)) < 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_exact_rows_are_probability_distributions(causal):
    N = 24
    q, k = _rand16(1, 1, N, N, scale=2.0), _rand16(1, 1, N, N, scale=2.0)
    eye = np.eye(N)[None, None]                       # V = I makes O equal to P
    P = O.exact_attention(q, k, eye, causal=causal, sm_scale=0.5)[0, 0]
    assert np.all(P >= 0)
    assert np.max(np.abs(P.sum(axis=1) - 1.0)) < 1e-13
    if causal:
        assert np.all(P[np.triu_indices(N, 1)] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_mean_smoothing_leaves_exact_attention_unchanged(causal):
    # "Approach": subtracting the mean of K across tokens leaves softmax attention unchanged.
    # Any per-channel shift shared by all tokens adds q.mu to a whole score row.
    q, k, v = _rand16(1, 2, 40, 32), _rand16(1, 2, 40, 32), _rand16(1, 2, 40, 32)
    mu = RNG.standard_normal((1, 2, 1, 32)) * 3.0
    a = O.exact_attention(q, k.astype(np.float64), v, causal=causal, sm_scale=0.2)
    b = O.exact_attention(q, k.astype(np.float64) - mu, v, causal=causal, sm_scale=0.2)
    assert np.max(np.abs(a - b)) < 1e-12


def test_exact_special_cases():
    v = _rand16(1, 1, 9, 4)
    # one key: O = V
    one = O.exact_attention(_rand16(1, 1, 1, 4), _rand16(1, 1, 1, 4), v[:, :, :1], causal=False, sm_scale=1.0)
    assert np.array_equal(one, v[:, :, :1].astype(np.float64))
    # Q = 0: flat scores, O = mean(V); causal: prefix means
    z = np.zeros((1, 1, 9, 4), np.float16)
    k = _rand16(1, 1, 9, 4)
    flat = O.exact_attention(z, k, v, causal=False, sm_scale=1.0)[0, 0]
    assert np.max(np.abs(flat - v[0, 0].astype(float).mean(axis=0))) < 1e-15
    pref = O.exact_attention(z, k, v, causal=True, sm_scale=1.0)[0, 0]
    cm = np.cumsum(v[0, 0].astype(float), axis=0) / np.arange(1, 10)[:, None]
    assert np.max(np.abs(pref - cm)) < 1e-15
    # causal row 0 sees only key 0
    c = O.exact_attention(_rand16(1, 1, 9, 4), k, v, causal=True, sm_scale=1.0)
    assert np.array_equal(c[0, 0, 0], v[0, 0, 0].astype(np.float64))
    # one dominant score: O ~= V_j
    q1 = np.zeros((1, 1, 1, 4), np.float16); q1[..., 0] = 100
    k1 = np.zeros((1, 1, 9, 4), np.float16); k1[0, 0, 5, 0] = 100
    dom = O.exact_attention(q1, k1, v, causal=False, sm_scale=1.0)[0, 0, 0]
    assert np.max(np.abs(dom - v[0, 0, 5].astype(float))) < 1e-12


# ---------------------------------------------------------------------------
# K mean (reading R1) against exact rational arithmetic
# ---------------------------------------------------------------------------

def test_k_mean_matches_exact_rational_mean():
    k = _rand16(2, 2, 77, 8, scale=3.0)
    k[0, 0, :5, 0] = np.float16(6.0e-8)        # fp16 subnormals take part too
    k[1, 1, :, 3] = np.float16(-65504.0)       # largest magnitude
    mu = O.k_mean(k)
    for b in range(2):
        for h in range(2):
            for c in range(8):
                s = sum(Fraction(float(x)) for x in k[b, h, :, c])
                want = np.float32(float(s / 77))   # Fraction -> float is correctly rounded
                assert mu[b, h, c] == want


def test_k_channel_sum_is_integer_exact():
    k = _rand16(1, 1, 300, 4, scale=100.0)
    tot = O.k_channel_sum(k)
    for c in range(4):
        exact = sum(Fraction(float(x)) for x in k[0, 0, :, c]) * 2 ** 24
        assert exact.denominator == 1 and tot[0, 0, c] == exact.numerator


# ---------------------------------------------------------------------------
# INT8 quantization (readings R3, R4) against exact rationals and brute force
# ---------------------------------------------------------------------------

def _f32_round(fr: Fraction) -> Fraction:
    """Round a rational to the nearest float32 (ties to even), normal range only."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    scaled = a / Fraction(2) ** (e - 23)               # in [2^23, 2^24)
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return sign * Fraction(m) * Fraction(2) ** (e - 23)


def _round_half_even(fr: Fraction) -> int:
    f = math.floor(fr)
    rem = fr - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        return f + 1
    return f


@pytest.mark.parametrize("blk,N", [(64, 64), (64, 70), (1, 5), (128, 200)])
def test_int8_codes_and_scales_exact(blk, N):
    x = (RNG.standard_normal((1, 2, N, 8)) * 2.5).astype(np.float32)
    codes, scales = O.int8_quant_blocks(x, blk)
    assert scales.shape == (1, 2, -(-N // blk))
    for h in range(2):
        for bi in range(scales.shape[2]):
            blkx = x[0, h, bi * blk:(bi + 1) * blk]
            a = Fraction(float(np.abs(blkx).max()))
            s = _f32_round(a / 127)
            assert Fraction(float(scales[0, h, bi])) == s
            for (r, c), xv in np.ndenumerate(blkx):
                want = _round_half_even(_f32_round(Fraction(float(xv)) / s))
                got = int(codes[0, h, bi * blk + r, c])
                assert got == want
                # near-optimal among all 255 codes: within half a step (+ one fp32 rounding)
                assert abs(Fraction(got) - Fraction(float(xv)) / s) <= Fraction(1, 2) + Fraction(1, 2 ** 16)
            # the block maximum lands on +-127
            i = np.unravel_index(np.argmax(np.abs(blkx)), blkx.shape)
            assert abs(int(codes[0, h, bi * blk + i[0], i[1]])) == 127
    assert codes.min() >= -127


def test_int8_exact_ties_round_to_even():
    # block max 127 gives scale exactly 1, so x / s lands exactly on half-integers
    x = np.zeros((1, 1, 1, 8), np.float32)
    x[0, 0, 0] = [127.0, 0.5, 1.5, 2.5, -2.5, 126.5, -0.5, 3.5]
    codes, scales = O.int8_quant_blocks(x, 1)
    assert scales[0, 0, 0] == 1.0
    assert codes[0, 0, 0].tolist() == [127, 0, 2, 2, -2, 126, 0, 4]


def test_int8_zero_block():
    x = np.zeros((1, 1, 64, 8), np.float32)
    x[0, 0, 40:] = 1.0
    codes, scales = O.int8_quant_blocks(x, 32)
    assert scales[0, 0, 0] == 0 and np.all(codes[0, 0, :32] == 0)
    assert np.all(codes[0, 0, 40:] == 127)


def test_dequantized_scores_within_quantization_bound():
    # Catches transposed operands and wrong scale indexing: |S_deq - S_exact| is bounded by
    # the per-element code errors (|x - c*s| <= s/2 up to one fp32 rounding).
    q, k, _ = make_custom(1, 1, 150, 32, seed=7)
    d = O.quant_qk_int8(q, k, blk_q=64, blk_k=32)
    ks = O.smooth_k(k, d["k_mean"]).astype(np.float64)[0, 0]
    qf = q.astype(np.float64)[0, 0]
    sq = d["q_scales"][0, 0][np.arange(150) // 64].astype(np.float64)
    sk = d["k_scales"][0, 0][np.arange(150) // 32].astype(np.float64)
    S_deq = (d["q_codes"][0, 0].astype(np.float64) @ d["k_codes"][0, 0].astype(np.float64).T) * sq[:, None] * sk[None, :]
    S_ex = qf @ ks.T
    bound = (np.abs(qf) @ np.ones((32, 150))) * sk[None, :] / 2 + (np.ones((150, 32)) @ np.abs(ks).T) * sq[:, None] / 2 \
        + 32 * sq[:, None] * sk[None, :] / 4
    assert np.all(np.abs(S_deq - S_ex) <= bound * (1 + 1e-5))


# ---------------------------------------------------------------------------
# INT8 attention emulation (c2)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_int8_emulation_without_quantization_is_exact_attention(causal):
    q, k, v = make_custom(1, 2, 150, 32, seed=3)
    ex = O.exact_attention(q, k, v, causal=causal, sm_scale=0.25)
    got = O.int8_attention(q, k, v, causal=causal, sm_scale=0.25, blk_q=64, blk_k=64,
                           quantize=False, smooth=False)
    assert np.max(np.abs(got - ex)) < 1e-12
    # with smoothing on and no quantization: exact attention on the fp32 smoothed K
    ks = O.smooth_k(k, O.k_mean(k)).astype(np.float64)
    ex_s = O.exact_attention(q, ks, v, causal=causal, sm_scale=0.25)
    got_s = O.int8_attention(q, k, v, causal=causal, sm_scale=0.25, blk_q=64, blk_k=64, quantize=False)
    assert np.max(np.abs(got_s - ex_s)) < 1e-12


def test_int8_emulation_tiling_changes_only_fp16_rounding():
    q, k, v = make_custom(1, 1, 256, 64, seed=4)
    a = O.int8_attention(q, k, v, causal=False, sm_scale=0.125, blk_q=64, blk_k=64, kv_tile=64)
    b = O.int8_attention(q, k, v, causal=False, sm_scale=0.125, blk_q=64, blk_k=64, kv_tile=256)
    assert np.max(np.abs(a - b)) < 2 ** -10 * np.abs(v.astype(float)).max()


def test_int8_emulation_constant_v():
    # l sums the same fp16 P that weights V, so a constant V comes back exactly
    q, k, _ = make_custom(1, 1, 200, 32, seed=5)
    v = np.full((1, 1, 200, 32), 1.5, np.float16)
    o = O.int8_attention(q, k, v, causal=True, sm_scale=0.2, blk_q=64, blk_k=64)
    assert np.max(np.abs(o - 1.5)) <= 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_fp16_baseline_is_exact_attention_up_to_p16_rounding(causal):
    # unquantized baseline: the only rounding on the way is P -> fp16
    # (relative error <= 2^-11 per weight), so O moves by at most ~2^-10 max|V|
    q, k, v = make_custom(1, 2, 300, 32, seed=12, k_offset_std=2.0)
    ex = O.exact_attention(q, k, v, causal=causal, sm_scale=0.3)
    got = O.fp16_attention(q, k, v, causal=causal, sm_scale=0.3)
    err = np.max(np.abs(got - ex))
    assert err <= 2 ** -10 * np.abs(v.astype(float)).max()
    assert err > 0  # P really is rounded


def test_fp16_baseline_constant_v_and_row_subsets():
    q, k, _ = make_custom(1, 1, 200, 32, seed=13)
    v = np.full((1, 1, 200, 32), -2.25, np.float16)
    o = O.fp16_attention(q, k, v, causal=True, sm_scale=0.2)
    assert np.max(np.abs(o + 2.25)) <= 1e-14
    q, k, v = make_custom(1, 2, 190, 32, seed=14)
    full = O.fp16_attention(q, k, v, causal=True, sm_scale=0.2)
    rows = np.array([0, 63, 64, 189])
    assert np.array_equal(O.fp16_attention(q, k, v, causal=True, sm_scale=0.2, rows=rows), full[:, :, rows])


def test_int8_rows_subset_matches_full():
    q, k, v = make_custom(1, 2, 300, 32, seed=6)
    full = O.int8_attention(q, k, v, causal=True, sm_scale=0.2, blk_q=128, blk_k=64)
    rows = np.array([0, 5, 127, 128, 299])
    sub = O.int8_attention(q, k, v, causal=True, sm_scale=0.2, blk_q=128, blk_k=64, rows=rows)
    assert np.array_equal(sub, full[:, :, rows])


def test_int8_method_accuracy_tiny_workload():
    # "Approach": the method's bar is cosine similarity above 99.8% against full precision.
    q, k, v = make_custom(1, 2, 256, 64, seed=0)
    ex = O.exact_attention(q, k, v, causal=False, sm_scale=0.125)
    em = O.int8_attention(q, k, v, causal=False, sm_scale=0.125, blk_q=64, blk_k=64)
    assert O.metrics(em, ex)["cos"] > 0.998


def test_smoothing_helps_with_large_k_offsets():
    # "Measured effects": smoothing K raises accuracy under INT8 quantization.
    q, k, v = make_custom(1, 2, 512, 64, seed=8, k_offset_std=20.0)
    ex = O.exact_attention(q, k, v, causal=False, sm_scale=0.125)
    on = O.metrics(O.int8_attention(q, k, v, causal=False, sm_scale=0.125, blk_q=64, blk_k=64), ex)["cos"]
    off = O.metrics(O.int8_attention(q, k, v, causal=False, sm_scale=0.125, blk_q=64, blk_k=64, smooth=False), ex)["cos"]
    assert on > off


# ---------------------------------------------------------------------------
# MX codecs (reading R8)
# ---------------------------------------------------------------------------

def _e2m1_from_bits(code: int) -> float:
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = (m / 2.0) if e == 0 else 2.0 ** (e - 1) * (1 + m / 2.0)
    return -mag if s else mag


def test_e2m1_table_matches_bit_field_definition():
    for code in range(8):
        assert O.E2M1_MAGNITUDES[code] == _e2m1_from_bits(code)
        assert -O.E2M1_MAGNITUDES[code] == _e2m1_from_bits(code | 8)


def test_e2m1_nearest_is_nearest_with_even_ties():
    ys = np.concatenate([np.arange(0, 8.5, 1 / 64), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 100.0]])
    idx = O.e2m1_nearest(ys)
    grid = [abs(_e2m1_from_bits(c)) for c in range(8)]
    for y, i in zip(ys.tolist(), idx.tolist()):
        dists = [abs(y - g) for g in grid]
        best = min(dists)
        assert dists[i] == best
        ties = [c for c in range(8) if dists[c] == best]
        if len(ties) > 1:
            assert i % 2 == 0 and i in ties


def _floor_log2(x: float) -> int:
    n, d = Fraction(x).as_integer_ratio()
    e = n.bit_length() - d.bit_length()
    return e if Fraction(2) ** e <= Fraction(n, d) else e - 1


def test_e8m0_exponent_rule():
    vals = [1.0, 2.0, 3.99, 4.0, 6.0, 7.9, 0.3, 1e-3, 1e-40, 2.0 ** -126, 3.0e38, 65504.0, 5.9e-8]
    e = O.e8m0_exponent(np.array(vals))
    for x, ei in zip(vals, e.tolist()):
        assert ei == max(-127, min(127, _floor_log2(x) - 2))
    assert O.e8m0_exponent(np.array([0.0]))[0] == 0


def test_mx_roundtrip_of_representable_blocks_and_error_bound():
    rng = np.random.default_rng(11)
    mags = rng.integers(0, 8, size=(4, 64))
    sign = rng.integers(0, 2, size=(4, 64))
    mags[:, 0] = 7; mags[:, 32] = 6                # block maxima 6 and 4 set the exponent
    exps = np.array([0, -3, 5, -10])
    x = (np.where(sign, -1, 1) * O.E2M1_MAGNITUDES[mags] * np.exp2(exps)[:, None]).astype(np.float32)
    codes, e8, vals = O.mx_quantize(x, axis=1)
    assert np.array_equal(vals, x.astype(np.float64))
    assert np.array_equal(e8[:, 0], (exps + 127).astype(np.uint8))
    # random data: error at most half a grid step, or the saturation gap above 6 * 2^e
    y = rng.standard_normal((8, 96)).astype(np.float32) * 3
    codes, e8, vals = O.mx_quantize(y, axis=1)
    e = e8.astype(np.int64) - 127
    step = np.repeat(np.exp2(e), 32, axis=1)
    err = np.abs(vals - y)
    assert np.all(err <= np.maximum(np.where(np.abs(y) < 2 * step, 0.25, np.where(np.abs(y) < 4 * step, 0.5, 1.0)) * step,
                                    (np.abs(y) - 6 * step)))


def test_mx_sign_bit_follows_the_sign_of_x():
    x = np.array([[4.0, -0.0, -1e-3, 1e-3] + [0.0] * 28], np.float32)
    codes, _, _ = O.mx_quantize(x, axis=1)
    assert codes[0, :4].tolist() == [6, 8, 8, 0]


def test_mx_v_blocks_run_along_tokens():
    v = np.ones((1, 1, 64, 64), np.float16)
    v[0, 0, 3, 5] = 64.0
    d = O.quant_mxfp4(v, v, v)
    vv = d["v_vals"][0, 0]
    assert vv[0, 5] == 0.0 and vv[40, 5] == 1.0      # same channel: shares the big value's exponent below token 32
    assert vv[3, 6] == 1.0 and vv[3, 5] == 64.0      # other channels of that token are untouched
    assert d["v_e8m0"].shape == (1, 1, 2, 64)


# --- MX-FP8 variant for P and V (reading R13): pinned to torch's float8_e4m3fn ---

def test_e4m3_decode_matches_torch_float8():
    codes = np.arange(256)
    ours = O.e4m3_value(codes)
    ref = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[~np.isnan(ours)], ref[~np.isnan(ref)])
    assert np.nanmax(ours) == 448.0 and ours[1] == 2.0 ** -9


def test_e4m3_nearest_matches_torch_cast_including_ties():
    rng = np.random.default_rng(21)
    y = np.abs(rng.standard_normal(50000)) * np.exp2(rng.integers(-12, 9, 50000))
    # exact midpoints between neighbouring magnitudes: ties go to the even code
    mags = O.e4m3_value(np.arange(0x7F))
    mids = (mags[:-1] + mags[1:]) / 2
    y = np.concatenate([np.minimum(y, 448.0), mids, mags]).astype(np.float32).astype(np.float64)
    ours = O.e4m3_nearest(y)
    ref = torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    assert np.array_equal(ours, ref)
    assert np.all(ours[len(y) - 2 * 0x7F + 1:len(y) - 0x7F] % 2 == 0)   # every midpoint lands on an even code


def test_e4m3_saturates_at_448():
    assert O.e4m3_nearest(np.array([448.0, 460.0, 1e6])).tolist() == [0x7E] * 3


def test_mx_fp8_block_rule_and_roundtrip():
    rng = np.random.default_rng(22)
    codes = rng.integers(0, 0x7F, size=(3, 64))
    codes[:, 0] = 0x7E; codes[:, 32] = 0x70          # block maxima 448 = 1.75 * 2^8 and 256 = 2^8
    exps = np.array([0, -7, 4])
    x = (O.e4m3_value(codes) * np.where(rng.integers(0, 2, (3, 64)), -1, 1) * np.exp2(exps)[:, None]).astype(np.float32)
    c, e8, vals = O.mx_quantize_fp8(x, axis=1)
    assert np.array_equal(vals, x.astype(np.float64))          # representable blocks come back exactly
    assert np.array_equal(e8[:, 0], (exps + 127).astype(np.uint8))   # floor(log2 448 * 2^e) - 8 = e
    assert np.array_equal(e8[:, 1], (exps + 127).astype(np.uint8))
    z = np.zeros((1, 32), np.float32)
    c, e8, vals = O.mx_quantize_fp8(z, axis=1)
    assert e8[0, 0] == 127 and not c.any() and not vals.any()
    # random data: relative error at most 2^-4 between the block's subnormal range
    # and 448 * 2^e; above that (the block max can reach 512 * 2^e) elements saturate
    y = (rng.standard_normal((16, 64)) * 3).astype(np.float32)
    _, e8, vals = O.mx_quantize_fp8(y, axis=1)
    e = np.repeat(e8.astype(np.int64) - 127, 32, axis=1)
    top = 448.0 * np.exp2(e.astype(np.float64))
    mid = (np.abs(y) >= np.exp2(e - 6.0)) & (np.abs(y) <= top)
    assert np.all(np.abs(vals - y)[mid] <= np.abs(y)[mid] * 2.0 ** -4)
    sat = np.abs(y) > top
    assert np.array_equal(vals[sat], np.sign(y[sat]) * top[sat])


@pytest.mark.parametrize("causal", [False, True])
def test_mxfp4_with_fp8_pv_equals_exact_attention_on_decoded_operands(causal):
    q, k, v = make_custom(1, 2, 160, 64, seed=15)
    d = O.quant_mxfp4(q, k, v, v_fp8=True)
    ex = O.exact_attention(d["q_vals"], d["k_vals"], d["v_vals"], causal=causal, sm_scale=0.125)
    got = O.mxfp4_attention(q, k, v, causal=causal, sm_scale=0.125, quantize_p=False, pv_fp8=True)
    assert np.max(np.abs(got - ex)) < 1e-12
    # FP8 P moves O far less than FP4 P does
    e8p = np.max(np.abs(O.mxfp4_attention(q, k, v, causal=causal, sm_scale=0.125, pv_fp8=True) - ex))
    d4 = O.quant_mxfp4(q, k, v)
    ex4 = O.exact_attention(d4["q_vals"], d4["k_vals"], d4["v_vals"], causal=causal, sm_scale=0.125)
    e4p = np.max(np.abs(O.mxfp4_attention(q, k, v, causal=causal, sm_scale=0.125) - ex4))
    assert 0 < e8p < e4p


def test_pack_fp4_low_nibble_first():
    c = np.array([[1, 2, 15, 0, 8, 7]], np.uint8)
    assert O.pack_fp4(c).tolist() == [[0x21, 0x0F, 0x78]]


def test_mxfp4_emulation_exact_on_representable_inputs():
    # Q, V exactly representable in MXFP4, K with an exactly zero token mean (pairs +x, -x)
    # so that smoothing is the identity: without P quantization the emulation must equal
    # exact attention; with it, stay within P's quantization error.
    rng = np.random.default_rng(12)
    N, d = 64, 64

    def grid(shape, axis_len_block):
        m = rng.integers(0, 7, size=shape)
        s = rng.integers(0, 2, size=shape)
        return np.where(s, -1, 1) * O.E2M1_MAGNITUDES[m] * 0.25

    q = grid((1, 1, N, d), 32); q[..., ::32] = 1.5   # block max 1.5 -> exponent -2 keeps values exact
    half = grid((1, 1, N // 2, d), 32); half[..., ::32] = 1.5
    k = np.concatenate([half, -half], axis=2)
    v = grid((1, 1, N, d), 32); v[:, :, ::32, :] = 1.5
    q, k, v = q.astype(np.float16), k.astype(np.float16), v.astype(np.float16)
    assert np.all(O.k_mean(k) == 0)
    ex = O.exact_attention(q, k, v, causal=False, sm_scale=0.3)
    got = O.mxfp4_attention(q, k, v, causal=False, sm_scale=0.3, quantize_p=False)
    assert np.max(np.abs(got - ex)) < 1e-12
    gotp = O.mxfp4_attention(q, k, v, causal=False, sm_scale=0.3)
    assert np.max(np.abs(gotp - ex)) < 0.25 * np.abs(v.astype(float)).max()


def test_metrics_definitions():
    a = np.array([1.0, 2.0, -3.0])
    m = O.metrics(a, a)
    assert abs(m["cos"] - 1) < 1e-15 and m["max_abs"] == 0 and m["rmse"] == 0
    m = O.metrics(-a, a)
    assert abs(m["cos"] + 1) < 1e-15 and m["rel_l1"] == 2.0


@pytest.mark.parametrize("causal", [False, True])
def test_int8_emulation_equals_exact_attention_on_dequantized_operands(causal):
    # The only rounding left after dequantization is P -> fp16 (2^-11 relative per weight).
    q, k, v = make_custom(1, 2, 200, 32, seed=13)
    d = O.quant_qk_int8(q, k, blk_q=128, blk_k=32)
    idx = np.arange(200)
    qh = d["q_codes"].astype(np.float64) * d["q_scales"][:, :, idx // 128, None]
    kh = d["k_codes"].astype(np.float64) * d["k_scales"][:, :, idx // 32, None]
    ex = O.exact_attention(qh, kh, v, causal=causal, sm_scale=0.3)
    got = O.int8_attention(q, k, v, causal=causal, sm_scale=0.3, blk_q=128, blk_k=32)
    vmax = np.abs(v.astype(float)).max()
    assert np.max(np.abs(got - ex)) < 2 ** -10 * vmax
    assert np.max(np.abs(got - ex)) > 1e-6       # the fp16 rounding of P is really applied


@pytest.mark.parametrize("causal", [False, True])
def test_mxfp4_emulation_equals_exact_attention_on_decoded_operands(causal):
    q, k, v = make_custom(1, 2, 160, 64, seed=14)
    d = O.quant_mxfp4(q, k, v)
    ex = O.exact_attention(d["q_vals"], d["k_vals"], d["v_vals"], causal=causal, sm_scale=0.125)
    got = O.mxfp4_attention(q, k, v, causal=causal, sm_scale=0.125, quantize_p=False)
    assert np.max(np.abs(got - ex)) < 1e-12
    gotp = O.mxfp4_attention(q, k, v, causal=causal, sm_scale=0.125)
    assert 0 < np.max(np.abs(gotp - ex)) < 0.5


def test_oracle_regression_fixture():
    # tests/golden/tiny_oracle.json was written by tests/golden/make_golden.py (oracle only).
    import json, os, importlib.util
    here = os.path.join(os.path.dirname(__file__), "golden")
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(here, "make_golden.py"))
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    with open(os.path.join(here, "tiny_oracle.json")) as f:
        stored = json.load(f)
    assert mg.build() == stored


def test_online_softmax_forms_p_against_the_running_max():
    # Reading R6: P of each tile is exp(S - m_t) with m_t the running max. Row 0 climbs
    # (the max moves on every tile), row 1 has its max in the first tile, row 2 starts
    # masked. The largest P handed to the rounding in a tile is exp(tile max - m_t): 1
    # where the tile holds the running max, below 1 where it does not.
    S = np.array([[0.0, 1.0, 2.0, 3.0, 2.5, 4.0],
                  [5.0, 1.0, 2.0, 3.0, 2.5, 4.0],
                  [-np.inf, -np.inf, 1.0, 0.5, -2.0, 0.0]])
    V = np.arange(12, dtype=np.float64).reshape(6, 2)
    seen = []
    got = O.online_softmax_pv(S, V, kv_tile=2, round_p=lambda P: (seen.append(P.copy()), P)[1])
    want_max = [[1.0, 1.0, 1.0], [1.0, math.exp(3.0 - 5.0), math.exp(4.0 - 5.0)], [0.0, 1.0, math.exp(0.0 - 1.0)]]
    for t, P in enumerate(seen):
        for r in range(3):
            assert abs(P[r].max() - want_max[r][t]) < 1e-15
    assert abs(seen[1][0, 0] - math.exp(2.0 - 3.0)) < 1e-15          # tile 1 of row 0: against m = 3
    ex = np.exp(S - S.max(axis=1, keepdims=True))
    assert np.max(np.abs(got - (ex @ V) / ex.sum(axis=1, keepdims=True))) < 1e-13


# ---------------------------------------------------------------------------
# INT8 P and V variant (reading R14)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N", [1, 37, 130])
def test_int8_v_channel_codes_exact(N):
    v = (RNG.standard_normal((1, 2, N, 6)) * 3.0).astype(np.float16)
    v[0, 1, :, 4] = 0                                    # an all-zero channel: scale 0, codes 0
    codes, scales = O.int8_quant_v_channels(v)
    assert codes.shape == v.shape and scales.shape == (1, 2, 6)
    for h in range(2):
        for c in range(6):
            col = v[0, h, :, c].astype(np.float32)
            a = Fraction(float(np.abs(col).max()))
            s = _f32_round(a / 127)
            assert Fraction(float(scales[0, h, c])) == s
            if s == 0:
                assert np.all(codes[0, h, :, c] == 0)
                continue
            for n in range(N):
                want = _round_half_even(_f32_round(Fraction(float(col[n])) / s))
                assert int(codes[0, h, n, c]) == want
            assert abs(int(codes[0, h, int(np.argmax(np.abs(col))), c])) == 127


def _int8_pv_direct(q, k, v, *, causal, sm_scale, blk):
    """Brute-force loops for the INT8 P,V variant when the softmax reference is the
    row max over all keys: P = exp(S - max), weight = round_half_even(127 P),
    O = sum(weight * V_hat) / sum(weight). Codes come from the (separately pinned)
    quantizers; scores, weights and sums are plain Python."""
    d = O.quant_qk_int8(q, k, blk_q=blk, blk_k=blk)
    vc, vs = O.int8_quant_v_channels(v)
    _, H, N, D = q.shape
    out = np.zeros((1, H, N, D))
    for h in range(H):
        for i in range(N):
            S = []
            for j in range(N):
                if causal and j > i:
                    continue
                dot = sum(int(d["q_codes"][0, h, i, c]) * int(d["k_codes"][0, h, j, c]) for c in range(D))
                S.append((j, dot * float(d["q_scales"][0, h, i // blk]) * float(d["k_scales"][0, h, j // blk]) * sm_scale))
            mx = max(s for _, s in S)
            w = [(j, round(127.0 * math.exp(s - mx))) for j, s in S]
            tot = sum(x for _, x in w)
            for c in range(D):
                out[0, h, i, c] = sum(x * int(vc[0, h, j, c]) * float(vs[0, h, c]) for j, x in w) / tot
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_int8_pv_single_tile_matches_direct_loops(causal):
    # one key tile: the running max is the row max, so the online form is the direct formula
    q, k, v = make_custom(1, 2, 50, 8, seed=31)
    got = O.int8_pv_attention(q, k, v, causal=causal, sm_scale=0.4, blk_q=64, blk_k=64)
    want = _int8_pv_direct(q, k, v, causal=causal, sm_scale=0.4, blk=64)
    assert np.max(np.abs(got - want)) < 1e-12


def test_int8_pv_max_in_first_tile_matches_direct_loops():
    # Key 0 dominates every row, so the running max never moves after the first tile and the
    # four tiles (last one ragged) must add up to the direct formula.
    rng = np.random.default_rng(32)
    q = (np.abs(rng.standard_normal((1, 1, 200, 8))) + 0.5).astype(np.float16)
    k = (rng.standard_normal((1, 1, 200, 8)) * 0.3).astype(np.float16)
    k[0, 0, 0] = 4.0
    v = rng.standard_normal((1, 1, 200, 8)).astype(np.float16)
    got = O.int8_pv_attention(q, k, v, causal=False, sm_scale=0.5, blk_q=1, blk_k=1, smooth=False)
    dq = O.quant_qk_int8(q, k, blk_q=1, blk_k=1, smooth=False)
    S0 = (dq["q_codes"][0, 0].astype(float) @ dq["k_codes"][0, 0].astype(float).T) * dq["q_scales"][0, 0][:, None] \
        * dq["k_scales"][0, 0][None, :]
    assert np.all(np.argmax(S0, axis=1) == 0)
    want = _int8_pv_direct_nosmooth(q, k, v, sm_scale=0.5)
    assert np.max(np.abs(got - want)) < 1e-12


def _int8_pv_direct_nosmooth(q, k, v, *, sm_scale):
    d = O.quant_qk_int8(q, k, blk_q=1, blk_k=1, smooth=False)
    vc, vs = O.int8_quant_v_channels(v)
    _, _, N, D = q.shape
    out = np.zeros((1, 1, N, D))
    for i in range(N):
        S = [sum(int(d["q_codes"][0, 0, i, c]) * int(d["k_codes"][0, 0, j, c]) for c in range(D))
             * float(d["q_scales"][0, 0, i]) * float(d["k_scales"][0, 0, j]) * sm_scale for j in range(N)]
        mx = max(S)
        w = [round(127.0 * math.exp(s - mx)) for s in S]
        for c in range(D):
            out[0, 0, i, c] = sum(w[j] * int(vc[0, 0, j, c]) * float(vs[0, 0, c]) for j in range(N)) / sum(w)
    return out


def test_int8_pv_running_max_moves_the_weights():
    # When the max moves, earlier tiles keep the weights they were given against the old max
    # (then rescaled by exp(m_old - m_new)). Scores 0 then 3 (natural log units), one key per tile:
    # tile 0 weight round(127) = 127, tile 1 weight 127 and tile 0 becomes 127 e^-3.
    S = np.array([[0.0, 3.0]])
    V = np.array([[1.0], [0.0]])
    got = O.online_softmax_pv(S, V, kv_tile=1, round_p=lambda P: np.rint(127.0 * P) / 127.0,
                              sum_rounded=True)
    w0 = 127 * math.exp(-3.0)
    assert abs(got[0, 0] - w0 / (w0 + 127)) < 1e-15
    # single-tile form of the same row: weights against the final max, round(127 e^-3) = 6
    one = O.online_softmax_pv(S, V, kv_tile=2, round_p=lambda P: np.rint(127.0 * P) / 127.0,
                              sum_rounded=True)
    assert abs(one[0, 0] - 6 / 133) < 1e-15


def test_int8_pv_constant_v_and_weights_in_range():
    q, k, _ = make_custom(1, 1, 200, 32, seed=33)
    v = np.full((1, 1, 200, 32), 1.5, np.float16)
    _, vs = O.int8_quant_v_channels(v)
    o = O.int8_pv_attention(q, k, v, causal=True, sm_scale=0.2, blk_q=64, blk_k=64)
    # l sums the same quantized P that weights V: a constant channel comes back as its
    # dequantized value 127 * s
    assert np.max(np.abs(o - 127.0 * vs[0, 0, 0].astype(np.float64))) <= 1e-14
    seen = []
    S = np.array([[0.0, -0.001, -5.0, -0.5, 2.0, 1.9999]])
    O.online_softmax_pv(S, np.ones((6, 1)), kv_tile=2,
                        round_p=lambda P: (seen.append(np.rint(127.0 * P)), np.rint(127.0 * P) / 127.0)[1],
                        sum_rounded=True)
    w = np.concatenate(seen, axis=1)
    assert w.min() >= 0 and w.max() == 127 and np.all(w == np.rint(w))


def test_int8_pv_is_less_accurate_than_fp16_pv():
    # "Measured effects": quantizing P and V to INT8 lowers cosine similarity (99.94% -> 99.70%
    # across real-model layers); the direction holds on the synthetic prefill-like data.
    q, k, v = make_custom(1, 2, 512, 64, seed=34, k_offset_std=3.0)
    ex = O.exact_attention(q, k, v, causal=False, sm_scale=0.125)
    fp16pv = O.metrics(O.int8_attention(q, k, v, causal=False, sm_scale=0.125, blk_q=128, blk_k=64), ex)["cos"]
    int8pv = O.metrics(O.int8_pv_attention(q, k, v, causal=False, sm_scale=0.125, blk_q=128, blk_k=64), ex)["cos"]
    assert int8pv < fp16pv
    assert int8pv > 0.99


@pytest.mark.parametrize("causal", [False, True])
def test_int8_pv_multi_tile_matches_python_loops(causal):
    # Three 64-key tiles (the last ragged) on data whose row max moves between tiles: a
    # pure-Python running-max loop with integer weights round(127 exp(S - m)), the earlier
    # partial sums rescaled by exp(m_old - m_new) when m moves.
    q, k, v = make_custom(1, 1, 150, 8, seed=35, k_offset_std=1.0)
    got = O.int8_pv_attention(q, k, v, causal=causal, sm_scale=0.6, blk_q=64, blk_k=64)
    d = O.quant_qk_int8(q, k, blk_q=64, blk_k=64)
    vc, vs = O.int8_quant_v_channels(v)
    N, D = 150, 8
    moved = 0
    for i in range(N):
        m, lsum, acc = -math.inf, 0.0, [0.0] * D
        for t0 in range(0, N, 64):
            keys = [j for j in range(t0, min(t0 + 64, N)) if not (causal and j > i)]
            if not keys:
                continue
            S = {j: sum(int(d["q_codes"][0, 0, i, c]) * int(d["k_codes"][0, 0, j, c]) for c in range(D))
                 * float(d["q_scales"][0, 0, i // 64]) * float(d["k_scales"][0, 0, j // 64]) * 0.6 for j in keys}
            mt = max(S.values())
            if mt > m:
                f = math.exp(m - mt) if m > -math.inf else 0.0
                lsum, acc = lsum * f, [a * f for a in acc]
                moved += m > -math.inf
                m = mt
            for j in keys:
                w = round(127.0 * math.exp(S[j] - m))
                assert 0 <= w <= 127
                lsum += w
                for c in range(D):
                    acc[c] += w * int(vc[0, 0, j, c]) * float(vs[0, 0, c])
        want = [a / lsum for a in acc]
        assert max(abs(got[0, 0, i, c] - want[c]) for c in range(D)) < 1e-12
    assert moved > 10      # the case really exercises a moving max


def test_per_tensor_scale_and_codes():
    # One scale for the whole tensor: fp32(max|x| / 127) over every head, codes by the
    # per-block rule; for a one-head tensor it equals the per-block form with a block of N.
    x = (RNG.standard_normal((2, 3, 40, 8)) * 2.0).astype(np.float32)
    s = O.int8_tensor_scale(x)
    assert Fraction(float(s)) == _f32_round(Fraction(float(np.abs(x).max())) / 127)
    c = O.int8_quant_with_scale(x, s)
    for idx in [(0, 0, 0, 0), (1, 2, 39, 7), (0, 1, 17, 3)]:
        assert int(c[idx]) == _round_half_even(_f32_round(Fraction(float(x[idx])) / Fraction(float(s))))
    assert np.abs(c).max() == 127
    one = x[:1, :1]
    cb, sb = O.int8_quant_blocks(one, 40)
    assert sb[0, 0, 0] == O.int8_tensor_scale(one) and np.array_equal(cb, O.int8_quant_with_scale(one, sb[0, 0, 0]))
    assert np.all(O.int8_quant_with_scale(x, np.float32(0)) == 0)


@pytest.mark.parametrize("pv_fp8", [False, True])
def test_mxfp4_constant_v_comes_back_exactly(pv_fp8):
    # Reading R6 for the MXFP4 path: l sums the same MX-quantized P that multiplies V, so a
    # V that the codec represents exactly (1.5 = E2M1 code 6 at e = -2, or E4M3 at e = -8)
    # is returned exactly; with l from the unquantized P it would be off by the P
    # quantization error.
    q, k, _ = make_custom(1, 1, 200, 64, seed=36)
    v = np.full((1, 1, 200, 64), 1.5, np.float16)
    o = O.mxfp4_attention(q, k, v, causal=True, sm_scale=0.125, pv_fp8=pv_fp8)
    assert np.max(np.abs(o - 1.5)) <= 1e-14


def test_int8_p_flip_allowance_covers_a_code_on_a_half_integer():
    # INT8 P (R14): code = rint(127 P). Row 0 holds P = 1/2, i.e. 127 P = 63.5 on the
    # tie between codes 63 and 64; row 1 only holds P with 127 P a quarter away from
    # any half-integer. The allowance built as int8_pv_attention builds it must cover
    # row 0 with that code rounded the other way and be exactly 0 on row 1.
    rng = np.random.default_rng(41)
    S = np.full((2, 64), -40.0)
    S[:, 0] = 0.0                                   # P = 1: code 127 either way
    S[0, 1] = math.log(0.5)
    S[1, 1] = math.log(67.25 / 127)
    ks = rng.integers(1, 120, size=(2, 10))
    S[:, 2:12] = np.log((ks + 0.25) / 127)
    V = rng.standard_normal((64, 4))
    round127 = lambda P: np.rint(127.0 * P) / 127.0
    delta = 2.0 ** -16
    alts = lambda P: [round127(P * (1 - delta)), round127(np.minimum(P * (1 + delta), 1.0))]
    out, allow = O.online_softmax_pv(S, V, kv_tile=64, round_p=round127, sum_rounded=True,
                                     p_alternatives=alts)
    base = O.online_softmax_pv(S, V, kv_tile=64, round_p=round127, sum_rounded=True)
    assert np.array_equal(out, base)
    c1 = round127(np.exp(S))[0, 1] * 127
    assert c1 in (63.0, 64.0)

    def forced(P):
        Q = round127(P)
        Q[0, 1] = (127.0 - c1) / 127.0   # 63 <-> 64
        return Q
    flipped = O.online_softmax_pv(S, V, kv_tile=64, round_p=forced, sum_rounded=True)
    assert np.all(np.abs(flipped[0] - out[0]) <= allow[0] * (1 + 1e-12))
    assert np.all(allow[0] > 0) and np.all(allow[1] == 0)
    assert np.max(np.abs(flipped[0] - out[0])) > 0.2 * np.max(allow[0])   # the bound is not vacuous


def test_int8_pv_attention_with_flip_delta_keeps_its_output():
    q, k, v = (_rand16(1, 2, 150, 64, scale=2.0) for _ in range(3))
    plain = O.int8_pv_attention(q, k, v, causal=True, sm_scale=0.3, blk_q=64, blk_k=64)
    out, allow = O.int8_pv_attention(q, k, v, causal=True, sm_scale=0.3, blk_q=64, blk_k=64, flip_delta=2.0 ** -16)
    assert np.array_equal(out, plain)
    assert np.all(allow >= 0) and np.all(np.isfinite(allow))
    # a wider window catches more codes, never fewer
    _, wide = O.int8_pv_attention(q, k, v, causal=True, sm_scale=0.3, blk_q=64, blk_k=64, flip_delta=0.02)
    assert np.all(wide >= allow) and np.count_nonzero(wide.max(axis=-1)) > 0


def test_flip_allowance_covers_a_p_code_on_a_rounding_boundary():
    # Row 0 holds a P right at an E2M1 boundary (block max 1 -> e = -2, P = 0.625 -> 2.5,
    # halfway between codes 2 and 3): the allowance must cover the output with that code
    # rounded the other way. Row 1 has no P near a boundary (its block max is the
    # reference score, P = 1, which stays in its binade): its allowance is exactly 0.
    rng = np.random.default_rng(37)
    S = np.full((2, 32), -30.0)
    S[:, 0] = 0.0
    S[0, 1] = math.log(0.625)
    S[1, 1] = math.log(0.55)
    S[:, 2:8] = np.log(rng.uniform(0.05, 0.2, size=(2, 6)))
    V = rng.standard_normal((32, 4))
    quant = lambda P: O.mx_quantize(P, axis=1)[2]
    delta = 2.0 ** -16
    # as mxfp4_attention builds them: the reference P of exactly 1 only moves up
    alts = lambda P: [quant(np.where(P == 1.0, P, P * (1 - delta))), quant(P * (1 + delta))]
    out, allow = O.online_softmax_pv(S, V, kv_tile=32, round_p=quant, sum_rounded=True, p_alternatives=alts)
    base = O.online_softmax_pv(S, V, kv_tile=32, round_p=quant, sum_rounded=True)
    assert np.array_equal(out, base)
    p1 = quant(np.exp(S))[0, 1]
    other = 0.75 if p1 == 0.5 else 0.5
    assert p1 in (0.5, 0.75)

    def forced(P):
        Q = quant(P)
        Q[0, 1] = other
        return Q
    flipped = O.online_softmax_pv(S, V, kv_tile=32, round_p=forced, sum_rounded=True)
    assert np.all(np.abs(flipped[0] - out[0]) <= allow[0] * (1 + 1e-12))
    assert np.all(allow[0] > 0) and np.all(allow[1] == 0)
    assert np.max(np.abs(flipped[0] - out[0])) > 0.2 * np.max(allow[0])   # the bound is not vacuous


def _mx_block_py(xs, fp8):
    """One MX block of nonnegative values in plain Python (reading R8 / R13): shared
    exponent e = floor(log2 max) - 2 (E2M1) or - 8 (E4M3) from frexp; each value goes
    to the nearest grid magnitude of x * 2^-e, a tie to the even code; the grid's top
    value is where larger ones saturate."""
    import bisect
    if fp8:
        grid = [(c & 7) * 2.0 ** -9 if c >> 3 == 0 else (8 + (c & 7)) * 2.0 ** ((c >> 3) - 10) for c in range(0x7F)]
    else:
        grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    a = max(xs)
    if a == 0.0:
        return [0.0] * len(xs)
    e = max(min(math.frexp(a)[1] - 1 - (8 if fp8 else 2), 127), -127)
    out = []
    for x in xs:
        y = x * 2.0 ** -e
        i = bisect.bisect_left(grid, y)
        if i == len(grid):
            c = len(grid) - 1
        elif i == 0 or grid[i] == y:
            c = i
        else:
            dl, dh = y - grid[i - 1], grid[i] - y
            c = i - 1 if (dl < dh or (dl == dh and (i - 1) % 2 == 0)) else i
        out.append(grid[c] * 2.0 ** e)
    return out


@pytest.mark.parametrize("causal,fp8", [(False, False), (True, False), (False, True), (True, True)])
def test_mxfp4_p_quantization_matches_python_loops(causal, fp8):
    # The MXFP4 path's P quantization (R6, R8, R13) written as plain loops: for each query
    # row, 64-key tiles in order (the last one ragged: 150 = 2 * 64 + 22), the running max,
    # P = exp(S - m) with masked and missing keys at 0, one MX block per 32 keys of the tile,
    # l and O summing the quantized P. Scores come from the separately pinned MX codecs of
    # Q, K_s and V; everything after them is independent of the oracle's own code.
    q, k, v = make_custom(1, 1, 150, 64, seed=38, k_offset_std=1.0)
    sm = 0.3
    got = O.mxfp4_attention(q, k, v, causal=causal, sm_scale=sm, pv_fp8=fp8)
    d = O.quant_mxfp4(q, k, v, v_fp8=fp8)
    qv, kv, vv = d["q_vals"][0, 0], d["k_vals"][0, 0], d["v_vals"][0, 0]
    N, D = 150, 64
    moved = 0
    for i in range(N):
        m, lsum, acc = -math.inf, 0.0, [0.0] * D
        for t0 in range(0, N, 64):
            S = []
            for j in range(t0, t0 + 64):
                if j >= N or (causal and j > i):
                    S.append(-math.inf)
                else:
                    S.append(math.fsum(float(qv[i, c]) * float(kv[j, c]) for c in range(D)) * sm)
            mt = max(m, max(S))
            if mt > m:
                f = math.exp(m - mt) if m > -math.inf else 0.0
                lsum, acc = lsum * f, [x * f for x in acc]
                moved += m > -math.inf
                m = mt
            P = [math.exp(s - m) if s > -math.inf else 0.0 for s in S]
            Pq = _mx_block_py(P[:32], fp8) + _mx_block_py(P[32:], fp8)
            for jj, w in enumerate(Pq):
                if w:
                    lsum += w
                    for c in range(D):
                        acc[c] += w * float(vv[t0 + jj, c])
        want = [x / lsum for x in acc]
        assert max(abs(got[0, 0, i, c] - want[c]) for c in range(D)) < 1e-12, i
    assert moved > 20      # the running max really moves between tiles
