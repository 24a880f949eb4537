"""GPU parity of the INT8 backward pass and of the training forward's log-sum-exp.

The HIP path (through the C ABI: sage_attn_fwd_lse, sage_attn_bwd) against the
CPU oracle (oracle.sage_bwd_oracle). The backward is fed the oracle's forward
output and log-sum-exp on both sides, so its parity is the backward's alone:
each gradient element must lie within 2^-12 of the sum of the absolute values
of the terms it adds up (the scale of fp32 accumulation rounding; "mag"), plus
the oracle's first-order allowance for the P and dS codes that float32
arithmetic may round the other way (Rb3), capped at 2^-6 of mag. A chained
test runs the GPU forward into the GPU backward and checks the method's
accuracy against the exact float64 gradients.
"""
import math

import numpy as np
import pytest

import oracle as O
from synthetic import make_custom, make_grad
from _parity import assert_output_parity, say, RECORDS

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL_BAR = 2.0 ** -12
ALLOW_CAP = 2.0 ** -6


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_attention_mean_amd as m
    return m


def _dev(*arrs):
    return [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrs]


def _mode(q128=True, smooth=True):
    return (0 if q128 else 1) | (0 if smooth else 0x100)


def assert_grad_parity(got, ref, mag, allow, what):
    """|got - ref| <= 2^-12 mag + min(allow, 2^-6 mag) + a floor of 1e-9 max|ref|."""
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradients"
    err = np.abs(got - ref)
    floor = 1e-9 * max(1.0, float(np.abs(ref).max()))
    bound = REL_BAR * mag + floor
    extra = np.minimum(allow, ALLOW_CAP * mag)
    excused = (err > bound) & (err <= bound + extra)
    bad = err > bound + extra
    n_exc = int(excused.sum())
    used = float(np.max((err - bound) / np.maximum(mag, 1e-300), where=excused, initial=0.0))
    say(f"  {what}: {err.size} elements, max err {err.max():.3e} (max|ref| {np.abs(ref).max():.3e}); "
        f"{n_exc} excused by the code-flip allowance (largest excess {used:.2e} of mag)")
    RECORDS.append((what, err.size, float(err.max()), n_exc, used, " of mag",
                    float(np.max(err / (bound + extra)))))
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound - extra), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements over tolerance; worst at {i}: got {got[i]!r} "
                             f"ref {ref[i]!r} err {err[i]:.3e} mag {mag[i]:.3e} allow {allow[i]:.3e}")


LSE_CASES = [
    # B, H, N, d, causal, q128, smooth, dist
    (1, 2, 256, 64, False, True, True, "normal"),
    (1, 2, 300, 64, True, True, True, "normal"),
    (1, 1, 520, 128, True, False, True, "student_t"),
    (2, 1, 200, 128, False, True, False, "normal"),
]


@pytest.mark.parametrize("case", LSE_CASES, ids=lambda c: "x".join(map(str, c[:4])) + f"-c{int(c[4])}-q{128 if c[5] else 64}-s{int(c[6])}-{c[7]}")
def test_training_forward_lse(sa, case):
    """sage_attn_fwd_lse: the output is the forward's (same bar as sage_attn_fwd)
    and the log-sum-exp is within 2^-10: the kernel's lazily moved reference
    max rounds the fp16 weights l sums at another point, a relative change of
    at most 2^-11 in l."""
    B, H, N, d, causal, q128, smooth, dist = case
    say("fwd_lse", case)
    q, k, v = make_custom(B, H, N, d, seed=21 + N, dist=dist)
    sm = 1.0 / math.sqrt(d)
    ref = O.int8_forward_for_training(q, k, v, causal=causal, sm_scale=sm, blk_q=128 if q128 else 64, smooth=smooth)
    qd, kd, vd = _dev(q, k, v)
    out, lse = sa.sage_attn_fwd_lse(qd, kd, vd, causal=causal, sm_scale=sm, mode=_mode(q128, smooth))
    torch.cuda.synchronize()
    assert_output_parity(out.cpu().numpy(), ref["o"], what=f"fwd_lse out {case}")
    dl = np.abs(lse.cpu().numpy().astype(np.float64) - ref["lse"])
    say(f"  lse: max |dL| {dl.max():.3e}")
    assert dl.max() <= 2.0 ** -10


BWD_CASES = [
    # B, H, N, d, causal, q128, smooth, dist, dO scale
    (1, 2, 256, 64, False, True, True, "normal", 1.0),
    (1, 2, 300, 64, True, True, True, "normal", 1.0),
    (1, 1, 520, 128, False, True, True, "normal", 1.0),
    (2, 1, 384, 128, True, True, True, "normal", 1.0),
    (1, 2, 200, 128, False, False, True, "normal", 1.0),
    (1, 2, 333, 64, True, True, False, "student_t", 1.0),
    (1, 1, 130, 128, True, False, False, "student_t", 1e-3),
    (1, 1, 1, 64, False, True, True, "normal", 1.0),
    (1, 2, 33, 128, True, True, True, "normal", 1.0),
]


def _run_bwd(sa, q, k, v, do, o16, lse, causal, sm, mode):
    qd, kd, vd, gd, od = _dev(q, k, v, do, o16)
    ld, = _dev(lse.astype(np.float32))
    dq, dk, dv = sa.sage_attn_bwd(qd, kd, vd, od, gd, ld, causal=causal, sm_scale=sm, mode=mode)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "x".join(map(str, c[:4])) + f"-c{int(c[4])}-q{128 if c[5] else 64}-s{int(c[6])}-{c[7]}-g{c[8]}")
def test_backward_matches_oracle(sa, case):
    B, H, N, d, causal, q128, smooth, dist, gscale = case
    say("bwd", case)
    q, k, v = make_custom(B, H, N, d, seed=31 + N, dist=dist)
    do = make_grad(B, H, N, d, seed=31 + N, scale=gscale)
    sm = 1.0 / math.sqrt(d)
    blk_q = 128 if q128 else 64
    fw = O.int8_forward_for_training(q, k, v, causal=causal, sm_scale=sm, blk_q=blk_q, smooth=smooth)
    ref = O.int8_attention_backward(q, k, v, do, fw["o16"], fw["lse"], causal=causal, sm_scale=sm, blk_q=blk_q,
                                    smooth=smooth, with_allowance=True)
    say(f"  oracle: {ref['p_flips']} P codes and {ref['ds_flips']} dS codes within float32 reach of a boundary")
    got = _run_bwd(sa, q, k, v, do, fw["o16"], fw["lse"], causal, sm, _mode(q128, smooth))
    for name, g in zip(("dq", "dk", "dv"), got):
        assert_grad_parity(g, ref[name], ref[name + "_mag"], ref[name + "_allow"], f"bwd {name} {case}")


def test_backward_zero_gradient_is_exactly_zero(sa):
    B, H, N, d = 1, 2, 200, 128
    q, k, v = make_custom(B, H, N, d, seed=5)
    sm = 1.0 / math.sqrt(d)
    fw = O.int8_forward_for_training(q, k, v, causal=True, sm_scale=sm)
    got = _run_bwd(sa, q, k, v, np.zeros((B, H, N, d), np.float16), fw["o16"], fw["lse"], True, sm, 0)
    for g in got:
        assert np.abs(g).max() == 0.0


@pytest.mark.parametrize("causal", [False, True])
def test_chained_gpu_forward_and_backward_track_exact_gradients(sa, causal):
    """GPU forward (out, lse) into the GPU backward: the gradients follow the exact
    float64 ones with the accuracy of the method (cosine similarity of each
    gradient >= 0.999 on unit-variance inputs; the oracle's emulation reaches
    0.9994-0.9996 here)."""
    B, H, N, d = 1, 2, 640, 128
    q, k, v = make_custom(B, H, N, d, seed=41)
    do = make_grad(B, H, N, d, seed=41)
    sm = 1.0 / math.sqrt(d)
    qd, kd, vd, gd = _dev(q, k, v, do)
    out, lse = sa.sage_attn_fwd_lse(qd, kd, vd, causal=causal, sm_scale=sm)
    dq, dk, dv = sa.sage_attn_bwd(qd, kd, vd, out, gd, lse, causal=causal, sm_scale=sm)
    torch.cuda.synchronize()
    ex = O.exact_attention_backward(q, k, v, do, causal=causal, sm_scale=sm)
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        a, b = g.cpu().numpy().astype(np.float64).ravel(), ex[name].ravel()
        cos = float(a @ b / np.linalg.norm(a) / np.linalg.norm(b))
        say(f"  chained {name} (causal={causal}): cos vs exact {cos:.6f}")
        assert cos >= 0.999


@pytest.mark.parametrize("causal", [False, True])
def test_backward_full_prefill_size_sampled_heads(sa, causal):
    """The prefill shape (B=4, H=32, N=4096, d=128, outlier K channels) in the launch
    configuration the bench times; two whole heads checked against the oracle.
    The backward's saved-forward inputs (out, lse) come from the GPU forward for
    every head except the two checked ones, whose slices are overwritten with the
    oracle's forward, so the oracle never reads a value the HIP path produced."""
    from synthetic import make_inputs
    q, k, v = make_inputs("prefill")
    B, H, N, d = q.shape
    do = make_grad(B, H, N, d, seed=1)
    sm = 1.0 / math.sqrt(d)
    qd, kd, vd, gd = _dev(q, k, v, do)
    out, lse = sa.sage_attn_fwd_lse(qd, kd, vd, causal=causal, sm_scale=sm)
    heads = ((0, 0), (3, 31))
    fws = {}
    for (b, h) in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        fws[b, h] = O.int8_forward_for_training(q[sl], k[sl], v[sl], causal=causal, sm_scale=sm)
        out[b, h] = torch.from_numpy(fws[b, h]["o16"][0, 0]).cuda()
        lse[b, h] = torch.from_numpy(fws[b, h]["lse"][0, 0].astype(np.float32)).cuda()
    dq, dk, dv = sa.sage_attn_bwd(qd, kd, vd, out, gd, lse, causal=causal, sm_scale=sm)
    torch.cuda.synchronize()
    for (b, h) in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = O.int8_attention_backward(q[sl], k[sl], v[sl], do[sl], fws[b, h]["o16"], fws[b, h]["lse"],
                                        causal=causal, sm_scale=sm, with_allowance=True)
        for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
            assert_grad_parity(g[sl].cpu().numpy(), ref[name], ref[name + "_mag"], ref[name + "_allow"],
                               f"bwd prefill head ({b},{h}) {name} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_autograd_function_is_the_c_abi_pair(sa, causal):
    """sage_attention under torch autograd: the output is sage_attn_fwd_lse's and the
    gradients reaching fp16 q, k, v are sage_attn_bwd's float32 gradients rounded to
    fp16 (the same kernels on the same inputs, so bit for bit)."""
    B, H, N, d = 1, 2, 200, 64
    say("autograd", (B, H, N, d, causal))
    q, k, v = make_custom(B, H, N, d, seed=51)
    do = make_grad(B, H, N, d, seed=51)
    qd, kd, vd, gd = _dev(q, k, v, do)
    for t in (qd, kd, vd):
        t.requires_grad_(True)
    out = sa.sage_attention(qd, kd, vd, causal=causal)
    out.backward(gd)
    torch.cuda.synchronize()
    with torch.no_grad():
        ref_out, lse = sa.sage_attn_fwd_lse(qd.detach(), kd.detach(), vd.detach(), causal=causal)
        dq, dk, dv = sa.sage_attn_bwd(qd.detach(), kd.detach(), vd.detach(), ref_out, gd, lse, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), ref_out)
    for name, t, g in (("dq", qd, dq), ("dk", kd, dk), ("dv", vd, dv)):
        assert t.grad is not None and t.grad.dtype == torch.float16, name
        assert torch.equal(t.grad, g.to(torch.float16)), name
