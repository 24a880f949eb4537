"""GPU parity on seeded random problem shapes: every forward mode (with and
without K smoothing) on random N (ragged tails from 1 token up), d, B, H,
causal masking and input distribution, against the CPU oracle with the bar of
tests/_parity.py. The cases are drawn once from a fixed seed, so a run is
reproducible and each case names its shape."""
import numpy as np
import pytest

import oracle as O
from synthetic import make_custom
from _parity import assert_output_parity, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FLIP_DELTA = 2.0 ** -16   # the oracle's float32 reach around P-code rounding boundaries


def _cases(n=24, seed=2026):
    rng = np.random.Generator(np.random.PCG64(seed))
    modes = [0, 1, 2, 3, 5, 6, 7, 0x100, 0x102, 0x106, 0x103, 0x105]
    out = []
    for i in range(n):
        mode = modes[i % len(modes)]
        d = int(rng.choice([64, 128]))
        N = int(rng.integers(1, 700))
        causal = bool(rng.random() < 0.5)
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        dist = "student_t" if rng.random() < 0.3 else "normal"
        out.append((B, H, N, d, causal, mode, dist, int(rng.integers(0, 1 << 30))))
    return out


def _oracle(q, k, v, *, causal, sm, mode):
    lo, smooth = mode & 0xFF, not (mode & 0x100)
    if lo in (0, 1, 3):
        bq, bk = {0: (128, 64), 1: (64, 64), 3: (1, 1)}[lo]
        return O.int8_attention(q, k, v, causal=causal, sm_scale=sm, blk_q=bq, blk_k=bk, smooth=smooth), None
    if lo in (6, 7):
        b = 1 if lo == 7 else None
        return O.int8_pv_attention(q, k, v, causal=causal, sm_scale=sm, blk_q=b or 128, blk_k=b or 64,
                                   smooth=smooth, flip_delta=FLIP_DELTA)
    return O.mxfp4_attention(q, k, v, causal=causal, sm_scale=sm, smooth=smooth, pv_fp8=lo == 5,
                             flip_delta=FLIP_DELTA)


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_attention_mean_amd as m
    return m


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "x".join(map(str, c[:4])) + f"-c{int(c[4])}-m{c[5]:#x}-{c[6]}")
def test_random_shape_matches_oracle(sa, case):
    B, H, N, d, causal, mode, dist, seed = case
    say("random shape", case)
    q, k, v = make_custom(B, H, N, d, seed=seed, dist=dist)
    sm = 1.0 / np.sqrt(d)
    ref, extra = _oracle(q, k, v, causal=causal, sm=sm, mode=mode)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    out = sa.sage_attn_fwd(qd, kd, vd, causal=causal, sm_scale=sm, mode=mode)
    torch.cuda.synchronize()
    assert_output_parity(out.cpu().numpy(), ref, what=f"random {case}", extra=extra)


def _bwd_cases(n=8, seed=2027):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for i in range(n):
        mode = [0, 1, 0x100, 0x101][i % 4]
        d = int(rng.choice([64, 128]))
        N = int(rng.integers(1, 600))
        causal = bool(rng.random() < 0.5)
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        dist = "student_t" if rng.random() < 0.3 else "normal"
        out.append((B, H, N, d, causal, mode, dist, int(rng.integers(0, 1 << 30))))
    return out


@pytest.mark.parametrize("case", _bwd_cases(), ids=lambda c: "x".join(map(str, c[:4])) + f"-c{int(c[4])}-m{c[5]:#x}-{c[6]}")
def test_random_shape_backward_matches_oracle(sa, case):
    """The INT8 backward on random shapes, fed the oracle's forward output and
    log-sum-exp, against the oracle's emulation with the bar of test_gpu_bwd."""
    from synthetic import make_grad
    from test_gpu_bwd import assert_grad_parity
    B, H, N, d, causal, mode, dist, seed = case
    say("random backward shape", case)
    q, k, v = make_custom(B, H, N, d, seed=seed, dist=dist)
    do = make_grad(B, H, N, d, seed=seed)
    sm = 1.0 / np.sqrt(d)
    blk_q, smooth = (64 if mode & 0xFF == 1 else 128), not (mode & 0x100)
    fw = O.int8_forward_for_training(q, k, v, causal=causal, sm_scale=sm, blk_q=blk_q, smooth=smooth)
    ref = O.int8_attention_backward(q, k, v, do, fw["o16"], fw["lse"], causal=causal, sm_scale=sm, blk_q=blk_q,
                                    smooth=smooth, with_allowance=True)
    qd, kd, vd, gd, od = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (q, k, v, do, fw["o16"]))
    ld = torch.from_numpy(fw["lse"].astype(np.float32)).cuda()
    dq, dk, dv = sa.sage_attn_bwd(qd, kd, vd, od, gd, ld, causal=causal, sm_scale=sm, mode=mode)
    torch.cuda.synchronize()
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert_grad_parity(g.cpu().numpy(), ref[name], ref[name + "_mag"], ref[name + "_allow"],
                           f"random bwd {name} {case}")
