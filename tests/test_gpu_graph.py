"""The C ABI's calls under HIP graph capture (torch.cuda.CUDAGraph), on the GPU.

The library only enqueues kernels on the caller's stream (no allocation,
memset, copy or synchronization inside a call), so a caller can capture a call
once and replay it. Each case captures one call with fixed buffers, then
replays it three times, each time with new inputs copied into the captured
buffers and an eager call on other buffers (its own workspace) plus a device
synchronization in between; every replay must equal the eager result bit for
bit. Forward: per-block INT8 below and above the size from which Q is
quantized in the attention kernel's prologue, MXFP4, INT8 P.V; and the INT8
backward pass.
"""
import pytest

from synthetic import make_custom, make_grad
from _parity import say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_attention_mean_amd as m
    return m


def _inputs(B, H, N, d, seed):
    return [torch.from_numpy(x).cuda() for x in make_custom(B, H, N, d, seed=seed)]


def _capture(fn):
    """Warm fn up on a side stream, then capture one call of it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


FWD_CASES = [
    # B, H, N, d, causal, mode
    (1, 2, 700, 128, True, 0),
    (1, 2, 40000, 128, False, 0),     # 80000 rows: Q quantized in the kernel's prologue
    (2, 1, 333, 64, False, 2),
    (1, 2, 515, 128, True, 6),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "x".join(map(str, c[:4])) + f"-c{int(c[4])}-m{c[5]}")
def test_forward_replays_in_a_graph(sa, case):
    B, H, N, d, causal, mode = case
    say("graph forward", case)
    sm = d ** -0.5
    qs, ks, vs = (torch.empty((B, H, N, d), dtype=torch.float16, device="cuda") for _ in range(3))
    for t, x in zip((qs, ks, vs), _inputs(B, H, N, d, seed=100)):
        t.copy_(x)
    out = torch.empty_like(qs)
    ws = sa.make_workspace(B, H, N, d, mode, qs.device)
    g = _capture(lambda: sa.sage_attn_fwd(qs, ks, vs, out, causal=causal, sm_scale=sm, mode=mode, workspace=ws))
    for rep in range(3):
        q, k, v = _inputs(B, H, N, d, seed=200 + rep)
        qs.copy_(q); ks.copy_(k); vs.copy_(v)
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = sa.sage_attn_fwd(q, k, v, causal=causal, sm_scale=sm, mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"replay {rep} differs from the eager call"
    say("  three replays bit-identical to eager calls")


@pytest.mark.parametrize("causal", [False, True])
def test_backward_replays_in_a_graph(sa, causal):
    B, H, N, d = 1, 2, 600, 64
    say("graph backward", (B, H, N, d, causal))
    sm = d ** -0.5
    bufs = [torch.empty((B, H, N, d), dtype=torch.float16, device="cuda") for _ in range(4)]  # q, k, v, dout
    qs, ks, vs, gs = bufs
    out = torch.empty_like(qs)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty((B, H, N, d), dtype=torch.float32, device="cuda") for _ in range(3))
    ws = sa.make_bwd_workspace(B, H, N, d, 0, qs.device)

    def step():
        sa.sage_attn_fwd_lse(qs, ks, vs, out, lse, causal=causal, sm_scale=sm, workspace=ws)
        sa.sage_attn_bwd(qs, ks, vs, out, gs, lse, dq, dk, dv, causal=causal, sm_scale=sm, workspace=ws)

    for t, x in zip(bufs, _inputs(B, H, N, d, seed=300) + [torch.from_numpy(make_grad(B, H, N, d, seed=300)).cuda()]):
        t.copy_(x)
    g = _capture(step)
    for rep in range(3):
        q, k, v = _inputs(B, H, N, d, seed=400 + rep)
        gd = torch.from_numpy(make_grad(B, H, N, d, seed=400 + rep)).cuda()
        for t, x in zip(bufs, (q, k, v, gd)):
            t.copy_(x)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (out, lse, dq, dk, dv)]
        o_ref, lse_ref = sa.sage_attn_fwd_lse(q, k, v, causal=causal, sm_scale=sm)
        ref = [o_ref, lse_ref, *sa.sage_attn_bwd(q, k, v, o_ref, gd, lse_ref, causal=causal, sm_scale=sm)]
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "lse", "dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
    say("  three replays bit-identical to eager calls")
