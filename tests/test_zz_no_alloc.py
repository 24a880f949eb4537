"""GPU: sage_attn_fwd_noalloc, the entry point that allocates nothing, against
sage_attn_fwd with a caller-provided workspace. The two run the same kernels,
so their outputs must be bit-identical; two calls in a row, the second on a
smaller input, check that nothing carried over in the shared scratch matters."""
import numpy as np
import pytest

from synthetic import make_custom
from _parity import say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_attention_mean_amd as m
    return m


def _dev(*arrs):
    return [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrs]


@pytest.mark.parametrize("mode,causal,d", [(0, False, 128), (2, True, 64), (6, False, 128), (3, True, 64),
                                           (5, False, 128), (4, True, 128), (1 | 0x100, False, 64)])
def test_noalloc_equals_fwd_on_two_calls_in_a_row(sa, mode, causal, d):
    say("no-alloc entry point, mode", hex(mode), "causal", causal, "d", d)
    shapes = [(2, 3, 1500), (1, 2, 333)]        # the second call is smaller
    inputs = [_dev(*make_custom(B, H, N, d, seed=B * N + d + mode)) for (B, H, N) in shapes]
    want = [sa.sage_attn_fwd(q, k, v, causal=causal, mode=mode) for (q, k, v) in inputs]
    outs = [torch.full_like(q, float("nan")) for (q, _, _) in inputs]
    torch.cuda.synchronize()
    for (q, k, v), o in zip(inputs, outs):
        sa.sage_attn_fwd_noalloc(q, k, v, o, causal=causal, mode=mode)
    torch.cuda.synchronize()
    for w, o in zip(want, outs):
        assert torch.isfinite(o).all()
        assert torch.equal(o, w)


@pytest.mark.parametrize("mode,causal,d", [(0, False, 128), (1, True, 64)])
def test_noalloc_equals_fwd_across_the_fused_q_threshold(sa, mode, causal, d):
    """From 65536 token rows on, both entry points quantize Q inside the attention
    kernel; the first call here is above that threshold, the second below it."""
    say("no-alloc entry point across the fused-Q threshold, mode", mode, "causal", causal, "d", d)
    shapes = [(1, 16, 4200), (2, 3, 1500)]      # 67200 token rows, then 9000
    inputs = [_dev(*make_custom(B, H, N, d, seed=B * N + d + mode)) for (B, H, N) in shapes]
    want = [sa.sage_attn_fwd(q, k, v, causal=causal, mode=mode) for (q, k, v) in inputs]
    outs = [torch.full_like(q, float("nan")) for (q, _, _) in inputs]
    torch.cuda.synchronize()
    for (q, k, v), o in zip(inputs, outs):
        sa.sage_attn_fwd_noalloc(q, k, v, o, causal=causal, mode=mode)
    torch.cuda.synchronize()
    for w, o in zip(want, outs):
        assert torch.isfinite(o).all()
        assert torch.equal(o, w)


def test_noalloc_allocates_no_device_memory(sa):
    say("no-alloc entry point: device memory")
    q, k, v = _dev(*make_custom(1, 4, 2048, 128, seed=3))
    out = torch.empty_like(q)
    sa.sage_attn_fwd_noalloc(q, k, v, out)          # first call on the device: scratch address looked up
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for mode in (0, 2, 6):
        sa.sage_attn_fwd_noalloc(q, k, v, out, mode=mode)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0


def test_noalloc_refuses_a_problem_beyond_its_scratch(sa):
    q = torch.empty(1, 64, 32768, 128, dtype=torch.float16, device="cuda")
    with pytest.raises(sa.SageError) as e:
        sa.sage_attn_fwd_noalloc(q, q, q, torch.empty_like(q))
    assert e.value.status == -3
