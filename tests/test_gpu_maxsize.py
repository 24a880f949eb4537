"""GPU parity at the longest sequence the library accepts: N = 2^22 tokens in one head.

The INT8 path (Q blocks of 128, K blocks of 64) at that length, once with a
ragged last key tile (N = 2^22 - 37, d = 128, non-causal) and once at exactly
2^22 (d = 64, causal): the K mean, the scales and every Q and K code bit for
bit against the oracle, then the attention output of sage_attn_fwd (which
quantizes Q inside the attention kernel at this size) on sampled query rows,
element by element. V carries a per-channel offset and the softmax scale is
three times 1/sqrt(d), so that the outputs are of order one rather than the
near-zero mean of unit-normal V over millions of keys: an error in the row sums
or in the accumulation over the 65536 key tiles then shows at full size.
Host memory: about 25 GB for the oracle's float64 copies.
"""
import numpy as np
import pytest

import oracle as O
from synthetic import make_custom
from _parity import assert_output_parity, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MAX_N = 1 << 22   # the largest N sage_attn_fwd accepts


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_attention_mean_amd as m
    return m


@pytest.mark.parametrize("N,d,causal", [(MAX_N - 37, 128, False), (MAX_N, 64, True)],
                         ids=["n4194267-d128", "n4194304-d64-causal"])
def test_maximum_sequence_length(sa, N, d, causal):
    say(f"maximum length: B=1 H=1 N={N} d={d} causal={causal} mode=int8_q128_k64")
    q, k, v = make_custom(1, 1, N, d, seed=4242 + d)
    voff = np.random.default_rng(77 + d).standard_normal(d).astype(np.float32)
    v = (v.astype(np.float32) + voff).astype(np.float16)
    sm = 3.0 / np.sqrt(d)
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))

    got = sa.sage_quant_qk(qd, kd, blk_q=128, blk_k=64)
    torch.cuda.synchronize()
    ref = O.quant_qk_int8(q, k, blk_q=128, blk_k=64)
    for key in ("k_mean", "q_scales", "k_scales"):
        assert np.array_equal(got[key].cpu().numpy().view(np.uint32), ref[key].view(np.uint32)), key
    for key in ("q_codes", "k_codes"):
        assert np.array_equal(got[key].cpu().numpy(), ref[key]), key
    del got
    say("  quantization bit-exact")

    out = sa.sage_attn_fwd(qd, kd, vd, causal=causal, sm_scale=sm, mode=sa.SAGE_MODE_INT8_Q128_K64)
    torch.cuda.synchronize()
    say("  attention done on the GPU")
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(N - 4, N), rng.choice(N, 16, replace=False)]))
    got_rows = out[0, 0, torch.from_numpy(rows).cuda()].cpu().numpy()
    assert np.all(np.isfinite(got_rows))
    ref_rows = O.int8_attention(q, k, v, causal=causal, sm_scale=sm, blk_q=128, blk_k=64, rows=rows, quant=ref)
    err = assert_output_parity(got_rows, ref_rows[0, 0], what=f"maximum length N={N} d={d}")
    say(f"  {rows.size} rows, max |gpu - oracle| = {err:.2e}, max |O| = {np.abs(ref_rows).max():.3f}")
