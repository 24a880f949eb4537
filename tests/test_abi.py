"""C ABI contract, checked on the CPU: the library loads, exports every function
include/sage_attn.h declares, and rejects every invalid argument before any HIP
call (so the same errors come back on a host without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage_attn.h")

sa = pytest.importorskip("bit_quantized_attention_mean_amd")
lib = sa.lib

OK, INVALID, UNSUP, WS, NODEV, HIP = 0, -1, -2, -3, -4, -5
A16 = 0x10000          # a 16/256-aligned fake address; never dereferenced in these tests


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sage_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    declared = _declared_functions()
    assert declared, "no declarations parsed"
    assert sorted(sa.EXPORTED_SYMBOLS) == declared
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings_cover_every_code():
    names = {c: sa.sage_status_string(c) for c in (OK, INVALID, UNSUP, WS, NODEV, HIP)}
    assert names[OK] == "SAGE_OK" and names[HIP] == "SAGE_ERR_HIP"
    assert len(set(names.values())) == 6
    assert sa.sage_status_string(-99) == "SAGE_ERR_UNKNOWN"


def test_workspace_sizes():
    assert sa.sage_attn_workspace_size(1, 2, 256, 64, 0) > 0
    assert sa.sage_attn_workspace_size(0, 2, 256, 64, 0) == 0
    assert sa.sage_attn_workspace_size(1, 2, 256, 96, 0) == 0
    assert sa.sage_attn_workspace_size(1, 2, 256, 64, 8) == 0
    small = sa.sage_attn_workspace_size(1, 2, 256, 128, 0)
    big = sa.sage_attn_workspace_size(1, 2, 4096, 128, 0)
    assert big > small
    # INT8 with fp16 P.V: Q, K codes (2 B/elem) dominate (V is read as given); MXFP4: ~1.6 B/elem
    n = 4 * 32 * 4096 * 128
    assert 2 * n <= sa.sage_attn_workspace_size(4, 32, 4096, 128, 0) < 2.2 * n
    assert 1.5 * n <= sa.sage_attn_workspace_size(4, 32, 4096, 128, 2) < 1.8 * n
    # FP16 baseline: only the K mean (Q, K, V are read as given); MXFP4 with MX-FP8 V: ~2.1 B/elem
    assert 0 < sa.sage_attn_workspace_size(4, 32, 4096, 128, 4) < 0.05 * n
    assert 2 * n <= sa.sage_attn_workspace_size(4, 32, 4096, 128, 5) < 2.3 * n
    # INT8 P.V: Q, K codes (2 B/elem) + INT8 V^T (1 B/elem)
    for mode in (6, 7):
        assert 3 * n <= sa.sage_attn_workspace_size(4, 32, 4096, 128, mode) < 3.2 * n
    assert sa.sage_attn_workspace_size(1, 2, (1 << 17) + 1, 64, 6) == 0     # int32 P.V sums bound N
    assert sa.sage_attn_workspace_size(1, 2, (1 << 17) + 1, 64, 0) > 0
    assert sa.sage_attn_workspace_size(1, 2, 256, 64, 0x200 | 2) == 0   # the V-format flag is quantization-only
    assert sa.sage_quant_workspace_size(1, 2, 256, 64) > 0


def _fwd(q=A16, k=A16, v=A16, out=A16, B=1, H=2, N=256, d=64, causal=0, scale=0.125, mode=0, ws=A16, wsb=None):
    if wsb is None:
        wsb = sa.sage_attn_workspace_size(B, H, N, d, mode) or 1 << 20
    return lib.sage_attn_fwd(q, k, v, out, B, H, N, d, causal, scale, mode, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(out=None), INVALID),
    (dict(q=A16 + 8), INVALID), (dict(out=A16 + 2), INVALID), (dict(ws=A16 + 16), INVALID),
    (dict(B=0), INVALID), (dict(H=-1), INVALID), (dict(N=0), INVALID), (dict(N=(1 << 22) + 1), INVALID),
    (dict(d=96), UNSUP), (dict(d=256), UNSUP), (dict(mode=9), UNSUP), (dict(mode=8), UNSUP),
    (dict(mode=0x200), UNSUP), (dict(mode=6, N=(1 << 17) + 1), UNSUP), (dict(mode=7 | 0x100, N=(1 << 17) + 1), UNSUP),
    (dict(scale=0.0), INVALID), (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(scale=-1.0), INVALID), (dict(causal=2), INVALID), (dict(wsb=1024), WS),
])
def test_fwd_rejects_invalid_arguments_before_touching_the_gpu(kw, code):
    assert _fwd(**kw) == code
    assert sa.sage_last_error() != ""


def test_prepare_compute_and_quant_validation():
    ws = sa.sage_attn_workspace_size(1, 2, 256, 64, 0)
    assert lib.sage_attn_prepare(None, A16, A16, 1, 2, 256, 64, 0, A16, ws, None) == INVALID
    assert lib.sage_attn_prepare(A16, A16, A16, 1, 2, 256, 64, 0, A16, 10, None) == WS
    assert lib.sage_attn_compute(None, None, A16, A16, 1, 2, 256, 64, 0, 0.0, 0, A16, ws, None) == INVALID
    assert lib.sage_attn_compute(None, None, A16, A16, 1, 2, 256, 48, 0, 0.1, 0, A16, ws, None) == UNSUP
    # the fp16 P.V modes read v in the attention phase: null or misaligned is refused
    assert lib.sage_attn_compute(None, None, None, A16, 1, 2, 256, 64, 0, 0.1, 0, A16, ws, None) == INVALID
    assert lib.sage_attn_compute(None, None, A16 + 2, A16, 1, 2, 256, 64, 0, 0.1, 0, A16, ws, None) == INVALID
    # the unquantized baseline reads q and k in the attention phase
    ws4 = sa.sage_attn_workspace_size(1, 2, 256, 64, 4)
    assert lib.sage_attn_compute(None, A16, A16, A16, 1, 2, 256, 64, 0, 0.1, 4, A16, ws4, None) == INVALID
    assert lib.sage_attn_compute(A16, A16 + 2, A16, A16, 1, 2, 256, 64, 0, 0.1, 4, A16, ws4, None) == INVALID
    assert lib.sage_attn_compute(A16, A16, None, A16, 1, 2, 256, 64, 0, 0.1, 4, A16, ws4, None) == INVALID
    assert lib.sage_attn_compute(A16, A16, A16, A16, 1, 2, 256, 64, 0, 0.1, 8, A16, ws4, None) == UNSUP
    # the INT8 P.V workspace also holds INT8 V^T and its channel scales (and v may be null)
    ws0 = sa.sage_attn_workspace_size(1, 2, 256, 64, 0)
    ws6 = sa.sage_attn_workspace_size(1, 2, 256, 64, 6)
    assert ws6 != ws0
    assert lib.sage_attn_compute(None, None, None, A16, 1, 2, 256, 64, 0, 0.1, 6, A16, ws6 - 1, None) == WS
    qw = sa.sage_quant_workspace_size(1, 2, 256, 64)
    assert lib.sage_quant_qk(A16, A16, 1, 2, 256, 64, 48, 64, 0, A16, A16, A16, A16, None, A16, qw, None) == UNSUP
    assert lib.sage_quant_qk(A16, A16, 1, 2, 256, 64, 64, 64, 4, A16, A16, A16, A16, None, A16, qw, None) == UNSUP
    assert lib.sage_quant_qk(A16, A16, 1, 2, 256, 64, 64, 64, 0, None, A16, A16, A16, None, A16, qw, None) == INVALID
    assert lib.sage_quant_qk(A16, A16, 1, 2, 256, 64, 64, 64, 0, A16, A16, A16, A16, None, A16, 8, None) == WS
    assert lib.sage_quant_mxfp4(A16, A16, A16, 1, 2, 256, 64, 0, A16, A16, A16, A16, A16 + 4, A16, None, A16, qw,
                                None) == INVALID
    # the integer-score dump: INT8 modes 0, 1, 3 only, tile indices in range
    assert lib.sage_attn_dump_scores(A16, A16, 1, 2, 1000, 64, 0.1, 0, A16, ws0 * 4, 0, 0, 0, None, None) == INVALID
    assert lib.sage_attn_dump_scores(A16, A16, 1, 2, 256, 64, 0.1, 2, A16, 1 << 30, 0, 0, 0, A16, None) == UNSUP
    assert lib.sage_attn_dump_scores(A16, A16, 1, 2, 256, 64, 0.1, 4, A16, 1 << 30, 0, 0, 0, A16, None) == UNSUP
    assert lib.sage_attn_dump_scores(A16, A16, 1, 2, 256, 64, 0.1, 0, A16, ws0, 2, 0, 0, A16, None) == INVALID
    assert lib.sage_attn_dump_scores(A16, A16, 1, 2, 256, 64, 0.1, 0, A16, ws0, 0, 1, 0, A16, None) == INVALID
    assert lib.sage_attn_dump_scores(A16, A16, 1, 2, 256, 64, 0.1, 0, A16, ws0, 0, 0, 4, A16, None) == INVALID
    assert lib.sage_attn_dump_scores(A16, A16, 1, 2, 256, 64, 0.0, 0, A16, ws0, 0, 0, 0, A16, None) == INVALID
    assert lib.sage_quant_v_int8(None, 1, 2, 256, 64, A16, A16, A16, qw, None) == INVALID
    assert lib.sage_quant_v_int8(A16, 1, 2, 256, 64, A16 + 8, A16, A16, qw, None) == INVALID
    assert lib.sage_quant_v_int8(A16, 1, 2, 256, 64, A16, A16 + 2, A16, qw, None) == INVALID
    assert lib.sage_quant_v_int8(A16, 1, 2, 256, 80, A16, A16, A16, qw, None) == UNSUP
    assert lib.sage_quant_v_int8(A16, 1, 2, 256, 64, A16, A16, A16, 8, None) == WS


def test_clock_probe_validation():
    assert lib.sage_clock_probe(1000, None, None) == INVALID
    assert lib.sage_clock_probe(1000, A16 + 4, None) == INVALID
    assert lib.sage_clock_probe(0, A16, None) == INVALID
    assert lib.sage_clock_probe((1 << 32) + 1, A16, None) == INVALID
    assert lib.sage_wall_clock_khz(None) == INVALID


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(_gpu_visible(), reason="fake device pointers must never reach a real GPU")
def test_valid_arguments_without_a_device_report_no_device():
    assert _fwd() == NODEV
    assert "device" in sa.sage_last_error()
    qw = sa.sage_quant_workspace_size(1, 2, 256, 64)
    assert lib.sage_quant_qk(A16, A16, 1, 2, 256, 64, 64, 64, 0, A16, A16, A16, A16, None, A16, qw, None) == NODEV
    assert lib.sage_quant_v_int8(A16, 1, 2, 256, 64, A16, A16, A16, qw, None) == NODEV
    assert _fwd(mode=6) == NODEV and _fwd(mode=7) == NODEV
    ws0 = sa.sage_attn_workspace_size(1, 2, 256, 64, 0)
    assert lib.sage_attn_dump_scores(A16, A16, 1, 2, 256, 64, 0.1, 0, A16, ws0, 1, 0, 3, A16, None) == NODEV
    assert lib.sage_clock_probe(1000, A16, None) == NODEV


def test_binding_checks_v_before_any_device_call():
    # the attention phase and the score dump take the caller's fp16 V: a shape
    # that differs from out, or a host tensor, is refused in the binding
    torch = pytest.importorskip("torch")
    out = torch.empty(1, 2, 256, 64, dtype=torch.float16)
    ws = torch.empty(16, dtype=torch.uint8)
    with pytest.raises(ValueError):
        sa.sage_attn_compute(out, ws, v=torch.empty(1, 2, 128, 64, dtype=torch.float16))
    with pytest.raises(ValueError):
        sa.sage_attn_dump_scores(out, ws, v=torch.empty(1, 1, 256, 64, dtype=torch.float16), bh=0, q_tile=0, k_tile=0)
    with pytest.raises(TypeError):
        sa.sage_attn_compute(out, ws, v=torch.empty(1, 2, 256, 64, dtype=torch.float16))


def test_noalloc_entry_point_validation():
    # sage_attn_fwd_noalloc: the same argument checks as sage_attn_fwd, and a problem whose
    # workspace exceeds the library's per-device scratch is refused before any HIP call
    f = lambda q=A16, out=A16, B=1, H=2, N=256, d=64, causal=0, scale=0.125, mode=0: \
        lib.sage_attn_fwd_noalloc(q, A16, A16, out, B, H, N, d, causal, scale, mode, None)
    assert f(q=None) == INVALID and f(out=A16 + 2) == INVALID
    assert f(d=96) == UNSUP and f(mode=9) == UNSUP and f(mode=6, N=(1 << 17) + 1) == UNSUP
    assert f(scale=0.0) == INVALID and f(causal=3) == INVALID
    big = sa.sage_attn_workspace_size(1, 64, 32768, 128, 0)
    assert big > sa.SAGE_NOALLOC_SCRATCH_BYTES
    assert f(B=1, H=64, N=32768, d=128) == WS
    assert "sage_attn_fwd_noalloc holds" in sa.sage_last_error()
    # the largest workloads it serves: prefill-sized INT8 and MXFP4 problems fit
    assert sa.sage_attn_workspace_size(4, 32, 4096, 128, 0) <= sa.SAGE_NOALLOC_SCRATCH_BYTES
    assert sa.sage_attn_workspace_size(4, 32, 8192, 128, 2) <= sa.SAGE_NOALLOC_SCRATCH_BYTES
    if not _gpu_visible():
        assert f() == NODEV


def test_backward_entry_points_validation():
    # the training forward and the backward pass: per-block INT8 modes only,
    # every argument checked before any HIP call
    ws = sa.sage_attn_bwd_workspace_size(1, 2, 256, 64, 0)
    assert ws > sa.sage_attn_workspace_size(1, 2, 256, 64, 0)
    assert sa.sage_attn_bwd_workspace_size(1, 2, 256, 64, 1 | sa.SAGE_FLAG_NO_SMOOTH) > 0
    for bad_mode in (2, 3, 4, 5, 6, 7):
        assert sa.sage_attn_bwd_workspace_size(1, 2, 256, 64, bad_mode) == 0
    assert sa.sage_attn_bwd_workspace_size(1, 2, 256, 96, 0) == 0
    LSE = ctypes.c_void_p(4096)
    fl = lambda q=A16, out=A16, lse=LSE, N=256, d=64, causal=0, scale=0.125, mode=0, w=A16, nb=1 << 30: \
        lib.sage_attn_fwd_lse(q, A16, A16, out, lse, 1, 2, N, d, causal, scale, mode, w, nb, None)
    assert fl(lse=None) == INVALID and fl(q=None) == INVALID and fl(out=A16 + 2) == INVALID
    assert fl(mode=2) == UNSUP and fl(mode=3) == UNSUP and fl(d=96) == UNSUP
    assert fl(scale=float("nan")) == INVALID and fl(causal=2) == INVALID
    assert fl(nb=16) == WS
    fb = lambda q=A16, dout=A16, lse=LSE, dq=A16, N=256, d=64, causal=0, scale=0.125, mode=0, w=A16, nb=1 << 30: \
        lib.sage_attn_bwd(q, A16, A16, A16, dout, lse, dq, A16, A16, 1, 2, N, d, causal, scale, mode, w, nb, None)
    assert fb(dout=None) == INVALID and fb(lse=None) == INVALID and fb(dq=A16 + 4) == INVALID
    assert fb(mode=6) == UNSUP and fb(mode=4) == UNSUP and fb(d=32) == UNSUP
    assert fb(scale=-1.0) == INVALID and fb(N=0) == INVALID
    assert fb(nb=ws - 1) == WS and "needed" in sa.sage_last_error()
    if not _gpu_visible():
        assert fl() == NODEV and fb() == NODEV


def test_trainable_attention_refuses_host_tensors():
    # sage_attention: the autograd Function's forward goes through the same
    # binding checks (host tensors are refused before any device call)
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 2, 64, 64, dtype=torch.float16, requires_grad=True)
    with pytest.raises(TypeError):
        sa.sage_attention(q, q.detach(), q.detach())
    with pytest.raises(ValueError):
        sa.sage_attention(torch.zeros(2, 64, 64, dtype=torch.float16), q, q)


def test_fused_q_flag_validation():
    # SAGE_FLAG_FUSED_Q goes with the per-block INT8 modes only, and the score
    # dump (which reads the workspace Q codes) refuses it
    F = sa.SAGE_FLAG_FUSED_Q
    fwd = lambda mode: lib.sage_attn_fwd(A16, A16, A16, A16, 1, 2, 256, 64, 0, 0.125, mode, A16, 1 << 30, None)
    for bad in (2, 3, 4, 5, 6, 7):
        assert fwd(bad | F) == UNSUP
    assert lib.sage_attn_prepare(A16, A16, A16, 1, 2, 256, 64, 3 | F, A16, 1 << 30, None) == UNSUP
    assert lib.sage_attn_compute(None, A16, A16, A16, 1, 2, 256, 64, 0, 0.125, 0 | F, A16, 1 << 30, None) == INVALID
    ws0 = sa.sage_attn_workspace_size(1, 2, 256, 64, 0)
    assert lib.sage_attn_dump_scores(A16, A16, 1, 2, 256, 64, 0.1, 0 | F, A16, ws0, 1, 0, 3, A16, None) == UNSUP
    if not _gpu_visible():
        assert fwd(0 | F) == NODEV and fwd(1 | F | sa.SAGE_FLAG_NO_SMOOTH) == NODEV
