"""Python binding of libsage_attn.so, the gfx950 quantized-attention library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/sage_attn.h). PyTorch supplies device memory
(tensors, the workspace) and the current HIP stream. If the library is not
built, importing this package raises ImportError; there is no fallback path.

Functions carry the C names:
  sage_attn_fwd(q, k, v, ...)          -> out
  sage_attn_fwd_noalloc(q, k, v, out, ...)  (no workspace: the library's per-device scratch)
  sage_attn_prepare / sage_attn_compute  (the two phases of sage_attn_fwd)
  sage_attn_workspace_size(B, H, N, d, mode)
  sage_attn_fwd_lse(q, k, v, ...)      -> (out, lse)   (the forward a training step saves)
  sage_attn_bwd(q, k, v, out, dout, lse, ...) -> (dq, dk, dv)   (INT8 backward pass)
  sage_attn_bwd_workspace_size(B, H, N, d, mode)
  sage_attention(q, k, v, ...)         -> out, differentiable: a torch.autograd.Function whose
                                          forward is sage_attn_fwd_lse and backward sage_attn_bwd
  sage_quant_qk(q, k, blk_q, blk_k, flags)  -> dict of codes/scales/mean
  sage_quant_mxfp4(q, k, v, flags)         -> dict of packed codes/exponents
  sage_quant_v_int8(v)                     -> dict of V^T codes and channel scales
  sage_clock_probe / measure_clock_mhz     (shader clock, for throughput reports)
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "SAGE_MODE_INT8_Q128_K64", "SAGE_MODE_INT8_Q64_K64", "SAGE_MODE_MXFP4", "SAGE_MODE_INT8_PER_TOKEN",
    "SAGE_MODE_FP16", "SAGE_MODE_MXFP4_FP8PV", "SAGE_MODE_INT8_PV", "SAGE_MODE_INT8_PV_PER_TOKEN",
    "SAGE_FLAG_NO_SMOOTH", "SAGE_FLAG_FP8_V", "SAGE_FLAG_FUSED_Q", "SageError", "LIB_PATH", "lib",
    "sage_attn_fwd", "sage_attn_fwd_noalloc", "SAGE_NOALLOC_SCRATCH_BYTES", "sage_attn_prepare", "sage_attn_compute", "sage_attn_workspace_size",
    "sage_quant_workspace_size", "sage_quant_qk", "sage_quant_mxfp4", "sage_quant_v_int8", "sage_attn_dump_scores", "sage_status_string", "sage_last_error",
    "sage_clock_probe", "sage_wall_clock_khz", "measure_clock_mhz",
    "sage_attn_fwd_lse", "sage_attn_bwd", "sage_attn_bwd_workspace_size", "make_bwd_workspace",
    "sage_attention",
    "EXPORTED_SYMBOLS",
]

SAGE_MODE_INT8_Q128_K64 = 0
SAGE_MODE_INT8_Q64_K64 = 1
SAGE_MODE_MXFP4 = 2
SAGE_MODE_INT8_PER_TOKEN = 3
SAGE_MODE_FP16 = 4
SAGE_MODE_MXFP4_FP8PV = 5
SAGE_MODE_INT8_PV = 6
SAGE_MODE_INT8_PV_PER_TOKEN = 7
SAGE_FLAG_NO_SMOOTH = 0x100
SAGE_FLAG_FP8_V = 0x200
SAGE_FLAG_FUSED_Q = 0x400
SAGE_NOALLOC_SCRATCH_BYTES = 256 << 20

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsage_attn.so")

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "sage_status_string": (ctypes.c_char_p, [_i]),
    "sage_last_error": (ctypes.c_char_p, []),
    "sage_attn_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "sage_quant_workspace_size": (_sz, [_i, _i, _i, _i]),
    "sage_attn_fwd": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]),
    "sage_attn_fwd_noalloc": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp]),
    "sage_attn_prepare": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "sage_attn_compute": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]),
    "sage_quant_qk": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "sage_quant_mxfp4": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "sage_quant_v_int8": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "sage_attn_dump_scores": (_i, [_vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _sz, _i, _i, _i, _vp, _vp]),
    "sage_clock_probe": (_i, [ctypes.c_longlong, _vp, _vp]),
    "sage_attn_bwd_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "sage_attn_fwd_lse": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]),
    "sage_attn_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]),
    "sage_wall_clock_khz": (_i, [ctypes.POINTER(_i)]),
}
EXPORTED_SYMBOLS = tuple(_SIGS)


def _load():
    # PyTorch ships its own HIP runtime (libamdhip64.so, SONAME libamdhip64.so.7).
    # Loading torch first makes the library bind to that same runtime by SONAME,
    # so torch's streams and allocations are valid handles for it; loading the
    # library first would bring in a second runtime from /opt/rocm.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python bit_quantized_attention_mean_amd/build.py` (or __graft_entry__.build())")
    so = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(so, name)
        fn.restype = res
        fn.argtypes = args
    return so


lib = _load()


class SageError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {sage_status_string(status)}: {sage_last_error()}")


def sage_status_string(status: int) -> str:
    return lib.sage_status_string(status).decode()


def sage_last_error() -> str:
    return lib.sage_last_error().decode()


def _check(rc: int, where: str):
    if rc != 0:
        raise SageError(rc, where)


def sage_attn_workspace_size(B: int, H: int, N: int, d: int, mode: int = 0) -> int:
    return int(lib.sage_attn_workspace_size(B, H, N, d, mode))


def sage_quant_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(lib.sage_quant_workspace_size(B, H, N, d))


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_ptr(t, name, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _shape4(q):
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    return tuple(int(x) for x in q.shape)


def make_workspace(B, H, N, d, mode=0, device=None):
    """A device workspace tensor (uint8) large enough for sage_attn_fwd."""
    torch = _torch()
    n = sage_attn_workspace_size(B, H, N, d, mode)
    if n == 0:
        raise ValueError("invalid problem size or mode")
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def sage_attn_fwd(q, k, v, out=None, *, causal=False, sm_scale=None, mode=SAGE_MODE_INT8_Q128_K64,
                  workspace=None, stream=None):
    """out[B,H,N,d] fp16 = quantized attention of fp16 q, k, v [B,H,N,d]."""
    torch = _torch()
    B, H, N, d = _shape4(q)
    if tuple(k.shape) != (B, H, N, d) or tuple(v.shape) != (B, H, N, d):
        raise ValueError("q, k, v must have the same shape")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = make_workspace(B, H, N, d, mode, q.device)
    rc = lib.sage_attn_fwd(_dev_ptr(q, "q", torch.float16), _dev_ptr(k, "k", torch.float16),
                           _dev_ptr(v, "v", torch.float16), _dev_ptr(out, "out", torch.float16),
                           B, H, N, d, int(bool(causal)), float(sm_scale), int(mode),
                           _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                           _stream(stream))
    _check(rc, "sage_attn_fwd")
    return out


def sage_attn_bwd_workspace_size(B: int, H: int, N: int, d: int, mode: int = 0) -> int:
    return int(lib.sage_attn_bwd_workspace_size(B, H, N, d, mode))


def make_bwd_workspace(B, H, N, d, mode=0, device=None):
    """A device workspace tensor (uint8) for sage_attn_bwd (it also serves sage_attn_fwd_lse)."""
    torch = _torch()
    n = sage_attn_bwd_workspace_size(B, H, N, d, mode)
    if n == 0:
        raise ValueError("invalid problem size or mode for the backward pass")
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def sage_attn_fwd_lse(q, k, v, out=None, lse=None, *, causal=False, sm_scale=None,
                      mode=SAGE_MODE_INT8_Q128_K64, workspace=None, stream=None):
    """(out fp16 [B,H,N,d], lse fp32 [B,H,N]): the forward pass and its row log-sum-exp."""
    torch = _torch()
    B, H, N, d = _shape4(q)
    if tuple(k.shape) != (B, H, N, d) or tuple(v.shape) != (B, H, N, d):
        raise ValueError("q, k, v must have the same shape")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = make_workspace(B, H, N, d, mode, q.device)
    rc = lib.sage_attn_fwd_lse(_dev_ptr(q, "q", torch.float16), _dev_ptr(k, "k", torch.float16),
                               _dev_ptr(v, "v", torch.float16), _dev_ptr(out, "out", torch.float16),
                               _dev_ptr(lse, "lse", torch.float32), B, H, N, d, int(bool(causal)),
                               float(sm_scale), int(mode), _dev_ptr(workspace, "workspace"),
                               workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "sage_attn_fwd_lse")
    return out, lse


def sage_attn_bwd(q, k, v, out, dout, lse, dq=None, dk=None, dv=None, *, causal=False, sm_scale=None,
                  mode=SAGE_MODE_INT8_Q128_K64, workspace=None, stream=None):
    """(dq, dk, dv) fp32 [B,H,N,d]: gradients of sum(out * dout) by the INT8 backward pass."""
    torch = _torch()
    B, H, N, d = _shape4(q)
    for t, name in ((k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        if tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"{name} must have the shape of q")
    if tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be [B, H, N]")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    dq = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device) if dq is None else dq
    dk = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device) if dk is None else dk
    dv = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device) if dv is None else dv
    if workspace is None:
        workspace = make_bwd_workspace(B, H, N, d, mode, q.device)
    rc = lib.sage_attn_bwd(_dev_ptr(q, "q", torch.float16), _dev_ptr(k, "k", torch.float16),
                           _dev_ptr(v, "v", torch.float16), _dev_ptr(out, "out", torch.float16),
                           _dev_ptr(dout, "dout", torch.float16), _dev_ptr(lse, "lse", torch.float32),
                           _dev_ptr(dq, "dq", torch.float32), _dev_ptr(dk, "dk", torch.float32),
                           _dev_ptr(dv, "dv", torch.float32), B, H, N, d, int(bool(causal)), float(sm_scale),
                           int(mode), _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                           _stream(stream))
    _check(rc, "sage_attn_bwd")
    return dq, dk, dv


_AUTOGRAD_FN = None


def _attention_function():
    """The autograd Function behind sage_attention, made on first use (torch is
    imported lazily)."""
    global _AUTOGRAD_FN
    if _AUTOGRAD_FN is None:
        torch = _torch()

        class SageAttentionFunction(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, causal, sm_scale, mode):
                out, lse = sage_attn_fwd_lse(q, k, v, causal=causal, sm_scale=sm_scale, mode=mode)
                ctx.save_for_backward(q, k, v, out, lse)
                ctx.causal, ctx.sm_scale, ctx.mode = causal, sm_scale, mode
                return out

            @staticmethod
            def backward(ctx, dout):
                q, k, v, out, lse = ctx.saved_tensors
                dq, dk, dv = sage_attn_bwd(q, k, v, out, dout.contiguous(), lse, causal=ctx.causal,
                                           sm_scale=ctx.sm_scale, mode=ctx.mode)
                # float32 gradients; autograd hands them to the fp16 inputs in their dtype
                return dq, dk, dv, None, None, None

        _AUTOGRAD_FN = SageAttentionFunction
    return _AUTOGRAD_FN


def sage_attention(q, k, v, *, causal=False, sm_scale=None, mode=SAGE_MODE_INT8_Q128_K64):
    """Trainable quantized attention: out = sage_attn_fwd_lse(q, k, v)[0], whose gradient
    with respect to q, k, v is the INT8 backward pass (sage_attn_bwd) on the saved
    (out, lse). q, k, v fp16 [B, H, N, d] on the GPU; modes 0 and 1, with or without
    SAGE_FLAG_NO_SMOOTH."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(_shape4(q)[3])
    return _attention_function().apply(q, k, v, bool(causal), float(sm_scale), int(mode))


def sage_attn_fwd_noalloc(q, k, v, out, *, causal=False, sm_scale=None, mode=SAGE_MODE_INT8_Q128_K64, stream=None):
    """sage_attn_fwd with the library's own per-device scratch as workspace (the C entry
    point allocates nothing; `out` must be given). Calls on one device share that scratch."""
    torch = _torch()
    B, H, N, d = _shape4(q)
    for t, name in ((k, "k"), (v, "v"), (out, "out")):
        if tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"q and {name} must have the same shape")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    rc = lib.sage_attn_fwd_noalloc(_dev_ptr(q, "q", torch.float16), _dev_ptr(k, "k", torch.float16),
                                   _dev_ptr(v, "v", torch.float16), _dev_ptr(out, "out", torch.float16),
                                   B, H, N, d, int(bool(causal)), float(sm_scale), int(mode), _stream(stream))
    _check(rc, "sage_attn_fwd_noalloc")
    return out


def sage_attn_prepare(q, k, v, workspace, *, mode=SAGE_MODE_INT8_Q128_K64, stream=None):
    torch = _torch()
    B, H, N, d = _shape4(q)
    rc = lib.sage_attn_prepare(_dev_ptr(q, "q", torch.float16), _dev_ptr(k, "k", torch.float16),
                               _dev_ptr(v, "v", torch.float16), B, H, N, d, int(mode),
                               _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                               _stream(stream))
    _check(rc, "sage_attn_prepare")


def sage_attn_compute(out, workspace, *, causal=False, sm_scale=None, mode=SAGE_MODE_INT8_Q128_K64, q=None, k=None,
                      v=None, stream=None):
    """Attention from a prepared workspace. q, k (the tensors given to prepare) are needed by SAGE_MODE_FP16,
    and q also with SAGE_FLAG_FUSED_Q; v (the V given to prepare) by every mode with an fp16 P.V (all but the
    MXFP4 and INT8 P.V modes)."""
    torch = _torch()
    B, H, N, d = _shape4(out)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        if t is not None and tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"{name} and out must have the same shape")
    qp = None if q is None else _dev_ptr(q, "q", torch.float16)
    kp = None if k is None else _dev_ptr(k, "k", torch.float16)
    vp = None if v is None else _dev_ptr(v, "v", torch.float16)
    rc = lib.sage_attn_compute(qp, kp, vp, _dev_ptr(out, "out", torch.float16), B, H, N, d, int(bool(causal)),
                               float(sm_scale), int(mode), _dev_ptr(workspace, "workspace"),
                               workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "sage_attn_compute")
    return out


def sage_quant_qk(q, k, *, blk_q=128, blk_k=64, flags=0, stream=None):
    """INT8 codes and scales of Q and the mean-smoothed K (plus the K mean)."""
    torch = _torch()
    B, H, N, d = _shape4(q)
    dev = q.device
    res = {
        "q_codes": torch.empty((B, H, N, d), dtype=torch.int8, device=dev),
        "k_codes": torch.empty((B, H, N, d), dtype=torch.int8, device=dev),
        "q_scales": torch.empty((B, H, -(-N // blk_q)), dtype=torch.float32, device=dev),
        "k_scales": torch.empty((B, H, -(-N // blk_k)), dtype=torch.float32, device=dev),
        "k_mean": torch.empty((B, H, d), dtype=torch.float32, device=dev),
    }
    ws = torch.empty(max(1, sage_quant_workspace_size(B, H, N, d)), dtype=torch.uint8, device=dev)
    rc = lib.sage_quant_qk(_dev_ptr(q, "q", torch.float16), _dev_ptr(k, "k", torch.float16), B, H, N, d,
                           int(blk_q), int(blk_k), int(flags),
                           _dev_ptr(res["q_codes"], "q_codes"), _dev_ptr(res["q_scales"], "q_scales"),
                           _dev_ptr(res["k_codes"], "k_codes"), _dev_ptr(res["k_scales"], "k_scales"),
                           _dev_ptr(res["k_mean"], "k_mean"), _dev_ptr(ws, "workspace"), ws.numel(),
                           _stream(stream))
    _check(rc, "sage_quant_qk")
    return res


def sage_quant_mxfp4(q, k, v, *, flags=0, stream=None):
    """MXFP4 codes (packed, low nibble first) and E8M0 exponents of Q, K_s and V^T."""
    torch = _torch()
    B, H, N, d = _shape4(q)
    dev = q.device
    Nv = -(-N // 32) * 32
    u8 = torch.uint8
    res = {
        "q_fp4": torch.empty((B, H, N, d // 2), dtype=u8, device=dev),
        "q_e8m0": torch.empty((B, H, N, d // 32), dtype=u8, device=dev),
        "k_fp4": torch.empty((B, H, N, d // 2), dtype=u8, device=dev),
        "k_e8m0": torch.empty((B, H, N, d // 32), dtype=u8, device=dev),
        "vt_fp4": torch.empty((B, H, d, Nv if flags & SAGE_FLAG_FP8_V else Nv // 2), dtype=u8, device=dev),
        "vt_e8m0": torch.empty((B, H, d, Nv // 32), dtype=u8, device=dev),
        "k_mean": torch.empty((B, H, d), dtype=torch.float32, device=dev),
    }
    ws = torch.empty(max(1, sage_quant_workspace_size(B, H, N, d)), dtype=u8, device=dev)
    rc = lib.sage_quant_mxfp4(_dev_ptr(q, "q", torch.float16), _dev_ptr(k, "k", torch.float16),
                              _dev_ptr(v, "v", torch.float16), B, H, N, d, int(flags),
                              *(_dev_ptr(res[n], n) for n in ("q_fp4", "q_e8m0", "k_fp4", "k_e8m0", "vt_fp4", "vt_e8m0")),
                              _dev_ptr(res["k_mean"], "k_mean"), _dev_ptr(ws, "workspace"), ws.numel(),
                              _stream(stream))
    _check(rc, "sage_quant_mxfp4")
    return res


def sage_quant_v_int8(v, *, stream=None):
    """Per-channel INT8 codes of V, transposed ([B, H, d, Nv], Nv = N rounded up to 16), and the scales."""
    torch = _torch()
    B, H, N, d = _shape4(v)
    dev = v.device
    Nv = -(-N // 16) * 16
    res = {
        "vt_codes": torch.empty((B, H, d, Nv), dtype=torch.int8, device=dev),
        "v_scales": torch.empty((B, H, d), dtype=torch.float32, device=dev),
    }
    ws = torch.empty(max(1, sage_quant_workspace_size(B, H, N, d)), dtype=torch.uint8, device=dev)
    rc = lib.sage_quant_v_int8(_dev_ptr(v, "v", torch.float16), B, H, N, d, _dev_ptr(res["vt_codes"], "vt_codes"),
                               _dev_ptr(res["v_scales"], "v_scales"), _dev_ptr(ws, "workspace"), ws.numel(),
                               _stream(stream))
    _check(rc, "sage_quant_v_int8")
    return res


def sage_attn_dump_scores(out, workspace, *, v, bh, q_tile, k_tile, sm_scale=None, mode=SAGE_MODE_INT8_Q128_K64,
                          stream=None):
    """Test hook: runs the INT8 attention kernel (non-causal) on a prepared workspace and V and returns the
    int32 scores its matrix op produced for key tile k_tile and query tile q_tile of head bh ([256, 64])."""
    torch = _torch()
    B, H, N, d = _shape4(out)
    if tuple(v.shape) != (B, H, N, d):
        raise ValueError("v and out must have the same shape")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    s_out = torch.zeros((256, 64), dtype=torch.int32, device=out.device)
    rc = lib.sage_attn_dump_scores(_dev_ptr(v, "v", torch.float16), _dev_ptr(out, "out", torch.float16), B, H, N, d, float(sm_scale), int(mode),
                                   _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                   int(bh), int(q_tile), int(k_tile), _dev_ptr(s_out, "s_out"), _stream(stream))
    _check(rc, "sage_attn_dump_scores")
    return s_out



def sage_wall_clock_khz() -> int:
    khz = ctypes.c_int(0)
    _check(lib.sage_wall_clock_khz(ctypes.byref(khz)), "sage_wall_clock_khz")
    return int(khz.value)


def sage_clock_probe(cycles: int, out, stream=None):
    """Enqueues the clock probe; `out` is an int64 CUDA tensor of at least 2 elements."""
    torch = _torch()
    if out.numel() < 2:
        raise ValueError("out needs 2 int64 elements")
    _check(lib.sage_clock_probe(int(cycles), _dev_ptr(out, "out", torch.int64), _stream(stream)), "sage_clock_probe")
    return out


def measure_clock_mhz(cycles: int = 12_000_000, stream=None, during=None) -> float:
    """Shader clock in MHz over `cycles` clocks of one probe wave.

    With `during` (a callable that enqueues work on the current stream) the
    probe runs on `stream` (a second stream) while that work runs, and the
    result is the clock under that load; the call synchronizes the device.
    """
    torch = _torch()
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    if during is not None:
        if stream is None:
            stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        during()          # the load is enqueued first, so it occupies the GPU when the probe starts
        sage_clock_probe(cycles, out, stream)
        during()
    else:
        sage_clock_probe(cycles, out, stream)
    torch.cuda.synchronize()
    c, w = (int(x) for x in out.cpu())
    if c <= 0 or w <= 0:
        raise RuntimeError(f"clock probe returned {c} cycles over {w} ticks")
    return c / w * sage_wall_clock_khz() / 1000.0
