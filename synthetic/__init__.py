"""Seeded synthetic inputs for the quantized-attention forward pass.

This module draws Q, K, V and nothing else: it holds none of the method's
arithmetic (no means, scales, rounding to codes or softmax). Both the CPU
oracle and the HIP path are fed from here, so the two see bit-identical fp16
tensors.

The workloads stand in for the real model layers that the SageAttention page
(atlas.scime.ai summary, "Key results" and "Experimental setup") evaluates on
(Llama2 prefill, CogVideoX-style video DiT, ...). Those weights and prompt sets
are not available, so every tensor is drawn from the distribution the
workload description names, from numpy's PCG64 generator:

  1. Q, K, V as float32 draws of shape [B, H, N, d], in that order:
     standard normal, or Student-t(nu) / sqrt(nu / (nu - 2)) (unit variance)
     for heavy-tailed workloads.
  2. A per-channel offset for K of shape [B, H, d], normal with the stated
     standard deviation, shared by every token of a (b, h) head and added to K.
  3. For the outlier workload: round(frac * H * d) of the H*d (head, channel)
     pairs, chosen without replacement and shared across the batch; the whole
     K channel (draw plus offset) is multiplied by the outlier factor.
  4. Offsets and outliers are applied in float32, then every tensor is cast to
     float16 with round-to-nearest-even.

For the backward pass, the gradient of the loss with respect to the attention
output (dO) stands in for what the layers above would send back: a standard
normal float32 draw of shape [B, H, N, d] from its own PCG64 stream (seed
derived from the workload's), cast to float16 the same way.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_custom", "make_grad"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    dist: str            # "normal" or "student_t"
    k_offset_std: float  # std of the per-channel K offset
    outlier_frac: float  # fraction of (head, channel) pairs of K scaled
    outlier_scale: float
    mode: str            # "int8_q128_k64", "int8_q64_k64" or "mxfp4"
    seed: int
    nu: float = 3.0      # Student-t degrees of freedom

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def attention_ops(self) -> float:
        """4*B*H*N^2*d, halved under a causal mask (the pages' TOPS convention)."""
        ops = 4.0 * self.B * self.H * self.N * self.N * self.d
        return ops / 2 if self.causal else ops


# Workload shapes and distributions. "tiny" is the small case the oracle runs
# in seconds; "prefill" an LLM prefill layer with outlier channels in K;
# "long_causal" a 32K-token causal layer; "video_dit" a video-DiT layer with a
# ragged token count and heavy-tailed activations; "mxfp4" the microscaled FP4
# path; "n16k" the 16K-token, d=128 shape used for the kernel throughput target.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 256, 64, False, "normal", 3.0, 0.0, 1.0, "int8_q64_k64", 0),
    "prefill": Workload("prefill", 4, 32, 4096, 128, False, "normal", 3.0, 0.01, 10.0, "int8_q128_k64", 1),
    "long_causal": Workload("long_causal", 1, 32, 32768, 128, True, "normal", 3.0, 0.0, 1.0, "int8_q128_k64", 2),
    "video_dit": Workload("video_dit", 2, 48, 17550, 64, False, "student_t", 2.0, 0.0, 1.0, "int8_q128_k64", 3),
    "mxfp4": Workload("mxfp4", 4, 32, 8192, 128, False, "normal", 3.0, 0.0, 1.0, "mxfp4", 4),
    "n16k": Workload("n16k", 1, 32, 16384, 128, False, "normal", 3.0, 0.0, 1.0, "int8_q128_k64", 5),
}


def _draw(rng: np.random.Generator, shape, dist: str, nu: float) -> np.ndarray:
    if dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if dist == "student_t":
        x = rng.standard_t(nu, size=shape)
        return (x / math.sqrt(nu / (nu - 2.0))).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def make_custom(B: int, H: int, N: int, d: int, *, seed: int, dist: str = "normal",
                k_offset_std: float = 3.0, outlier_frac: float = 0.0,
                outlier_scale: float = 10.0, nu: float = 3.0):
    """Draw fp16 (q, k, v), each [B, H, N, d], C-contiguous, by the recipe above."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, N, d)
    q = _draw(rng, shape, dist, nu)
    k = _draw(rng, shape, dist, nu)
    v = _draw(rng, shape, dist, nu)
    off = (rng.standard_normal((B, H, d), dtype=np.float32) * np.float32(k_offset_std)).astype(np.float32)
    k += off[:, :, None, :]
    n_out = int(round(outlier_frac * H * d))
    if n_out > 0:
        pick = rng.choice(H * d, size=n_out, replace=False)
        hs, cs = np.divmod(pick, d)
        for h, c in zip(hs.tolist(), cs.tolist()):
            k[:, h, :, c] *= np.float32(outlier_scale)
    return q.astype(np.float16), k.astype(np.float16), v.astype(np.float16)


def make_inputs(name: str, *, N: int | None = None, B: int | None = None, H: int | None = None,
                seed: int | None = None):
    """Inputs for a named workload; B, H, N may be overridden to draw a reduced copy."""
    w = WORKLOADS[name]
    return make_custom(B or w.B, H or w.H, N or w.N, w.d, seed=w.seed if seed is None else seed,
                       dist=w.dist, k_offset_std=w.k_offset_std, outlier_frac=w.outlier_frac,
                       outlier_scale=w.outlier_scale, nu=w.nu)


def make_grad(B: int, H: int, N: int, d: int, *, seed: int, scale: float = 1.0):
    """Draw the output gradient dO (fp16 [B, H, N, d], C-contiguous): standard
    normal times `scale`, from PCG64(seed + 1000) so it never repeats a Q/K/V stream."""
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    g = rng.standard_normal((B, H, N, d), dtype=np.float32) * np.float32(scale)
    return g.astype(np.float16)
