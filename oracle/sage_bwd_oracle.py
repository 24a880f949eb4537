"""CPU oracle for the 8-bit attention backward pass.

TEST INFRASTRUCTURE, like sage_oracle.py: only tests/, __graft_entry__.smoke()
and bench.py's cpu_baseline leg may import it; the HIP library never does, and
the two share no code, table or constant.

What the pages fix. "SageAttention3: Microscaling FP4 Attention for Inference
and An Exploration of 8-Bit Training" (abstract, mlsanity.com and the
Transistor oEmbed page) reports an accurate and efficient 8-bit attention for
the forward and the backward pass of training; the scifaro.com page of
related papers describes that trainable attention as INT8 ("SageBwd"). The
SageAttention page's "Experimental setup" says the method builds on
FlashAttention-2, whose backward pass recomputes the scores from Q and K and
the softmax probabilities from the forward's saved row log-sum-exp. Nothing
else is on the pages: no granularity, no choice of products, no precision of
the gradients. The readings below fill that in.

  Rb1 structure (FlashAttention-2's backward): with S the forward's scaled
      scores and L its row log-sum-exp, P = exp(S - L); dV = P^T dO;
      dP = dO V^T; D_i = sum_c dO_ic O_ic with O the forward's output;
      dS = P o (dP - D); dQ = sm_scale dS K_s; dK = sm_scale dS^T Q.
      K_s is the mean-smoothed K of the forward: each row of dS sums to zero
      (sum_j P_ij dP_ij = D_i), so dS K_s = dS K, and the gradient that flows
      back through the mean (minus the token mean of dK) is zero for the same
      reason; both are exact identities of the unquantized pass.
  Rb2 8-bit means INT8 codes with int32 accumulation in every one of the five
      products, each operand with scales constant along the contraction, all
      by the rules R3, R4 of sage_oracle (a = max|x| over the block, s =
      fp32(a / 127), code = rint_half_even(x / s); a = 0 gives zero codes),
      with the two granularities the SageAttention page's "Approach" names,
      per block and per token:
        S     the forward's codes: Q per block of 128 (or 64) tokens, K_s per
              block of 64 tokens;
        dP    dO per block of 64 tokens x all channels; V per token (one scale
              per key: heavy-tailed V keeps its accuracy, and a per-key scale
              stays constant along dP's contraction over channels);
        dV    P and dS (below) per block of 32 queries x 32 keys (aligned
              tiles of the N x N matrices); dO with the codes of dP;
        dQ,dK dS per 32 x 32 block; K_s and Q with the codes of S.
      P = exp(S - L) is at most 1 but mostly far below it (it is normalized),
      so a fixed scale 1/127 (R14's rule for the forward's unnormalized P)
      would round most weights to zero; the block maximum sets its scale
      instead. Partial products over one 32-block of the contraction are exact
      int32 sums; each is scaled and summed over the blocks.
  Rb3 code decisions: the oracle takes them on float64 values; an
      implementation taking them on float32 values may round a code that sits
      within a few float32 ulps of a rounding boundary the other way. The
      emulation can report, per code, whether it is such a candidate, and the
      first-order effect of flipping every candidate (an allowance for tests).
  Rb4 D_i is the dot product of the fp16 dO and O rows (exact products; the
      oracle sums them in float64).
  Rb5 L_i = m_i + ln(l_i), the final running max and row sum of the forward's
      online softmax (R6: l sums the fp16-rounded P), in natural-log units of
      the scaled scores.
  Rb6 gradients are float32 [B, H, N, d] (the oracle returns float64).
  Rb7 causal masking as R7: masked P is exactly 0.
"""
from __future__ import annotations

import numpy as np

from .sage_oracle import (
    _causal_mask,
    as_f64,
    int8_attention,
    int8_quant_blocks,
    int8_quant_v_channels,
    quant_qk_int8,
)

DS_BLOCK = 32      # dS quantization block: 32 queries x 32 keys (Rb2)
BWD_BLK = 64       # token blocks of dO and V for dP (Rb2)


# ---------------------------------------------------------------------------
# Exact backward in float64: the reference for the method's own accuracy.
# ---------------------------------------------------------------------------

def exact_attention_backward(q, k, v, do, *, causal: bool, sm_scale: float):
    """dQ, dK, dV of O = softmax(sm_scale Q K^T) V for the loss sum(O o dO), float64.

    The closed-form gradients of softmax attention written out per (b, h) with
    full N x N matrices (small N only): P the row softmax, dV = P^T dO,
    dP = dO V^T, D = rowsum(dO o O), dS = P o (dP - D), dQ = sm_scale dS K,
    dK = sm_scale dS^T Q. Returns a dict of float64 [B, H, N, d] arrays plus
    "o" (the output) and "lse" (the row log-sum-exp, [B, H, N]).
    """
    B, H, N, d = q.shape
    keys = np.arange(N)
    res = {n: np.empty((B, H, N, d)) for n in ("dq", "dk", "dv", "o")}
    res["lse"] = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            Q, K, V, G = as_f64(q[b, h]), as_f64(k[b, h]), as_f64(v[b, h]), as_f64(do[b, h])
            S = sm_scale * (Q @ K.T)
            if causal:
                S[_causal_mask(keys, keys)] = -np.inf
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            l = E.sum(axis=1, keepdims=True)
            P = E / l
            O = P @ V
            dV = P.T @ G
            dP = G @ V.T
            D = (G * O).sum(axis=1, keepdims=True)
            dS = P * (dP - D)
            res["dq"][b, h] = sm_scale * (dS @ K)
            res["dk"][b, h] = sm_scale * (dS.T @ Q)
            res["dv"][b, h] = dV
            res["o"][b, h] = O
            res["lse"][b, h] = (m + np.log(l))[:, 0]
    return res


# ---------------------------------------------------------------------------
# INT8 emulation (Rb1-Rb7).
# ---------------------------------------------------------------------------

def int8_forward_for_training(q16, k16, v16, *, causal: bool, sm_scale: float, blk_q: int = 128,
                              blk_k: int = 64, smooth: bool = True):
    """The forward pass a training step saves: the INT8 forward's output (float64
    and its fp16 copy) and the row log-sum-exp (Rb5)."""
    B, H, N, d = q16.shape
    lse = np.empty((B, H, N))
    o = int8_attention(q16, k16, v16, causal=causal, sm_scale=sm_scale, blk_q=blk_q, blk_k=blk_k,
                       smooth=smooth, lse=lse)
    return dict(o=o, o16=o.astype(np.float16), lse=lse)


def _near_half(x: np.ndarray, band: np.ndarray) -> np.ndarray:
    """True where |x| is within `band` of a rounding boundary k + 1/2."""
    f = np.abs(x) - np.floor(np.abs(x))
    return np.abs(f - 0.5) <= band


def _block_quant(X: np.ndarray):
    """Per-block INT8 codes of an [N, N] matrix in DS_BLOCK x DS_BLOCK tiles (Rb2).

    Returns (codes as float64, scale of each element's tile [N, N], the
    quotient X / s the code was rounded from, tile maxima [nb, nb], tile scales
    [nb, nb])."""
    N = X.shape[0]
    nb = -(-N // DS_BLOCK)
    pad = nb * DS_BLOCK - N
    blocks = np.pad(X, ((0, pad), (0, pad))).reshape(nb, DS_BLOCK, nb, DS_BLOCK)
    amax = np.abs(blocks).max(axis=(1, 3))
    s_blk = (amax.astype(np.float32) / np.float32(127.0)).astype(np.float32).astype(np.float64)
    s_full = np.repeat(np.repeat(s_blk, DS_BLOCK, axis=0), DS_BLOCK, axis=1)[:N, :N]
    xq = X / np.where(s_full > 0, s_full, 1.0)
    codes = np.where(s_full > 0, np.clip(np.rint(xq), -127, 127), 0.0)
    return codes, s_full, xq, amax


def _flip_candidates(X: np.ndarray, err: np.ndarray, xq: np.ndarray, s_full: np.ndarray, amax: np.ndarray):
    """Rb3 for a block-quantized matrix X whose float32 value may be off by up
    to `err` per element: the codes that could round the other way (including
    through the tile scale, which carries its largest element's error), and
    the relative uncertainty of each element's tile scale."""
    N = X.shape[0]
    nb = amax.shape[0]
    pad = nb * DS_BLOCK - N
    t = lambda Y: np.pad(Y, ((0, pad), (0, pad))).reshape(nb, DS_BLOCK, nb, DS_BLOCK).transpose(0, 2, 1, 3).reshape(nb, nb, -1)
    arg = t(np.abs(X)).argmax(axis=2)
    err_m = np.take_along_axis(t(err), arg[..., None], axis=2)[..., 0]
    rho = np.where(amax > 0, err_m / np.where(amax > 0, amax, 1.0), 0.0) + 2.0 ** -22
    rho_full = np.repeat(np.repeat(rho, DS_BLOCK, axis=0), DS_BLOCK, axis=1)[:N, :N]
    safe = np.where(s_full > 0, s_full, 1.0)
    band = 4.0 * (np.abs(xq) * (rho_full + 2.0 ** -22) + err / safe)
    return (s_full > 0) & _near_half(xq, band), rho_full


def int8_attention_backward(q16, k16, v16, do16, o16, lse, *, causal: bool, sm_scale: float,
                            blk_q: int = 128, blk_k: int = 64, smooth: bool = True,
                            with_allowance: bool = False, quant=None):
    """Emulated INT8 attention backward (Rb1-Rb7), float64 gradients.

    q16, k16, v16, do16, o16: fp16 [B, H, N, d]; lse: float [B, H, N] (the
    forward's row log-sum-exp, natural log). Returns dict(dq, dk, dv) of float64
    [B, H, N, d]; with_allowance adds, per gradient, "<g>_mag" (the sum of the
    absolute values of the terms each element adds up, the scale of any
    rounding in its accumulation) and "<g>_allow" (the first-order change if
    every code that float32 arithmetic could round the other way did so, Rb3),
    plus counts of such codes ("p_flips", "ds_flips").
    """
    B, H, N, d = q16.shape
    qd = quant if quant is not None else quant_qk_int8(q16, k16, blk_q=blk_q, blk_k=blk_k, smooth=smooth)
    vc, vs = int8_quant_blocks(np.asarray(v16).astype(np.float32), 1)
    gc, gs = int8_quant_blocks(np.asarray(do16).astype(np.float32), BWD_BLK)
    keys = np.arange(N)
    out = {n: np.empty((B, H, N, d)) for n in ("dq", "dk", "dv")}
    if with_allowance:
        for n in ("dq", "dk", "dv"):
            out[n + "_mag"] = np.empty((B, H, N, d))
            out[n + "_allow"] = np.empty((B, H, N, d))
        out["p_flips"] = 0
        out["ds_flips"] = 0
    log2e = 1.0 / np.log(2.0)
    for b in range(B):
        for h in range(H):
            # scores exactly as the forward dequantizes them (R5)
            cq = qd["q_codes"][b, h].astype(np.float64)
            ck = qd["k_codes"][b, h].astype(np.float64)
            sq = qd["q_scales"][b, h][keys // blk_q].astype(np.float64)
            sk = qd["k_scales"][b, h][keys // blk_k].astype(np.float64)
            S = (cq @ ck.T) * sq[:, None] * sk[None, :] * sm_scale
            L = np.asarray(lse[b, h], dtype=np.float64)
            mask = _causal_mask(keys, keys) if causal else np.zeros((N, N), bool)
            with np.errstate(over="ignore"):
                P = np.where(mask, 0.0, np.exp(np.where(mask, 0.0, S) - L[:, None]))
            gdq = gc[b, h].astype(np.float64) * gs[b, h][keys // BWD_BLK].astype(np.float64)[:, None]
            vdq = vc[b, h].astype(np.float64) * vs[b, h].astype(np.float64)[:, None]
            # dV = P^T dO with P per 32 x 32 block
            Pc, sP, xP, aP = _block_quant(P)
            Pq = Pc * sP
            out["dv"][b, h] = Pq.T @ gdq
            # dP = dO V^T (exact integer dot products, then the two scales), D (Rb4)
            dP = gdq @ vdq.T
            D = (as_f64(do16[b, h]) * as_f64(o16[b, h])).sum(axis=1)
            dS = P * (dP - D[:, None])
            dSc, sS, xS, aS = _block_quant(dS)
            dSq = dSc * sS
            kdq = ck * sk[:, None]                               # K_s codes x their scales
            qdq = cq * sq[:, None]
            out["dq"][b, h] = sm_scale * (dSq @ kdq)
            out["dk"][b, h] = sm_scale * (dSq.T @ qdq)
            if with_allowance:
                # Rb3: how far float32 arithmetic can move the values the codes
                # are decided on. P: the exponent's argument carries ~|S| + |L|
                # ulps; dS: P's error plus the rounding of dP and D before their
                # difference.
                arg = np.abs(np.where(mask, 0.0, S)) + np.abs(L)[:, None]
                errP = P * 2.0 ** -22 * (2.0 + log2e * arg)
                errS = (np.abs(dS) * (errP / np.maximum(P, 1e-300) + 2.0 ** -21)
                        + P * (np.abs(dP) + np.abs(D)[:, None]) * 2.0 ** -22)
                flipP, rhoP = _flip_candidates(P, errP, xP, sP, aP)
                flipS, rhoS = _flip_candidates(dS, errS, xS, sS, aS)
                flipP &= ~mask
                flipS &= ~mask
                out["p_flips"] += int(flipP.sum())
                out["ds_flips"] += int(flipS.sum())
                absK, absQ, absG = np.abs(kdq), np.abs(qdq), np.abs(gdq)
                # a flipped code moves by one scale unit; a tile's scale by rho
                movP = flipP * sP + rhoP * np.abs(Pq)
                movS = flipS * sS + rhoS * np.abs(dSq)
                out["dv_mag"][b, h] = np.abs(Pq).T @ absG
                out["dv_allow"][b, h] = movP.T @ absG
                out["dq_mag"][b, h] = sm_scale * (np.abs(dSq) @ absK)
                out["dq_allow"][b, h] = sm_scale * (movS @ absK)
                out["dk_mag"][b, h] = sm_scale * (np.abs(dSq).T @ absQ)
                out["dk_allow"][b, h] = sm_scale * (movS.T @ absQ)
    return out
