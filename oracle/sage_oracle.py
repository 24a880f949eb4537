"""CPU oracle for the SageAttention-style quantized attention forward pass.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py may import this module. The product path (the HIP library and
its Python binding) never imports, calls or links it, and this module shares no
code, table or constant with the HIP sources.

Plain, slow and meant to be read against the pages. Everything that is not a
quantization rounding runs in float64; every rounding the method performs
(fp32 subtraction, fp32 division, round-to-nearest-even to INT8 / FP16 / E2M1)
is reproduced exactly with numpy's IEEE float32/float16 arithmetic.

Citations name the page and its section:
  [SA-Approach]   "SageAttention: Accurate 8-Bit Attention for Plug-and-play
                  Inference Acceleration" (atlas.scime.ai AI-written summary),
                  section "Approach": subtract the mean of K across tokens,
                  which leaves softmax attention unchanged; INT8 Q and K with
                  per-token or per-block scales; P and V kept in FP16 for P.V;
                  cosine similarity above 99.8% as the selection bar.
  [SA-Summary]    same page, the one-paragraph summary at the top: INT8 QK^T
                  with K mean-smoothing, FP16 PV.
  [SA-Setup]      same page, "Experimental setup": builds on FlashAttention-2,
                  dynamic quantization and online softmax; metrics cosine
                  similarity, relative L1, RMSE.
  [SA-Effects]    same page, "Measured effects reported in the paper" table
                  (smoothing ablations, FP16 vs FP32 accumulator, INT8 P,V).
  [SA3-Abstract]  "SageAttention3: Microscaling FP4 Attention for Inference and
                  An Exploration of 8-Bit Training" (mlsanity.com and the
                  Transistor oEmbed page), abstract: microscaling FP4 attention
                  on FP4 matrix units. Its reference list names "Microscaling
                  Data Formats for Deep Learning" (the MX format) and "Online
                  normalizer calculation for softmax".

Readings where the pages are silent:
  R1 K mean: exact int64 sum of K * 2^24 over tokens (every fp16 is a multiple
     of 2^-24), then mu = fp32(fp64(sum) * 2^-24 / N). Order-independent.
  R2 smoothing: K_s = fp32(fp32(K) - mu), one RNE subtraction, not re-rounded
     to fp16. With smoothing off, K_s = fp32(K).
  R3 INT8 scale: per block (a head, `blk` consecutive tokens, all channels),
     a = max|x|, s = fp32(a / 127); symmetric codes, -128 never produced.
  R4 INT8 code: rint_half_even(fp32(x / s)), clamp [-127, 127]; a = 0 gives
     s = 0 and all codes 0.
  R5 sm_scale is applied at dequantization, not folded into Q.
  R6 online softmax over key tiles of `kv_tile` keys in ascending order
     (FlashAttention-2 style, [SA-Setup]): m_t = max(m_{t-1}, tile row max), the
     plain running max; P = exp(S - m_t) is formed against it; what was
     accumulated under m_{t-1} is scaled by exp(m_{t-1} - m_t). P16 =
     fp16_RNE(P); O accumulates P16 . V and the row sum l accumulates the same
     P16, so O is an exact weighted mean of V rows up to accumulation rounding
     (a constant V comes back exactly). In the MXFP4 path l likewise sums the
     MX-quantized P that multiplies V.
  R7 causal: key j is masked for query i when j > i (N_q = N_k).
  R8 MX blocks: 32 contiguous elements along the contraction dimension (d for
     Q and K_s; tokens, per channel, for V; keys, per query row inside a key
     tile, for P). E8M0 exponent e = floor(log2 a) - 2 clamped to [-127, 127];
     a = 0 gives e = 0 and all codes 0. Element code = nearest E2M1 value to
     x * 2^-e, ties to the even code index, saturating at +-6; the sign bit is
     the sign bit of x. Packing: element 2k in the low nibble of byte k.
  R14 INT8 P and V (the INT8 P,V ablation of [SA-Effects]; the page gives no
     granularity): V gets one scale per (head, channel) over
     all tokens, with the R3/R4 rules (a = max|V|, s = fp32(a / 127), code =
     rint_half_even(fp32(V / s))); P is formed against the running max (R6),
     so 0 <= P <= 1, and quantized with the fixed scale 1/127:
     code = rint_half_even(127 P). l sums the quantized P, O accumulates the
     quantized P times the dequantized V.
  R13 MX-FP8 variant for P and V (not on the pages; the accuracy variant of
     the FP4 path): the same blocks as R8, e = floor(log2 a) - 8 (E4M3's largest
     binade is 2^8), element = nearest E4M3 value to x * 2^-e, ties to the even
     code, saturating at 448; Q and K_s stay MXFP4.
"""
from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# Small helpers
# ---------------------------------------------------------------------------

LOG2E = 1.0 / math.log(2.0)


def as_f64(x16: np.ndarray) -> np.ndarray:
    """Exact widening of fp16 (or fp32) data to float64."""
    return np.asarray(x16).astype(np.float64)


def _causal_mask(rows: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """True where key j is hidden from query i (j > i), reading R7."""
    return keys[None, :] > rows[:, None]


# ---------------------------------------------------------------------------
# (c1) Exact attention in float64 -- the "full precision" reference that the
# cosine-similarity bar of [SA-Approach] is measured against.
# ---------------------------------------------------------------------------

def exact_attention(q, k, v, *, causal: bool, sm_scale: float, rows=None, row_chunk: int = 512):
    """O = softmax(sm_scale * Q K^T) V per (b, h), in float64.

    q, k, v: [B, H, N, d] fp16 (or any float) arrays. `rows` selects query rows
    (all rows if None). Softmax subtracts the row max before exponentiating.
    Returns float64 [B, H, len(rows), d].
    """
    B, H, N, d = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    keys = np.arange(N)
    out = np.empty((B, H, rows.size, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            K = as_f64(k[b, h])
            V = as_f64(v[b, h])
            for r0 in range(0, rows.size, row_chunk):
                rr = rows[r0:r0 + row_chunk]
                S = sm_scale * (as_f64(q[b, h, rr]) @ K.T)
                if causal:
                    S[_causal_mask(rr, keys)] = -np.inf
                S -= S.max(axis=1, keepdims=True)
                P = np.exp(S)
                P /= P.sum(axis=1, keepdims=True)
                out[b, h, r0:r0 + rr.size] = P @ V
    return out


# ---------------------------------------------------------------------------
# (c2) INT8 path, step by step: [SA-Approach], [SA-Summary].
# ---------------------------------------------------------------------------

def k_channel_sum(k16: np.ndarray) -> np.ndarray:
    """Exact sum over tokens of K * 2^24 per (b, h, channel) as int64 (reading R1)."""
    fixed = (as_f64(k16) * float(2 ** 24)).astype(np.int64)   # exact: integers below 2^41
    return fixed.sum(axis=2, dtype=np.int64)


def k_mean(k16: np.ndarray) -> np.ndarray:
    """mu[b, h, c]: the mean of K across tokens [SA-Approach], reading R1. float32 [B, H, d]."""
    N = k16.shape[2]
    total = k_channel_sum(k16).astype(np.float64)              # int64 -> f64, RNE
    return ((total * 2.0 ** -24) / float(N)).astype(np.float32)


def smooth_k(k16: np.ndarray, mu: np.ndarray | None) -> np.ndarray:
    """K_s = fp32(K) - mu in float32 (reading R2); mu=None means smoothing off."""
    kf = np.asarray(k16).astype(np.float32)
    if mu is None:
        return kf
    return kf - mu[:, :, None, :].astype(np.float32)


def int8_quant_blocks(x32: np.ndarray, blk: int):
    """Symmetric per-block INT8 quantization of x [B, H, N, d] (float32).

    Blocks are `blk` consecutive tokens x all d channels of one head
    ([SA-Approach]: per-token (blk=1) or per-block scales); the last block holds
    only the valid tokens. Readings R3, R4.
    Returns (codes int8 [B, H, N, d], scales float32 [B, H, ceil(N/blk)]).
    """
    x32 = np.asarray(x32, dtype=np.float32)
    B, H, N, d = x32.shape
    nblk = -(-N // blk)
    pad = nblk * blk - N
    xp = np.concatenate([x32, np.zeros((B, H, pad, d), np.float32)], axis=2) if pad else x32
    blocks = xp.reshape(B, H, nblk, blk, d)
    amax = np.abs(blocks).max(axis=(3, 4))                       # exact
    scales = (amax / np.float32(127.0)).astype(np.float32)       # fp32 division, correctly rounded
    safe = np.where(scales > 0, scales, np.float32(1.0)).astype(np.float32)
    q = blocks / safe[:, :, :, None, None]                       # fp32 division, correctly rounded
    codes = np.clip(np.rint(q), -127, 127)                       # rint: ties to even
    codes = np.where((scales > 0)[:, :, :, None, None], codes, 0.0)
    codes = codes.reshape(B, H, nblk * blk, d)[:, :, :N].astype(np.int8)
    return codes, scales


def int8_tensor_scale(x32: np.ndarray) -> np.float32:
    """One scale for a whole tensor (the per-tensor granularity of the smoothing
    ablation in [SA-Effects]): s = fp32(max|x| / 127), reading R3 with the block
    being the whole tensor."""
    return np.float32(np.float32(np.abs(np.asarray(x32, dtype=np.float32)).max()) / np.float32(127.0))


def int8_quant_with_scale(x32: np.ndarray, s: np.float32) -> np.ndarray:
    """Codes rint_half_even(fp32(x / s)) clamped to [-127, 127] with one given scale
    (reading R4; s = 0 gives zero codes). Returns int8 codes of x's shape."""
    x32 = np.asarray(x32, dtype=np.float32)
    s = np.float32(s)
    if s == 0:
        return np.zeros(x32.shape, np.int8)
    return np.clip(np.rint(x32 / s), -127, 127).astype(np.int8)


def quant_qk_int8(q16, k16, *, blk_q: int, blk_k: int, smooth: bool = True):
    """The quantization half of the INT8 path: mu, K_s, Q and K_s codes and scales.

    Returns dict(q_codes, q_scales, k_codes, k_scales, k_mean). k_mean is None
    when smoothing is off.
    """
    mu = k_mean(k16) if smooth else None
    ks = smooth_k(k16, mu)
    qc, qs = int8_quant_blocks(np.asarray(q16).astype(np.float32), blk_q)
    kc, kscl = int8_quant_blocks(ks, blk_k)
    return dict(q_codes=qc, q_scales=qs, k_codes=kc, k_scales=kscl, k_mean=mu)


def online_softmax_pv(S: np.ndarray, V: np.ndarray, *, kv_tile: int, round_p,
                      sum_rounded: bool = False, p_alternatives=None, lse_out=None):
    """FlashAttention-2 style online softmax and P.V over key tiles ([SA-Setup]).

    S: float64 scores [R, N] (already scaled, -inf where masked).
    V: float64 values [N, d] (already in the precision P.V consumes).
    round_p(P_tile) -> the P that multiplies V (fp16 RNE for the INT8 path, the
    MX-quantized P for the FP4 path, identity for an exact run).
    Reading R6: ascending tiles, P against the running max; l sums round_p(P)
    if sum_rounded else P. Returns O [R, d] float64.

    p_alternatives (test tolerance only, with sum_rounded): a callable giving,
    for a tile's P, other quantized P that an implementation computing P with
    a slightly different rounding could produce (a code decided by floating
    point lands on the other side of a rounding boundary). Then the function
    returns (O, allowance), allowance [R, d] bounding |O' - O| to first order
    for any mix of those alternatives: a weight that moves by dP changes O by
    dP * (v_j - O) / l, and |v_j - O| <= |v_j| + max|v| per channel.

    lse_out (optional float64 [R] array): receives the row log-sum-exp m + ln(l)
    of the final running max and row sum (reading Rb5), what a backward pass
    recomputes P from.
    """
    R, N = S.shape
    d = V.shape[1]
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    O = np.zeros((R, d))
    A = np.zeros((R, d)) if p_alternatives is not None else None
    dl = np.zeros(R)
    vbound = np.abs(V) + np.abs(V).max(axis=0, keepdims=True)
    for t0 in range(0, N, kv_tile):
        St = S[:, t0:t0 + kv_tile]
        with np.errstate(invalid="ignore"):
            m_new = np.maximum(m, St.max(axis=1))
            # factor for what was accumulated under the old max (0 before any valid key)
            alpha = np.where(np.isneginf(m_new), 0.0, np.exp(m - m_new))
            P = np.where(np.isneginf(St), 0.0, np.exp(St - m_new[:, None]))
        Pr = round_p(P)
        l = l * alpha + (Pr if sum_rounded else P).sum(axis=1)
        O = O * alpha[:, None] + Pr @ V[t0:t0 + kv_tile]
        if p_alternatives is not None:
            dP = np.zeros_like(Pr)
            for alt in p_alternatives(P):
                dP = np.maximum(dP, np.abs(alt - Pr))
            A = A * alpha[:, None] + dP @ vbound[t0:t0 + kv_tile]
            dl = dl * alpha + dP.sum(axis=1)
        m = m_new
    if lse_out is not None:
        lse_out[...] = m + np.log(l)
    if A is not None:
        return O / l[:, None], A / np.maximum(l - dl, 0.5 * l)[:, None]
    return O / l[:, None]


def int8_attention(q16, k16, v16, *, causal: bool, sm_scale: float, blk_q: int, blk_k: int,
                   kv_tile: int = 64, smooth: bool = True, rows=None, quantize: bool = True,
                   quant=None, lse=None):
    """Emulated INT8 SageAttention forward ([SA-Approach], [SA-Summary]), float64 out.

    Steps: mu and K_s (R1, R2); per-block INT8 codes of Q and K_s (R3, R4);
    S_int = codes_q . codes_k^T exactly; S = S_int * s_q * s_k * sm_scale (R5);
    causal mask (R7); online softmax with fp16 P and fp16 V, l from the fp16 P (R6).
    quantize=False replaces every code by the unquantized value (scale 1) and
    P16 by P: the same tiled arithmetic then reduces to exact attention.
    `quant` may pass a precomputed quant_qk_int8 result. `lse` (optional float64
    [B, H, len(rows)]) receives each row's log-sum-exp (online_softmax_pv).
    Returns float64 [B, H, len(rows), d].
    """
    B, H, N, d = q16.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    keys = np.arange(N)
    if quantize:
        qd = quant if quant is not None else quant_qk_int8(q16, k16, blk_q=blk_q, blk_k=blk_k, smooth=smooth)
    else:
        mu = k_mean(k16) if smooth else None
        ks = smooth_k(k16, mu)
    out = np.empty((B, H, rows.size, d))
    round16 = (lambda P: P.astype(np.float16).astype(np.float64)) if quantize else (lambda P: P)
    for b in range(B):
        for h in range(H):
            if quantize:
                cq = qd["q_codes"][b, h, rows].astype(np.float64)
                ck = qd["k_codes"][b, h].astype(np.float64)
                S_int = cq @ ck.T                                  # exact: |partial sums| < 2^53
                sq = qd["q_scales"][b, h][rows // blk_q].astype(np.float64)
                sk = qd["k_scales"][b, h][keys // blk_k].astype(np.float64)
                S = S_int * sq[:, None] * sk[None, :] * sm_scale
            else:
                S = (as_f64(q16[b, h, rows]) @ ks[b, h].astype(np.float64).T) * sm_scale
            if causal:
                S[_causal_mask(rows, keys)] = -np.inf
            out[b, h] = online_softmax_pv(S, as_f64(v16[b, h]), kv_tile=kv_tile, round_p=round16,
                                          sum_rounded=True, lse_out=None if lse is None else lse[b, h])
    return out


def int8_quant_v_channels(v16):
    """INT8 codes of V with one scale per (b, h, channel) over all tokens (reading R14).

    a = max over tokens of |V|, s = fp32(a / 127) (correctly rounded), code =
    rint_half_even(fp32(V / s)) in [-127, 127]; a = 0 gives s = 0 and codes 0.
    Returns (codes int8 [B, H, N, d], scales float32 [B, H, d]).
    """
    v32 = np.asarray(v16).astype(np.float32)
    amax = np.abs(v32).max(axis=2)                               # [B, H, d], exact
    scales = (amax / np.float32(127.0)).astype(np.float32)       # fp32 division, correctly rounded
    safe = np.where(scales > 0, scales, np.float32(1.0)).astype(np.float32)
    codes = np.clip(np.rint(v32 / safe[:, :, None, :]), -127, 127)   # fp32 division, ties to even
    codes = np.where((scales > 0)[:, :, None, :], codes, 0.0).astype(np.int8)
    return codes, scales


def int8_pv_attention(q16, k16, v16, *, causal: bool, sm_scale: float, blk_q: int, blk_k: int,
                      kv_tile: int = 64, smooth: bool = True, rows=None, quant=None,
                      flip_delta: float | None = None):
    """The INT8 P,V variant ([SA-Effects]: the ablation with P and V in INT8
    instead of FP16; [SA-Approach]: the faster kernel chosen per layer where
    cosine similarity stays above 99.8%), float64 out.

    Q and K_s as in int8_attention (R1-R5; blk_q = blk_k = 1 is the per-token
    form). V: per-channel INT8 (R14). Online softmax against the running max
    (R6), P quantized to rint(127 P) / 127 (R14); l sums the
    quantized P; O accumulates quantized P times dequantized V.
    Returns float64 [B, H, len(rows), d].

    flip_delta (test tolerance only): the P codes are decided by floating
    point, so an implementation whose P differs by a few ulps can round a
    127 P that lies next to a half-integer the other way. With flip_delta, P
    is also quantized after scaling by (1 -+ flip_delta) (never above 1, the
    largest P: its code is 127 either way) and the function returns
    (O, allowance) with the first-order bound of online_softmax_pv on what
    such flips can change.
    """
    B, H, N, d = q16.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    keys = np.arange(N)
    qd = quant if quant is not None else quant_qk_int8(q16, k16, blk_q=blk_q, blk_k=blk_k, smooth=smooth)
    vc, vs = int8_quant_v_channels(v16)
    round127 = lambda P: np.rint(127.0 * P) / 127.0
    alts = None
    if flip_delta is not None:
        alts = lambda P: [round127(P * (1.0 - flip_delta)), round127(np.minimum(P * (1.0 + flip_delta), 1.0))]
    out = np.empty((B, H, rows.size, d))
    allow = np.zeros_like(out) if alts is not None else None
    for b in range(B):
        for h in range(H):
            cq = qd["q_codes"][b, h, rows].astype(np.float64)
            ck = qd["k_codes"][b, h].astype(np.float64)
            sq = qd["q_scales"][b, h][rows // blk_q].astype(np.float64)
            sk = qd["k_scales"][b, h][keys // blk_k].astype(np.float64)
            S = (cq @ ck.T) * sq[:, None] * sk[None, :] * sm_scale
            if causal:
                S[_causal_mask(rows, keys)] = -np.inf
            Vh = vc[b, h].astype(np.float64) * vs[b, h].astype(np.float64)[None, :]
            r = online_softmax_pv(S, Vh, kv_tile=kv_tile, round_p=round127, sum_rounded=True,
                                  p_alternatives=alts)
            if alts is not None:
                out[b, h], allow[b, h] = r
            else:
                out[b, h] = r
    return (out, allow) if alts is not None else out


def fp16_attention(q16, k16, v16, *, causal: bool, sm_scale: float, kv_tile: int = 64, rows=None):
    """Unquantized FlashAttention-style forward, the baseline the method is
    measured against ([SA-Setup]: the kernels build on FlashAttention-2's
    tiled online softmax; [SA-Summary]: the speedup is quoted over it).

    S = (Q K^T) * sm_scale from the fp16 inputs, exactly (float64); causal mask
    (R7); the same tiled online softmax as the INT8 path (R6) with fp16 P and
    fp16 V, l summing the fp16 P. No quantization, no smoothing.
    Returns float64 [B, H, len(rows), d].
    """
    B, H, N, d = q16.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    keys = np.arange(N)
    round16 = lambda P: P.astype(np.float16).astype(np.float64)
    out = np.empty((B, H, rows.size, d))
    for b in range(B):
        for h in range(H):
            S = (as_f64(q16[b, h, rows]) @ as_f64(k16[b, h]).T) * sm_scale
            if causal:
                S[_causal_mask(rows, keys)] = -np.inf
            out[b, h] = online_softmax_pv(S, as_f64(v16[b, h]), kv_tile=kv_tile, round_p=round16,
                                          sum_rounded=True)
    return out


# ---------------------------------------------------------------------------
# (c3) Microscaled FP4 path: [SA3-Abstract] and the MX format it builds on.
# ---------------------------------------------------------------------------

# E2M1 magnitudes by code index 0..7 (sign is bit 3): 1 sign, 2 exponent
# (bias 1), 1 mantissa bit; exponent field 0 is subnormal (m * 0.5).
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
MX_BLOCK = 32


def e8m0_exponent(amax: np.ndarray) -> np.ndarray:
    """Shared block exponent e = floor(log2 a) - 2, clamped to [-127, 127]; 0 where a == 0 (R8).

    floor(log2 a) comes from frexp: a = f * 2^x with f in [0.5, 1) gives x - 1,
    exact for every positive float including subnormals.
    """
    a = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.clip(ex.astype(np.int64) - 1 - 2, -127, 127)
    return np.where(a > 0, e, 0)


def e2m1_nearest(y: np.ndarray) -> np.ndarray:
    """Code index 0..7 of the E2M1 magnitude nearest to y >= 0; ties go to the even index.

    Brute force over the eight magnitudes; values above 6 land on 6 (saturation).
    """
    y = np.asarray(y, dtype=np.float64)
    dist = np.abs(y[..., None] - E2M1_MAGNITUDES)
    idx = np.argmin(dist, axis=-1)                           # first (lower) index on a tie
    nxt = np.minimum(idx + 1, 7)
    d_idx = np.take_along_axis(dist, idx[..., None], -1)[..., 0]
    d_nxt = np.take_along_axis(dist, nxt[..., None], -1)[..., 0]
    tie_to_next = (idx % 2 == 1) & (nxt != idx) & (d_nxt == d_idx)
    return np.where(tie_to_next, nxt, idx)


def mx_quantize(x: np.ndarray, axis: int):
    """MXFP4-quantize x in blocks of 32 along `axis` (zero-padded at the end).

    x is taken at its own precision (float32 for Q, K_s and V, float64 for the
    oracle's P); the arithmetic below is exact in float64.
    Returns (codes uint8 0..15 [same shape as x], e8m0 uint8 [.., nblk ..],
    decoded float64 values [same shape as x]).
    """
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
    n = x.shape[-1]
    nblk = -(-n // MX_BLOCK)
    pad = nblk * MX_BLOCK - n
    if pad:
        x = np.concatenate([x, np.zeros(x.shape[:-1] + (pad,))], axis=-1)
    xb = x.reshape(x.shape[:-1] + (nblk, MX_BLOCK))
    amax = np.abs(xb).max(axis=-1)
    e = e8m0_exponent(amax)
    y = np.abs(xb) * np.exp2(-e.astype(np.float64))[..., None]       # exact power-of-two scaling
    mag = e2m1_nearest(y)
    sign = np.signbit(xb)
    codes = (mag + 8 * sign).astype(np.uint8)
    vals = np.where(sign, -1.0, 1.0) * E2M1_MAGNITUDES[mag] * np.exp2(e.astype(np.float64))[..., None]
    codes = codes.reshape(x.shape)[..., :n]
    vals = vals.reshape(x.shape)[..., :n]
    e8 = (e + 127).astype(np.uint8)
    return np.moveaxis(codes, -1, axis), np.moveaxis(e8, -1, axis), np.moveaxis(vals, -1, axis)


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes along the last axis (even length): element 2k -> low nibble of byte k."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


# MX-FP8 (E4M3 elements, E8M0 block exponent): the accuracy variant for P and V
# (reading R13). E4M3: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits;
# exponent field 0 is subnormal (m * 2^-9); code 0x7F (and 0xFF) is NaN, so the
# largest magnitude is 0x7E = 448 = 1.75 * 2^8.
E4M3_MAX = 448.0


def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """Decode E4M3 bytes to float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(ef == 0, m * 2.0 ** -9, (8.0 + m) * np.exp2(ef.astype(np.float64) - 10.0))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


def e4m3_nearest(y: np.ndarray) -> np.ndarray:
    """Code (0..0x7E) of the E4M3 magnitude nearest to y >= 0, ties to the even
    code, saturating at 448.

    In the binade [2^e, 2^(e+1)) (e clamped to [-6, 8]; below 2^-6 the subnormal
    spacing 2^-9 continues) the representable magnitudes are multiples of
    2^(e-3), so the nearest one is q * 2^(e-3) with q = round-half-even(y / 2^(e-3))
    (q = 8 + mantissa, or the subnormal mantissa; q even <=> code even).
    """
    y = np.asarray(y, dtype=np.float64)
    _, ex = np.frexp(np.where(y > 0, y, 1.0))
    e = np.clip(ex.astype(np.int64) - 1, -6, 8)
    step = np.exp2((e - 3).astype(np.float64))
    q = np.round(y / step)                         # numpy rounds halves to even; y/step is exact
    val = np.minimum(q * step, E4M3_MAX)
    # encode val (a representable magnitude) as a code
    _, vx = np.frexp(np.where(val > 0, val, 1.0))
    ve = vx.astype(np.int64) - 1
    normal = val >= 2.0 ** -6
    ef = np.where(normal, ve + 7, 0)
    mant = np.where(normal, val / np.exp2(ve.astype(np.float64)) * 8 - 8, val * 2.0 ** 9)
    return np.where(y > 0, ef * 8 + np.round(mant).astype(np.int64), 0).astype(np.int64)


def mx_quantize_fp8(x: np.ndarray, axis: int):
    """MX-FP8 quantization of x in blocks of 32 along `axis` (zero-padded at the
    end): e = floor(log2 amax) - 8 clamped to [-127, 127] (0 for an all-zero
    block), element = nearest E4M3 to x * 2^-e, ties to even, saturating at 448,
    sign bit = sign bit of x. Returns (codes uint8, e8m0 uint8, values float64)
    like mx_quantize."""
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
    n = x.shape[-1]
    nblk = -(-n // MX_BLOCK)
    pad = nblk * MX_BLOCK - n
    if pad:
        x = np.concatenate([x, np.zeros(x.shape[:-1] + (pad,))], axis=-1)
    xb = x.reshape(x.shape[:-1] + (nblk, MX_BLOCK))
    amax = np.abs(xb).max(axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    e = np.where(amax > 0, np.clip(ex.astype(np.int64) - 1 - 8, -127, 127), 0)
    y = np.abs(xb) * np.exp2(-e.astype(np.float64))[..., None]
    mag = e4m3_nearest(y)
    sign = np.signbit(xb)
    codes = (mag + 0x80 * sign).astype(np.uint8)
    vals = np.where(sign, -1.0, 1.0) * e4m3_value(mag) * np.exp2(e.astype(np.float64))[..., None]
    codes = codes.reshape(x.shape)[..., :n]
    vals = vals.reshape(x.shape)[..., :n]
    e8 = (e + 127).astype(np.uint8)
    return np.moveaxis(codes, -1, axis), np.moveaxis(e8, -1, axis), np.moveaxis(vals, -1, axis)


def quant_mxfp4(q16, k16, v16, *, smooth: bool = True, v_fp8: bool = False):
    """MX quantization of Q (along d), K_s (along d) and V (along tokens, per channel).

    V is MXFP4, or MX-FP8 with v_fp8 (R13). Returns dict with codes/e8m0/values
    for q, k, v; v arrays are in [B, H, N, d] orientation (blocks run along N).
    k_mean is None with smoothing off.
    """
    mu = k_mean(k16) if smooth else None
    ks = smooth_k(k16, mu)
    qc, qe, qv = mx_quantize(np.asarray(q16).astype(np.float32), axis=3)
    kc, ke, kv = mx_quantize(ks, axis=3)
    vq = mx_quantize_fp8 if v_fp8 else mx_quantize
    vc, ve, vv = vq(np.asarray(v16).astype(np.float32), axis=2)
    return dict(q_codes=qc, q_e8m0=qe, q_vals=qv, k_codes=kc, k_e8m0=ke, k_vals=kv,
                v_codes=vc, v_e8m0=ve, v_vals=vv, k_mean=mu)


def mxfp4_attention(q16, k16, v16, *, causal: bool, sm_scale: float, kv_tile: int = 64,
                    smooth: bool = True, rows=None, quant=None, quantize_p: bool = True,
                    pv_fp8: bool = False, flip_delta: float | None = None):
    """Emulated microscaled-FP4 attention ([SA3-Abstract] with the MX format, reading R8).

    Q, K_s, V and the softmax P are MXFP4 (with pv_fp8, P and V are MX-FP8
    instead, reading R13); the scores are the exact products of the decoded
    values (what an FP32-accumulating block-scaled matrix unit computes up to
    accumulation rounding); online softmax as in the INT8 path with the
    MX-quantized P in place of P16 (l sums the same quantized P, reading R6).
    Returns float64 [B, H, len(rows), d].

    flip_delta (test tolerance only): the P codes and block exponents are
    decided by floating point, so an implementation whose P differs by a few
    ulps can round a P that lies next to a boundary the other way. With
    flip_delta, P is also quantized after scaling by (1 -+ flip_delta) (a P of
    exactly 1, the reference score, only upwards) and the function returns
    (O, allowance) with the first-order bound of online_softmax_pv on what
    such flips can change.
    """
    B, H, N, d = q16.shape
    if kv_tile % MX_BLOCK:
        raise ValueError("kv_tile must be a multiple of 32")
    rows = np.arange(N) if rows is None else np.asarray(rows)
    keys = np.arange(N)
    qd = quant if quant is not None else quant_mxfp4(q16, k16, v16, smooth=smooth, v_fp8=pv_fp8)
    out = np.empty((B, H, rows.size, d))
    pq = mx_quantize_fp8 if pv_fp8 else mx_quantize
    if quantize_p:
        def round_p(P):
            # blocks of 32 keys inside the tile; a short tail tile is zero-padded by the quantizer
            return pq(P, axis=1)[2]
    else:
        def round_p(P):
            return P
    alts = None
    if flip_delta is not None and quantize_p:
        # a P of exactly 1 is the row's running max itself; an implementation that
        # rounds its reference down keeps that P >= 1, so it only moves up
        alts = lambda P: [round_p(np.where(P == 1.0, P, P * (1.0 - flip_delta))), round_p(P * (1.0 + flip_delta))]
    allow = np.zeros_like(out) if alts is not None else None
    for b in range(B):
        for h in range(H):
            S = (qd["q_vals"][b, h, rows] @ qd["k_vals"][b, h].T) * sm_scale
            if causal:
                S[_causal_mask(rows, keys)] = -np.inf
            r = online_softmax_pv(S, qd["v_vals"][b, h], kv_tile=kv_tile, round_p=round_p,
                                  sum_rounded=True, p_alternatives=alts)
            if alts is not None:
                out[b, h], allow[b, h] = r
            else:
                out[b, h] = r
    return (out, allow) if alts is not None else out


# ---------------------------------------------------------------------------
# Metrics named by [SA-Setup]: cosine similarity, relative L1, RMSE (+ max abs).
# ---------------------------------------------------------------------------

def metrics(test: np.ndarray, ref: np.ndarray) -> dict:
    a = np.asarray(test, dtype=np.float64).ravel()
    b = np.asarray(ref, dtype=np.float64).ravel()
    cos = float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))
    return dict(cos=cos,
                max_abs=float(np.max(np.abs(a - b))) if a.size else 0.0,
                rel_l1=float(np.sum(np.abs(a - b)) / np.sum(np.abs(b))),
                rmse=float(np.sqrt(np.mean((a - b) ** 2))))
