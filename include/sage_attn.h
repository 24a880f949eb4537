/*
 * sage_attn.h -- C ABI of the MI355X (gfx950) quantized-attention library.
 *
 * The library computes the forward pass that the SageAttention page
 * ("SageAttention: Accurate 8-Bit Attention for Plug-and-play Inference
 * Acceleration", atlas.scime.ai summary, sections "Approach" and the summary
 * paragraph) describes as a plug-and-play replacement for attention: Q, K, V
 * in, O out. INT8 path: subtract the per-channel mean of K over tokens,
 * quantize Q and K to INT8 with per-block float scales, QK^T with integer
 * accumulation, dequantize, online softmax (FlashAttention-2 style, the page's
 * "Experimental setup: builds on"), P.V in FP16. MXFP4 path: the microscaled
 * FP4 idea of "SageAttention3: Microscaling FP4 Attention for Inference and
 * An Exploration of 8-Bit Training" (abstract), using E2M1 elements with one
 * E8M0 scale per 32 elements (the MX format its reference list names).
 * INT8 P.V variants (modes 6, 7): the page's "Measured effects" ablation in
 * which the second product also runs in INT8 (P and V quantized, no FP16
 * operand left), the faster kernel its "Approach" selects per layer where
 * cosine similarity stays above 99.8%: V with one scale per (head, channel)
 * over all tokens, P = exp(S - running row max) in [0, 1] as the integer
 * weight round(127 P), P.V accumulated exactly in int32, the row sum from the
 * same integer weights.
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, C-contiguous [B, H, N, d] (batch, head, token,
 *     channel) unless stated otherwise. fp16 means IEEE binary16.
 *   - Pointers named q, k, v, out, *_codes, *_scales, *_fp4, *_e8m0, k_mean
 *     and workspace are DEVICE pointers on the current HIP device. q, k, v,
 *     out and workspace must be 16-byte aligned; workspace 256-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream). All
 *     work is enqueued on it; the library never synchronizes, allocates or
 *     frees device memory. Results are valid once the stream reaches them.
 *   - The caller owns every buffer. The library keeps no state besides a
 *     per-device architecture check, a thread-local error message and, for
 *     sage_attn_fwd_noalloc only, one static device scratch array per GPU, so
 *     calls are re-entrant; calls that share a workspace (or, for the
 *     allocation-free entry point, a GPU) must be stream-ordered.
 *   - Supported head dims d: 64 and 128. 1 <= N <= 4194304. B, H >= 1.
 *   - q, k, v (and dout) hold finite fp16 values; outputs for inputs with inf
 *     or NaN are unspecified (no fault, no error code).
 *   - Every argument check happens before the first HIP call, so every error
 *     except SAGE_ERR_HIP and SAGE_ERR_NO_DEVICE is reported on a host with no
 *     GPU. Errors return a negative sage_status_t and set sage_last_error();
 *     no exception crosses the ABI and the library never aborts.
 */
#ifndef SAGE_ATTN_H
#define SAGE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sage_status {
  SAGE_OK = 0,
  SAGE_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, bad size, non-finite scale */
  SAGE_ERR_UNSUPPORTED = -2,  /* d, mode or block size not supported; device is not gfx950 */
  SAGE_ERR_WORKSPACE = -3,    /* workspace smaller than the *_workspace_size() query */
  SAGE_ERR_NO_DEVICE = -4,    /* no HIP device is visible */
  SAGE_ERR_HIP = -5           /* a HIP launch or runtime call failed */
} sage_status_t;

/* Modes (low byte of `mode`). */
#define SAGE_MODE_INT8_Q128_K64 0  /* INT8 Q,K; Q scale blocks of 128 tokens, K blocks of 64 */
#define SAGE_MODE_INT8_Q64_K64 1   /* INT8 Q,K; Q and K scale blocks of 64 tokens            */
#define SAGE_MODE_MXFP4 2          /* MXFP4 Q, K_s, V and P, E8M0 scale per 32 elements      */
#define SAGE_MODE_INT8_PER_TOKEN 3 /* INT8 Q,K with one scale per token (blocks of 1)        */
#define SAGE_MODE_FP16 4           /* no quantization: fp16 Q K^T on the FP16 matrix op, same */
                                   /* online softmax and fp16 P.V (FlashAttention-style        */
                                   /* baseline of the same kernel; reads q, k when computing)  */
#define SAGE_MODE_MXFP4_FP8PV 5    /* MXFP4 Q, K_s; P and V in MX-FP8 (E4M3 + E8M0 per 32):   */
                                   /* the accuracy variant of SAGE_MODE_MXFP4                 */
#define SAGE_MODE_INT8_PV 6        /* as SAGE_MODE_INT8_Q128_K64, with P and V in INT8 as well */
                                   /* (P.V on the INT8 matrix op; N <= 131072)                */
#define SAGE_MODE_INT8_PV_PER_TOKEN 7 /* as SAGE_MODE_INT8_PER_TOKEN, with P and V in INT8   */
                                   /* (N <= 131072)                                           */
#define SAGE_MODE_MASK 0xff

/* Flags OR-ed into `mode` (or passed as `flags`). */
#define SAGE_FLAG_NO_SMOOTH 0x100  /* skip the K mean subtraction (ablation only) */
#define SAGE_FLAG_FP8_V 0x200      /* sage_quant_mxfp4 only: V in MX-FP8 (E4M3) codes */
#define SAGE_FLAG_FUSED_Q 0x400    /* modes 0 and 1: Q quantized inside the attention kernel (see
                                      sage_attn_prepare / sage_attn_compute) */

/* Human-readable name of a status code; never NULL. */
const char* sage_status_string(int status);

/* Detail text of the last error raised on the calling thread ("" if none). */
const char* sage_last_error(void);

/*
 * Bytes of device workspace sage_attn_fwd / sage_attn_prepare /
 * sage_attn_compute need for this problem (0 if the arguments are invalid).
 * The workspace holds the quantized operands between the two phases.
 */
size_t sage_attn_workspace_size(int B, int H, int N, int d, int mode);

/*
 * Full forward pass: out = attention(q, k, v) computed by the quantized
 * method of `mode` (SageAttention page, "Approach"; SageAttention3 abstract
 * for SAGE_MODE_MXFP4). Equivalent to sage_attn_prepare followed by
 * sage_attn_compute on the same stream and workspace. In modes 0 and 1 with
 * at least 65536 token rows (B * H * N) both phases run with
 * SAGE_FLAG_FUSED_Q (whatever `mode` says about that flag): the attention
 * kernel quantizes Q itself, to the same codes and scales.
 *   q, k, v  fp16 [B, H, N, d] device, read only.
 *   out      fp16 [B, H, N, d] device, written (may not alias q, k, v).
 *   causal   0: no mask; 1: key j is hidden from query i when j > i.
 *   sm_scale softmax temperature applied to QK^T; finite and > 0
 *            (the usual value is 1/sqrt(d)).
 *   mode     SAGE_MODE_* | SAGE_FLAG_*.
 *   workspace, workspace_bytes  scratch of at least sage_attn_workspace_size().
 * Returns SAGE_OK or a negative sage_status_t; on error nothing is enqueued
 * (except after SAGE_ERR_HIP, where earlier kernels of the call may run).
 */
int sage_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int N,
                  int d, int causal, float sm_scale, int mode, void* workspace,
                  size_t workspace_bytes, void* stream);

/* Bytes of device scratch sage_attn_fwd_noalloc holds on each device. */
#define SAGE_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/*
 * sage_attn_fwd for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * allocation. Same arguments (without the workspace), kernels and results as
 * sage_attn_fwd; the workspace is a scratch array of SAGE_NOALLOC_SCRATCH_BYTES
 * (256 MiB) that the library holds on every device it runs on, from the
 * loading of its code object until the process ends. The call allocates and
 * frees nothing; its first call on a device looks up that device's scratch
 * address once.
 *   Limit: a problem whose workspace (sage_attn_workspace_size) exceeds
 *   SAGE_NOALLOC_SCRATCH_BYTES returns SAGE_ERR_WORKSPACE and enqueues nothing.
 *   Sharing: every call on one device uses that device's one scratch array.
 *   Calls whose work can overlap on a device (unordered streams, several host
 *   threads) race on it and may produce wrong outputs; order them on one
 *   stream. The scratch keeps the last call's quantized operands; each call's
 *   prepare phase writes every byte its attention kernel reads, so nothing has
 *   to be cleared between calls.
 */
int sage_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, int B, int H, int N,
                          int d, int causal, float sm_scale, int mode, void* stream);

/*
 * Training forward: sage_attn_fwd that also writes the row log-sum-exp a
 * backward pass needs (FlashAttention-2's saved statistic; the SageAttention
 * page's "Experimental setup" names FlashAttention-2 as the base).
 *   lse   fp32 [B, H, N] device, written: lse[b,h,i] = ln sum_j exp(s_ij)
 *         over the scaled (and, with smoothing, mean-smoothed) scores the
 *         kernel used, where the sum adds the fp16-rounded weights that
 *         multiply V. 4-byte aligned.
 *   mode  SAGE_MODE_INT8_Q128_K64 or SAGE_MODE_INT8_Q64_K64, optionally
 *         | SAGE_FLAG_NO_SMOOTH; other modes return SAGE_ERR_UNSUPPORTED.
 * Other arguments, the workspace and the errors as sage_attn_fwd (a workspace
 * of sage_attn_bwd_workspace_size bytes also serves).
 */
int sage_attn_fwd_lse(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                      int N, int d, int causal, float sm_scale, int mode, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace sage_attn_bwd needs (0 if the arguments are
 * invalid or the mode is not a per-block INT8 mode).
 */
size_t sage_attn_bwd_workspace_size(int B, int H, int N, int d, int mode);

/*
 * INT8 backward pass: the gradients of the loss sum(out * dout) with respect
 * to q, k and v, for the 8-bit attention training of "SageAttention3:
 * Microscaling FP4 Attention for Inference and An Exploration of 8-Bit
 * Training" (abstract; INT8 per the scifaro.com list of related papers) in
 * FlashAttention-2's form (recompute the scores from Q and K, P = exp(S -
 * lse)). Every one of its five matrix products runs on INT8 codes with int32
 * accumulation: the forward's Q and mean-smoothed K codes for the scores, dO
 * per 64-token block and V per token for dO V^T, and P and dS quantized per
 * aligned 32 x 32 tile (max|x| / 127) for P^T dO, dS K and dS^T Q.
 *   q, k, v      fp16 [B, H, N, d] device: the forward's inputs.
 *   out, lse     the forward's output (fp16 [B, H, N, d]) and row log-sum-exp
 *                (fp32 [B, H, N]) from sage_attn_fwd_lse with the same mode,
 *                causal and sm_scale.
 *   dout         fp16 [B, H, N, d] device: the gradient of the loss with
 *                respect to out.
 *   dq, dk, dv   fp32 [B, H, N, d] device, written (16-byte aligned; may not
 *                alias the inputs). dk is the gradient with respect to k
 *                itself: the one through the token mean of the smoothing is
 *                zero in exact arithmetic (every row of dS sums to zero) and
 *                is not formed.
 *   mode         SAGE_MODE_INT8_Q128_K64 or SAGE_MODE_INT8_Q64_K64 (the Q
 *                block of the scores), optionally | SAGE_FLAG_NO_SMOOTH.
 *   workspace, workspace_bytes  at least sage_attn_bwd_workspace_size().
 * Returns SAGE_OK or a negative sage_status_t with the conventions of
 * sage_attn_fwd.
 */
int sage_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                  const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, int d,
                  int causal, float sm_scale, int mode, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * First phase of sage_attn_fwd: the K channel mean and the quantization of
 * Q, K (and of V, in the modes that quantize it: MXFP4, MX-FP8 or INT8 codes)
 * into `workspace`. The steps are those of sage_quant_qk / sage_quant_mxfp4 /
 * sage_quant_v_int8; the workspace layout is private. SAGE_MODE_FP16 has
 * nothing to prepare (the call only validates its arguments). With
 * SAGE_FLAG_FUSED_Q (modes 0 and 1 only; other modes return
 * SAGE_ERR_UNSUPPORTED) Q is left out: sage_attn_compute with that flag
 * quantizes it in the attention kernel's prologue (block maxima, scales and
 * codes as sage_quant_qk defines them).
 */
int sage_attn_prepare(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                      int mode, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Second phase of sage_attn_fwd: the fused attention kernel (quantized QK^T,
 * dequantization, online softmax, P.V, normalization) reading the operands a
 * previous sage_attn_prepare with the same B, H, N, d and mode left in
 * `workspace`, writing fp16 `out` [B, H, N, d]. Arguments as for sage_attn_fwd.
 *   q, k  the fp16 tensors given to sage_attn_prepare. Only SAGE_MODE_FP16
 *         reads them here, and q also with SAGE_FLAG_FUSED_Q (the quantized
 *         modes read their codes from the workspace and accept NULL).
 *   v     the fp16 V given to sage_attn_prepare, read here by every mode whose
 *         P.V runs in fp16 (all but SAGE_MODE_MXFP4, SAGE_MODE_MXFP4_FP8PV and
 *         the INT8 P.V modes, which read V codes from the workspace and
 *         accept NULL). Its contents must not change between the two calls.
 */
int sage_attn_compute(const void* q, const void* k, const void* v, void* out, int B, int H, int N,
                      int d, int causal, float sm_scale, int mode, const void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * Test hook for the integer scores of the INT8 modes (SageAttention page,
 * "Approach": QK^T of the INT8 codes with integer accumulation). Runs the
 * attention kernel of `mode` (0, 1 or 3; non-causal; SAGE_FLAG_FUSED_Q is
 * refused, the hook reads the Q codes) on a workspace prepared by
 * sage_attn_prepare for the same B, H, N, d and mode, writing `out` as
 * sage_attn_compute does (reading fp16 `v`, the V given to sage_attn_prepare),
 * and copies the int32 scores q_codes . k_codes^T that
 * the kernel's INT8 matrix op produced for key tile `k_tile` (keys 64 k_tile ..
 * +63) and query tile `q_tile` (queries 256 q_tile .. +255) of head `bh` into
 * s_out, int32 [256, 64] device, query-major. Rows and keys at or past N hold
 * the scores of the zero-padded codes (0).
 *   bh in [0, B*H), q_tile in [0, ceil(N/256)), k_tile in [0, ceil(N/64)).
 */
int sage_attn_dump_scores(const void* v, void* out, int B, int H, int N, int d, float sm_scale, int mode,
                          const void* workspace, size_t workspace_bytes, int bh, int q_tile, int k_tile,
                          int32_t* s_out, void* stream);

/* Bytes of device workspace sage_quant_qk, sage_quant_mxfp4 and
 * sage_quant_v_int8 need. */
size_t sage_quant_workspace_size(int B, int H, int N, int d);

/*
 * INT8 quantization of Q and the mean-smoothed K (SageAttention page,
 * "Approach": subtract the mean of K across tokens, then INT8 with per-block
 * or per-token scales).
 *   q, k       fp16 [B, H, N, d] device.
 *   blk_q, blk_k  tokens per scale block: 1 (per token), 16, 32, 64 or 128.
 *   flags      0 or SAGE_FLAG_NO_SMOOTH.
 *   q_codes, k_codes   int8 [B, H, N, d] device, written.
 *   q_scales   fp32 [B, H, ceil(N/blk_q)] device, written.
 *   k_scales   fp32 [B, H, ceil(N/blk_k)] device, written.
 *   k_mean     fp32 [B, H, d] device, written; may be NULL.
 * Definitions (bit-exact):
 *   mu[b,h,c] = fp32( fp64(sum_n K[b,h,n,c] * 2^24 as an exact int64) * 2^-24 / N ).
 *   K_s = fp32(K) - mu (fp32 subtraction); with SAGE_FLAG_NO_SMOOTH, K_s = fp32(K).
 *   per block: a = max |x|, s = fp32(a / 127) (correctly rounded division),
 *   code = round_half_even(fp32(x / s)) in [-127, 127]; a = 0 gives s = 0, codes 0.
 */
int sage_quant_qk(const void* q, const void* k, int B, int H, int N, int d, int blk_q, int blk_k,
                  int flags, int8_t* q_codes, float* q_scales, int8_t* k_codes, float* k_scales,
                  float* k_mean, void* workspace, size_t workspace_bytes, void* stream);

/*
 * MXFP4 quantization of Q, the mean-smoothed K and V (SageAttention3 abstract;
 * MX format: 32 elements share one E8M0 exponent).
 *   q_fp4, k_fp4   uint8 [B, H, N, d/2]: E2M1 codes, element 2i in the low nibble.
 *   q_e8m0, k_e8m0 uint8 [B, H, N, d/32]: blocks of 32 channels.
 *   vt_fp4   uint8 [B, H, d, Nv/2], Nv = N rounded up to a multiple of 32:
 *            V transposed, blocks of 32 tokens per channel, zero-padded.
 *            With SAGE_FLAG_FP8_V: uint8 [B, H, d, Nv] E4M3 codes (one per byte).
 *   vt_e8m0  uint8 [B, H, d, Nv/32].
 *   k_mean   fp32 [B, H, d] or NULL.
 *   flags    0, SAGE_FLAG_NO_SMOOTH and/or SAGE_FLAG_FP8_V.
 * Definitions (bit-exact): a = max |x| over the block; e = floor(log2 a) - 2
 * clamped to [-127, 127] (e = 0 when a = 0); E8M0 byte = e + 127; element =
 * E2M1 value nearest to x * 2^-e (ties to the even code, saturating at 6),
 * sign bit = sign bit of x. MX-FP8 (V with SAGE_FLAG_FP8_V): e = floor(log2 a)
 * - 8, element = E4M3 value nearest to x * 2^-e (ties to the even code,
 * saturating at 448).
 */
int sage_quant_mxfp4(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                     int flags, uint8_t* q_fp4, uint8_t* q_e8m0, uint8_t* k_fp4, uint8_t* k_e8m0,
                     uint8_t* vt_fp4, uint8_t* vt_e8m0, float* k_mean, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * Per-channel INT8 quantization of V, the V operand of the INT8 P.V modes
 * (SageAttention page, "Measured effects": P and V quantized to INT8; the
 * page gives no granularity, and one scale per channel is constant along the
 * contraction over tokens).
 *   v          fp16 [B, H, N, d] device.
 *   vt_codes   int8 [B, H, d, Nv] device, written: V transposed, Nv = N rounded
 *              up to a multiple of 16, tokens >= N zero.
 *   v_scales   fp32 [B, H, d] device, written.
 * Definitions (bit-exact): a = max over tokens of |V[b,h,:,c]| (V finite),
 * s = fp32(a / 127) (correctly rounded), code = round_half_even(fp32(V / s))
 * in [-127, 127]; a = 0 gives s = 0 and zero codes.
 */
int sage_quant_v_int8(const void* v, int B, int H, int N, int d, int8_t* vt_codes, float* v_scales,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Shader-clock probe, for throughput reports (not part of the attention path).
 * One wave spins until the device's shader-clock counter has advanced by
 * `cycles` (1 <= cycles <= 2^32) and writes to `out` (device, int64 [2],
 * 8-byte aligned) the cycles it counted and the ticks of the device's
 * constant-rate wall clock over the same interval:
 *   shader clock (kHz) = out[0] / out[1] * sage_wall_clock_khz().
 * Enqueued on a second stream while a workload runs, it gives the clock under
 * that load (lower than nominal when the chip throttles). It occupies one
 * wave slot of one compute unit for its duration.
 */
int sage_clock_probe(long long cycles, long long* out, void* stream);
/* The current device's wall-clock rate in kHz, written to *khz (host). */
int sage_wall_clock_khz(int* khz);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_ATTN_H */
