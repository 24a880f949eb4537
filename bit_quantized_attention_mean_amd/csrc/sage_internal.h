// Internal declarations of the gfx950 quantized-attention library: vector
// types, the private workspace layout and the kernel launchers. Not part of
// the public C ABI (include/sage_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sage {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

// Rows per quantization tile (and per MXFP4 attention workgroup), query rows
// per INT8 attention workgroup, and keys per key tile. Every per-head row
// count in the workspace is padded to a multiple of kRowPad, with zero rows,
// so the attention kernels' tile loads never need bounds checks.
constexpr int kQTile = 128;
constexpr int kWGQ = 256;
constexpr int kKTile = 64;
constexpr int kRowPad = 256;

constexpr int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Workgroup barrier that orders LDS only: waits for this wave's LDS reads and
// writes, then s_barrier. Unlike __syncthreads() it does not wait for
// outstanding global loads, so tile prefetches stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Raw buffer resource over `bytes` bytes at p (gfx9 descriptor word 3): loads
// through it take a per-lane offset and a scalar offset, and return zeros past
// `bytes`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}

// INT8 codes of a per-block quantization (shared by the quantization kernels
// and the attention kernel's in-kernel Q quantization).
// Codes. fp32(x / s) is formed without a division per element: with
// y = fp32(1 / s) (one IEEE division per scale) and q0 = fp32(x * y), the
// remainder x - q0 * s is exact in one fma and q0 + r * y rounded once is the
// correctly rounded quotient (Markstein's correction step; its preconditions
// hold here: y is the rounded reciprocal of s, q0 is within one ulp, the
// quotient is at most 127 in magnitude, and with s >= 2^-60 every x whose
// code can be nonzero is far above the subnormal range, so the remainder is
// exact). Smaller scales take the plain division; s = 0 means an all-zero
// block and zero codes.
// The result is returned as the bits of t = fp32(q + 1.5 * 2^23), which rounds
// q to the nearest integer, ties to even (the sum lies in [2^23, 2^24), whose
// ulp is 1, and 1.5 * 2^23 is even): the low byte of t is that integer as a
// two's complement int8. |q| <= 127 needs no clamp: q = x / s with |x| <= a and
// s = fp32(a / 127), so |q| <= 127 * (1 + 2^-24).
constexpr float kMarksteinMinScale = 0x1p-60f;
constexpr float kRound = 12582912.0f;

// s >= kMarksteinMinScale, y = fp32(1 / s)
__device__ __forceinline__ unsigned int8_code_bits(float x, float s, float y) {
  const float q0 = x * y;
  const float r = __builtin_fmaf(-q0, s, x);
  return __float_as_uint(__builtin_fmaf(r, y, q0) + kRound);
}
// The same code for an fp16 x, with the widening folded into the two
// operations that read x (v_fma_mix_f32 takes an fp16 operand): q0 =
// fma(x, y, +0) is the rounded product x * y, except that a -0 product
// becomes +0 (only x = -0 gives one: |x * y| >= 2^-24 * 127 / 65504 otherwise),
// and for x = +-0 both forms end at t = 1.5 * 2^23. The bits equal
// int8_code_bits(float(x), s, y).
__device__ __forceinline__ unsigned int8_code_bits_h(_Float16 x, float s, float y) {
  const float q0 = __builtin_fmaf(static_cast<float>(x), y, 0.0f);
  const float r = __builtin_fmaf(-q0, s, static_cast<float>(x));
  return __float_as_uint(__builtin_fmaf(r, y, q0) + kRound);
}
// any s >= 0 (the slow path for tiny scales; s = 0 gives code 0)
__device__ __forceinline__ unsigned int8_code_bits_div(float x, float s) {
  return __float_as_uint((s > 0.f ? x / s : 0.f) + kRound);
}

// Low bytes of w[0..3] -> one word, byte i = low byte of w[i].
__device__ __forceinline__ unsigned pack_low_bytes(unsigned w0, unsigned w1, unsigned w2, unsigned w3) {
  return __builtin_amdgcn_perm(__builtin_amdgcn_perm(w3, w2, 0x04000c0cu),
                               __builtin_amdgcn_perm(w1, w0, 0x0c0c0400u), 0x07060100u);
}

// Tokens per partial-sum chunk of the K column sum: at least 256 and large
// enough that no head has more than 64 chunks.
constexpr int ksum_chunk(int N) {
  return round_up((N + 63) / 64, 64) < 256 ? 256 : round_up((N + 63) / 64, 64);
}
// Most tokens one thread of the column-sum block adds up (16 threads per token
// row at d = 128, so 16 rows per pass; 32 at d = 64): the exactness of its
// fp64 running sums needs at most 8192.
constexpr int ksum_rows_per_thread(int N) { return ksum_chunk(N) / 16; }

// Byte offsets of the regions of a workspace. All offsets are 256-aligned.
struct Layout {
  int Npad = 0;      // rows per head of every padded operand
  int nchunk = 0;    // K column-sum chunks per head
  int chunk = 0;     // tokens per chunk
  size_t ksum = 0;   // int64 [BH, nchunk, d] partial column sums
  size_t kmean = 0;  // fp32 [BH, d]
  // INT8 modes
  size_t q_codes = 0, k_codes = 0;    // int8 [BH, Npad, d]
  size_t q_scales = 0, k_scales = 0;  // fp32 [BH, Npad] (enough for any block size)
  size_t vt = 0;                      // int8 V^T codes [BH, d, Npad], zero-padded (INT8 P.V only)
  size_t vscale = 0;                  // fp32 [BH, d] per-channel V scales (INT8 P.V)
  size_t vmax = 0;                    // uint32 [BH, nchunk, d] partial channel maxima of |V|
  // MXFP4 mode
  size_t q_fp4 = 0, k_fp4 = 0;    // uint8 [BH, Npad, d/2]
  size_t q_e8 = 0, k_e8 = 0;      // uint8 [BH, Npad, d/32]
  size_t vt_fp4 = 0, vt_e8 = 0;   // uint8 [BH, d, Npad/2] (E4M3 variant: [BH, d, Npad]), [BH, d, Npad/32]
  size_t total = 0;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Modes whose P.V runs in INT8 (SAGE_MODE_INT8_PV, SAGE_MODE_INT8_PV_PER_TOKEN).
inline bool mode_pv_int8(int mode_lo) { return mode_lo == 6 || mode_lo == 7; }

// mode_lo: SAGE_MODE_* without flags; attention=false gives the layout of the
// standalone quantization entry points (column sums and mean only).
inline Layout make_layout(long long BH, int N, int d, int mode_lo, bool attention) {
  Layout L;
  L.Npad = round_up(N, kRowPad);
  L.chunk = ksum_chunk(N);
  L.nchunk = (N + L.chunk - 1) / L.chunk;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off = align256(off + bytes); return at; };
  L.ksum = take(size_t(BH) * L.nchunk * d * 8);
  L.kmean = take(size_t(BH) * d * 4);
  if (attention) {
    const size_t rows = size_t(BH) * L.Npad;
    if (mode_lo == 2 || mode_lo == 5) {
      L.q_fp4 = take(rows * d / 2);
      L.k_fp4 = take(rows * d / 2);
      L.q_e8 = take(rows * d / 32);
      L.k_e8 = take(rows * d / 32);
      L.vt_fp4 = take(mode_lo == 5 ? rows * d : rows * d / 2);  // V^T codes: E2M1 (packed) or E4M3
      L.vt_e8 = take(rows * d / 32);
    } else if (mode_lo != 4) {  // (SAGE_MODE_FP16 reads Q, K and V as given)
      const bool pv8 = mode_pv_int8(mode_lo);
      L.q_codes = take(rows * d);
      L.k_codes = take(rows * d);
      L.q_scales = take(rows * 4);
      L.k_scales = take(rows * 4);
      if (pv8) {
        L.vt = take(rows * d);
        L.vscale = take(size_t(BH) * d * 4);
        L.vmax = take(size_t(BH) * L.nchunk * d * 4);
      }
    }
  } else {
    L.vmax = take(size_t(BH) * L.nchunk * d * 4);  // for sage_quant_v_int8
  }
  L.total = off;
  return L;
}

// ---------------------------------------------------------------------------
// Launchers (return the hipError_t of the launch). All take B*H as BH.
// ---------------------------------------------------------------------------

// K column sums (exact int64 fixed point) and the per-channel mean.
hipError_t launch_kmean(const void* k, long long* ksum, float* kmean_ws, float* kmean_out, int BH,
                        int N, int d, int chunk, int nchunk, hipStream_t s);

// One INT8 quantization job: `src` fp16 [BH, N, d] -> codes [BH, code_rows, d],
// scales [BH, nscale]; rows in [N, code_rows) are written as zero codes.
struct Int8Job {
  const void* src = nullptr;
  int8_t* codes = nullptr;
  float* scales = nullptr;
  const float* mu = nullptr;  // [BH, d] subtracted when non-null
  int blk = 64;
  int code_rows = 0;
  int nscale = 0;
  int ntile = 0;  // 128-row tiles per head to process
};
hipError_t launch_int8_quant(const Int8Job& j0, const Int8Job& j1, int BH, int N, int d, hipStream_t s);

// Per-channel INT8 V: channel maxima over chunks of `chunk` tokens into part
// [BH, nchunk, d], then scales [BH, d] and codes V^T [BH, d, ldv] (ldv a
// multiple of 16, tokens >= N zero).
hipError_t launch_v_int8(const void* v, unsigned* part, int8_t* codes, float* scales, int BH, int N, int ldv,
                         int d, int chunk, int nchunk, hipStream_t s);

// The whole prepare phase of the INT8 modes: K column sums and Q codes in one
// launch, the K mean, the K codes, and the INT8 V codes if used (fp16 V is
// read by the attention kernel as given).
struct PrepInt8 {
  const void* k = nullptr;
  const void* v = nullptr;
  long long* ksum = nullptr;   // int64 [BH, nchunk, d]
  float* kmean = nullptr;      // fp32 [BH, d], written when smooth
  int chunk = 0, nchunk = 0;
  bool smooth = true;
  Int8Job jq, jk;              // jk.mu = kmean when smooth
  void* vt = nullptr;          // INT8 V: V^T codes [BH, d, Npad]
  unsigned* vmax = nullptr;    // INT8 V: partial channel maxima [BH, nchunk, d]; null: no V work
  float* vscale = nullptr;     // INT8 V: scales [BH, d]
  int Npad = 0;
};
hipError_t launch_prepare_int8(const PrepInt8& P, int BH, int N, int d, hipStream_t s);

// MXFP4 quantization along channels: src fp16 [BH, N, d] -> fp4 [BH, rows, d/2],
// e8 [BH, rows, d/32]; rows in [N, rows) get zero codes and exponent byte 127.
struct MxRowJob {
  const void* src = nullptr;
  uint8_t* fp4 = nullptr;
  uint8_t* e8 = nullptr;
  const float* mu = nullptr;
  int rows = 0;
};
hipError_t launch_mx_rows(const MxRowJob& j0, const MxRowJob& j1, int BH, int N, int d, hipStream_t s);

// The whole prepare phase of the MXFP4 modes: K column sums, Q codes and V^T
// codes (E2M1, or E4M3 when v_fp8) in one launch, the K mean, then the K codes.
struct PrepMx {
  int BH = 0;
  const void* k = nullptr;
  const void* v = nullptr;
  long long* ksum = nullptr;
  float* kmean = nullptr;
  int chunk = 0, nchunk = 0;
  bool smooth = true;
  MxRowJob jq, jk;          // jk.mu = kmean when smooth
  uint8_t* vt = nullptr;    // V^T codes [BH, d, Nv/2] (E2M1) or [BH, d, Nv] (E4M3)
  uint8_t* vte8 = nullptr;  // [BH, d, Nv/32]
  int Nv = 0;
  bool v_fp8 = false;
};
hipError_t launch_prepare_mx(const PrepMx& P, int N, int d, hipStream_t s);

// MXFP4 quantization of V along tokens: -> fp4 [BH, d, Nv/2], e8 [BH, d, Nv/32]
// (Nv a multiple of 32, tokens >= N are zeros).
hipError_t launch_mx_vt(const void* v, uint8_t* fp4, uint8_t* e8, int BH, int N, int Nv, int d, hipStream_t s);
// The same with MX-FP8 (E4M3, one byte per element) codes: fp8 [BH, d, Nv].
hipError_t launch_mx_vt8(const void* v, uint8_t* fp8, uint8_t* e8, int BH, int N, int Nv, int d, hipStream_t s);

// Fused attention from a prepared workspace.
struct AttnArgs {
  int BH = 0, N = 0, Npad = 0, d = 0;
  bool causal = false;
  float sl2 = 0.f;  // sm_scale * log2(e)
  int mode = 0;     // SAGE_MODE_* (no flags)
  void* out = nullptr;
  float* lse = nullptr;  // fp32 [BH, N] row log-sum-exp (natural log), fp16-P modes only; may be null
  bool qin = false;      // per-block INT8 modes: q is the caller's fp16 Q, quantized in the kernel's prologue
};
// q, k: INT8 codes (padded to Npad rows) with scales qs, ks; or, for
// SAGE_MODE_FP16, the caller's fp16 Q and K [BH, N, d] (qs, ks unused); with
// a.qin (modes 0 and 1), q is the caller's fp16 Q [BH, N, d] and qs unused.
// v: the caller's fp16 V [BH, N, d], or for the INT8 P.V modes int8 V^T codes
// [BH, d, Npad] with per-channel scales vs [BH, d] (unused otherwise).
hipError_t launch_attn_int8(const AttnArgs& a, const void* q, const void* k, const void* v,
                            const float* qs, const float* ks, const float* vs, hipStream_t s);
// The INT8 attention kernel (non-causal, modes 0, 1, 3) with a copy of the
// integer scores of key tile dkt for query tile dqt of head dbh into dump
// (int32 [256, 64], query-major).
hipError_t launch_attn_int8_dump(const AttnArgs& a, const void* q, const void* k, const void* v,
                                 const float* qs, const float* ks, int* dump, int dbh, int dqt, int dkt,
                                 hipStream_t s);
// v4 holds E2M1 V^T codes, or E4M3 ones for SAGE_MODE_MXFP4_FP8PV (a.mode 5,
// where P is quantized to MX-FP8 as well).
hipError_t launch_attn_mxfp4(const AttnArgs& a, const uint8_t* q4, const uint8_t* qe,
                             const uint8_t* k4, const uint8_t* ke, const uint8_t* v4,
                             const uint8_t* ve, hipStream_t s);

// Workspace of the backward pass: the forward layout of its mode (Q and K_s
// codes and scales, K sums and mean) followed by the backward's own regions.
struct BwdLayout {
  Layout f;
  size_t qt = 0, kt = 0, gt = 0;   // int8 transposed codes [BH, d, Npad] of Q, K_s, dO
  size_t vc = 0, gc = 0;           // int8 codes [BH, Npad, d] of V (per token) and dO (per 64 rows)
  size_t vs = 0, gs = 0;           // fp32 scales [BH, Npad] and [BH, Npad / 64]
  size_t ld = 0;                   // float2 (L2, D) per row [BH, Npad]
  size_t total = 0;
};
inline BwdLayout make_bwd_layout(long long BH, int N, int d, int mode_lo) {
  BwdLayout L;
  L.f = make_layout(BH, N, d, mode_lo, true);
  size_t off = L.f.total;
  auto take = [&](size_t bytes) { size_t at = off; off = align256(off + bytes); return at; };
  const size_t rows = size_t(BH) * L.f.Npad;
  L.qt = take(rows * d);
  L.kt = take(rows * d);
  L.gt = take(rows * d);
  L.vc = take(rows * d);
  L.gc = take(rows * d);
  // vs and ld are read in 1 KiB tile loads that run up to 768 bytes past a
  // head's last row (the surplus is unused): 1 KiB of slack keeps even the
  // last head's reads inside the workspace
  L.vs = take(rows * 4 + 1024);
  L.gs = take(rows / 64 * 4);
  L.ld = take(rows * 8 + 1024);
  L.total = off;
  return L;
}

// The backward pass after its quantization: row terms, transposed codes, then
// the dK/dV and dQ kernels.
struct BwdLaunch {
  int BH = 0, N = 0, Npad = 0, d = 0, qblk = 128;
  bool causal = false;
  float sl2 = 0.f, sm = 0.f;
  const _Float16* o = nullptr;     // forward output [BH, N, d]
  const _Float16* dout = nullptr;  // dO [BH, N, d]
  const float* lse = nullptr;      // [BH, N]
  const int8_t* qc = nullptr; const int8_t* kc = nullptr; const int8_t* vc = nullptr; const int8_t* gc = nullptr;
  int8_t* qt = nullptr; int8_t* kt = nullptr; int8_t* gt = nullptr;
  const float* qs = nullptr; const float* ks = nullptr; const float* vs = nullptr; const float* gs = nullptr;
  float2* ld = nullptr;
  float* dq = nullptr; float* dk = nullptr; float* dv = nullptr;  // fp32 [BH, N, d]
};
hipError_t launch_attn_bwd(const BwdLaunch& b, hipStream_t s);

// One wave spins for `cycles` shader clocks and writes to out[0..1] the
// cycles counted and the device wall-clock ticks over the same interval.
hipError_t launch_clock_probe(long long cycles, long long* out, hipStream_t s);

}  // namespace sage
