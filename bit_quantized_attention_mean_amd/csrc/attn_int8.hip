// Fused INT8 attention kernel for gfx950 (CDNA4).
//
// Computes, per head, O = softmax(sm_scale * dequant(Qc Kc^T)) V from the
// INT8 codes and per-block scales of Q and the mean-smoothed K, with P and V
// in FP16 for P.V (SageAttention page, "Approach" and summary paragraph) and
// the softmax taken online over key tiles, FlashAttention-2 style ("Experimental
// setup: builds on FlashAttention-2 ... online softmax").
//
// Work decomposition
//   * one workgroup = 8 waves = 256 query rows of one head, in two groups of
//     4 waves (128 rows each; one Q scale block). Waves w and w + 4 share a
//     SIMD. The groups alternate phases ("ping-pong"): while one group runs
//     its matrix ops for a key tile (P.V of the previous tile, then the scores
//     of this one), the other runs its softmax on the VALU; a workgroup
//     barrier separates the phases. 64-key tiles of K and V are staged in
//     LDS (double-buffered) and shared by all 8 waves. Instances whose VALU
//     work outweighs their matrix work more (per-token scores, INT8 P.V) use
//     4-wave workgroups of 128 rows instead, several per CU, each wave doing
//     its matrix ops and softmax in turn (attn_pingpong below).
//   * scores are computed transposed, S^T = K Q^T, on v_mfma_i32_32x32x32_i8:
//     in the 32x32 accumulator layout every lane owns one query column
//     (lane % 32) and 16 key rows, so the row max and row sum of the softmax
//     are in-lane reductions plus one swap between lanes l and l + 32.
//   * K rows are placed in LDS in a permuted order so that, after the score
//     MFMA, lane group g = lane / 32 holds exactly keys g*32 .. g*32+31 of the
//     tile, in order. Those values, rounded to fp16, are already the B operand
//     of O^T = V^T P^T on v_mfma_f32_32x32x16_f16: no shuffle and no LDS round
//     trip for P.
//   * fp16 V is read as the caller gave it ([N, d] per head, 64 key rows of
//     d channels per tile, rows past N read as zeros by the buffer's range
//     check): the V^T operand comes from gfx950's transposing LDS read
//     (ds_read_b64_tr_b16, 4 keys x 16 channels per 16 lanes), so no
//     transposed copy of V is written to HBM and read back.
//   * O^T accumulates in fp32 (CDNA4's FP16 matrix op accumulates in FP32; the
//     page reports no accuracy difference between FP16 and FP32 accumulators).
//   * softmax in base 2: the row max is taken on the integer scores, then one
//     fma per score applies s_q * s_k * sm_scale * log2(e) and subtracts the
//     reference max; P = exp2(.) on v_exp_f32; the reference max moves lazily
//     (see kRefSlack); the row sum adds the fp16 P pairwise on v_dot2_f32_f16.
//   * causal: key tiles wholly above the workgroup's last query are skipped;
//     masking runs only on tiles that cross the diagonal or the ragged tail.
//   * INT8 P.V variant (the SageAttention page's "Measured effects" ablation
//     with P and V in INT8; the faster kernel its "Approach" picks per layer where
//     accuracy allows): V^T arrives as INT8 codes with one scale per channel,
//     P is formed against the exact running max (so P <= 1) and converted to
//     the integer round(127 P) in one v_cvt_pk_u8_f32 per value, and O^T
//     accumulates exactly in int32 on v_mfma_i32_32x32x32_i8 (half the matrix
//     ops of the FP16 form). There is no INT8 matrix op with a float
//     accumulator, and an int32 sum cannot be rescaled by alpha without
//     rounding; so the int32 sum only ever holds weights formed against one
//     reference max, and when a row max moves it is flushed into an fp32 O^T
//     kept against a fixed per-row reference m0 (O_f += float(sum) *
//     2^(m_old - m0)), the next P.V starting a fresh int32 sum. The row sum
//     adds the integer weights on v_dot4_i32_i8, and the epilogue combines
//     the two accumulators and applies the channel scales.
#include "sage_internal.h"

#include <limits.h>
#include <math.h>

namespace sage {

namespace {

// The fp16-P kernels move a row's softmax reference max only when a tile's row
// max exceeds it by more than this (log2 units), so P <= 2^8 and the O rescale
// is skipped on most tiles: the same softmax, with P rounded to fp16 at a point
// a power of at most 2^8 away from the running max's (a relative difference of
// at most half an fp16 ulp per weight). The INT8 P.V variant forms P against
// the running max exactly (slack 0): its weights round(127 P) are the method's.
constexpr float kRefSlack = 8.0f;
// INT8 P.V: the fp32 accumulator's reference m0 is moved up to the current
// one when the factor 2^(m - m0) would exceed 2^kRebase (fp32 range guard).
constexpr float kRebase = 32.0f;

// Two of gfx950's transposing LDS reads (ds_read_b64_tr_b16), at p and at
// p + stride, as one 8-value fp16 operand.
__device__ __forceinline__ v8h lds_read_tr_v8h(const unsigned char* p, int stride) {
  typedef __fp16 h4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
  typedef __attribute__((address_space(3))) h4 lds_h4;
  typedef unsigned u2 __attribute__((ext_vector_type(2)));
  const u2 a = __builtin_bit_cast(u2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h4*)(p)));
  const u2 b = __builtin_bit_cast(u2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h4*)(p + stride)));
  return __builtin_bit_cast(v8h, v4u{a[0], a[1], b[0], b[1]});
}

// Waits until at most n (0..7, wave-uniform) of this wave's vector memory
// operations are outstanding (s_waitcnt with only the vmcnt field set).
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0xF70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0xF71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0xF72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0xF73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0xF74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0xF75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0xF76); break;
    default: __builtin_amdgcn_s_waitcnt(0xF77); break;
  }
}

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// lds + 16 l (buffer_load_dwordx4 with an LDS destination; the LDS address
// is wave-uniform). Kept out of the kernel template: the host-side pass of a
// template instantiation that names this builtin silently drops the kernel.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// Key tile row held in LDS row r: the inverse of lds_row_of_key below.
__device__ __forceinline__ int key_of_lds_row(int r) {
  const int t = r >> 5, rem = r & 31;
  return ((rem >> 2) & 1) * 32 + t * 16 + ((rem >> 3) << 2) + (rem & 3);
}

// log2(127): exp2(x + log2(127)) = 127 * exp2(x), the integer P weight's scale.
constexpr float kLog2_127 = 6.98868468677216585f;

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
constexpr v2h kOnes2 = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};

// LDS row (0..63) holding key k of a 64-key tile. Row t*32 + r feeds row r of
// score MFMA t; its accumulator register i of lane group g is row
// (i/4)*8 + g*4 + i%4, and the placement below makes that key g*32 + t*16 + i.
__device__ __forceinline__ int lds_row_of_key(int k) {
  const int g = k >> 5, t = (k >> 4) & 1, i = k & 15;
  return t * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
}

// Max of the 32 scores a lane holds, as four independent chains of eight.
__device__ __forceinline__ int max32_i(const v16i& a, const v16i& b) {
  int c0 = max(a[0], a[1]), c1 = max(a[8], a[9]), c2 = max(b[0], b[1]), c3 = max(b[8], b[9]);
#pragma unroll
  for (int i = 2; i < 8; ++i) {
    c0 = max(c0, a[i]); c1 = max(c1, a[8 + i]); c2 = max(c2, b[i]); c3 = max(c3, b[8 + i]);
  }
  return max(max(c0, c1), max(c2, c3));
}
__device__ __forceinline__ float max32_f(const v16i& a, const v16i& b) {
  float c0 = fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
  float c1 = fmaxf(__int_as_float(a[8]), __int_as_float(a[9]));
  float c2 = fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
  float c3 = fmaxf(__int_as_float(b[8]), __int_as_float(b[9]));
#pragma unroll
  for (int i = 2; i < 8; ++i) {
    c0 = fmaxf(c0, __int_as_float(a[i])); c1 = fmaxf(c1, __int_as_float(a[8 + i]));
    c2 = fmaxf(c2, __int_as_float(b[i])); c3 = fmaxf(c3, __int_as_float(b[8 + i]));
  }
  return fmaxf(fmaxf(c0, c1), fmaxf(c2, c3));
}

// The next float below x (x finite).
__device__ __forceinline__ float below_ulp(float x) {
  if (x == 0.f) return -0x1p-149f;
  return __uint_as_float(__float_as_uint(x) + (x > 0.f ? 0xffffffffu : 1u));
}

// Combines a per-lane value with the one in lane l ^ 32 (same query column).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ int pair_max_i(int x) {
  const auto r = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(x), static_cast<unsigned>(x), false, false);
  return max(static_cast<int>(r[0]), static_cast<int>(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup id -> (head, query tile). Workgroups are dispatched round-robin
// over the 8 XCDs (id % 8); each XCD is given a contiguous range of heads so
// that K and V of a head stay in one XCD's L2. Causal grids run the longest
// query tiles (most key tiles) first.
__device__ __forceinline__ void map_workgroup(int bid, int BH, int nqt, bool causal, int& bh, int& qt) {
  if (BH % 8 == 0) {
    const int x = bid & 7, r = bid >> 3, hpx = BH >> 3;
    if (causal) {
      bh = x * hpx + r % hpx;
      qt = nqt - 1 - r / hpx;
    } else {
      bh = x * hpx + r / nqt;
      qt = r % nqt;
    }
  } else {
    bh = bid / nqt;
    qt = bid % nqt;
    if (causal) qt = nqt - 1 - qt;
  }
}

}  // namespace

// Score variants of the kernel: INT8 codes with one scale per (query block,
// key tile), INT8 codes with per-token scales, or unquantized fp16 Q and K on
// the FP16 matrix op (the FlashAttention-style baseline of the same design).
constexpr int kScoresInt8Block = 0, kScoresInt8Token = 1, kScoresF16 = 2;

// Schedule of a kernel instance. The two-group ping-pong (8 waves, 256 query
// rows per workgroup) overlaps one group's matrix ops with the other's
// softmax. Where the VALU work outweighs the matrix work more (per-token
// scores, INT8 P.V) the matrix pipe would idle in it, so those instances run
// 4 waves (128 rows) that do their matrix ops and softmax in turn, three
// workgroups per CU at d = 64 and two at d = 128, the waves of different
// workgroups filling each other's gaps (measured +17 to +25% at d = 64, +1 to
// +9% at d = 128; the plain INT8 modes at d = 64 measured 0.8% slower that way
// and keep the ping-pong). The per-block INT8 P.V instance at d = 64 is only
// bounded to two per CU: it needs 181 registers, and squeezed into the 168 of
// three per CU it spilled 16 and ran 3-6% slower. (The bound is a minimum;
// instances that fit in 168 registers still run three per CU.)
constexpr bool attn_pingpong(int D, int SM, bool PV8, bool DUMP) {
  return DUMP || SM == kScoresF16 || (SM == kScoresInt8Block && !PV8);
}

// DUMP: a test instance that also copies the integer scores of key tile dkt,
// as the score matrix op produced them, for the 256 queries of query tile dqt
// of head dbh into dump (int32 [256, 64], query-major).
template <int D, bool CAUSAL, int SM, bool PV8, bool DUMP = false>
__global__ __launch_bounds__(attn_pingpong(D, SM, PV8, DUMP) ? 512 : 256,
                             attn_pingpong(D, SM, PV8, DUMP) ? 1 : (D == 64 && !PV8 ? 3 : 2)) void attn_int8_kernel(
    const void* __restrict__ qsrc, const void* __restrict__ ksrc, const void* __restrict__ vsrc,
    const float* __restrict__ qs, const float* __restrict__ ks, const float* __restrict__ vsc,
    _Float16* __restrict__ out, int N, int Npad, int qblk, float sl2, int BH, int* __restrict__ dump = nullptr,
    int dbh = 0, int dqt = 0, int dkt = 0, float* __restrict__ lse = nullptr, int qin = 0) {
  constexpr bool PERTOK = SM == kScoresInt8Token;
  constexpr bool F16 = SM == kScoresF16;
  static_assert(!(PV8 && F16), "INT8 P.V goes with INT8 scores");
  static_assert(!(DUMP && F16), "the score dump is for the integer scores");
  constexpr float SLACK = PV8 ? 0.f : kRefSlack;
  constexpr float PLOG = PV8 ? kLog2_127 : 0.f;  // P (fp16 form) or 127 P (INT8 form)
  constexpr int EB = F16 ? 2 : 1;        // bytes per Q / K element
  constexpr int NC = D / 32;             // 32-channel tiles of O^T
  constexpr int NQF = F16 ? D / 16 : D / 32;  // score matrix ops per 32 keys (16 bytes of Q each)
  constexpr bool PP = attn_pingpong(D, SM, PV8, DUMP);
  // The INT8 ping-pong instances load tiles straight into LDS (buffer loads
  // with an LDS destination, 1 KiB per wave instruction) into three stages,
  // two tiles ahead, with unpadded rows whose 16-byte chunks are permuted
  // within the row (XOR swizzle) so the matrix ops' LDS reads stay free of
  // bank conflicts; the others stage tiles through registers into two
  // buffers of padded rows.
  constexpr bool DMA = PP && !F16;
  // With qin (a runtime flag), the per-block INT8 ping-pong instances read the
  // caller's fp16 Q ([N, d] per head) and quantize it in their prologue, with
  // the arithmetic of the quantization kernel (block maximum over the qblk
  // rows of the Q block, s = fp32(a / 127), correctly rounded quotients), so
  // the codes are the ones sage_quant_qk writes. Its fp16 loads are issued
  // before, and its arithmetic after, the first tile loads.
  constexpr bool QIN = DMA && SM == kScoresInt8Block && !DUMP;
  // K in LDS: 64 key rows of d codes (fp16: 2d bytes). The rows are unpadded
  // with XOR-swizzled chunks (below) in the LDS-loaded instances and in the
  // register-staged per-token ones at d = 64, where padded 80-byte rows left
  // the tile stores 2-way bank-conflicted. Elsewhere K rows keep 16 bytes of
  // padding: at d = 128 the padded stores conflict on one 16-byte unit only,
  // and the INT8 P.V instances have no registers left for the swizzle's
  // per-lane read offsets.
  constexpr bool KSWZ = DMA || (!F16 && !PV8 && D == 64);
  constexpr int KROW = KSWZ ? D * EB : D * EB + 16;   // LDS bytes per K row
  // V in LDS: fp16 V as given, 64 key rows of d channels (without DMA +64
  // bytes, so that the 4 rows x 64 bytes of one transposing read fall in
  // distinct banks; with DMA the 64-byte segments are swizzled instead), or
  // the INT8 V^T codes, d channel rows of 64 keys (+16 bytes).
  constexpr bool VRM = !PV8;
  constexpr int VROW = VRM ? (DMA ? D * 2 : D * 2 + 64) : kKTile + 16;  // LDS bytes per V row
  // swizzles of the DMA layouts: K row r keeps data chunk q at chunk
  // q ^ kswz(r); V row r keeps data segment s (64 bytes = 32 channels) at
  // segment s ^ vswz(r). kswz(r) = (r >> KSH) & (KCPR - 1) makes any 16
  // consecutive rows put a given chunk in distinct banks; vswz(r) = (r >> VSH)
  // & (VSEG - 1) does the same for the 4 rows of a transposing read.
  constexpr int KCPR = D * EB / 16;                  // 16-byte chunks per K row
  constexpr int KSH = KCPR == 8 ? 1 : (KCPR == 4 ? 2 : 0);
  constexpr int VSEG = D * 2 / 64;                   // 64-byte segments per V row
  constexpr int VSH = VSEG == 4 ? 0 : 1;
  constexpr int KT_BYTES = kKTile * KROW;
  constexpr int VT_BYTES = (VRM ? kKTile : D) * VROW;
  constexpr int KB0 = 0, KB1 = KT_BYTES, VB0 = 2 * KT_BYTES, VB1 = 2 * KT_BYTES + VT_BYTES;
  constexpr int KCHN = kKTile * D * EB / 16;  // 16-byte chunks of a K tile
  constexpr int RPV = PV8 ? 2 : 4;       // P.V matrix ops per 32-channel tile
  constexpr int VRD = VRM ? 2 : 1;       // LDS reads per P.V A operand
  constexpr int NTH = PP ? 512 : 256;          // threads per workgroup
  constexpr int WGQ = PP ? kWGQ : kWGQ / 2;    // query rows per workgroup
  constexpr int KPT = (KCHN + NTH - 1) / NTH;
  constexpr int VCPR = VRM ? D * 2 / 16 : kKTile / 16;  // 16-byte chunks per V row in global memory
  constexpr int VCHN = (VRM ? kKTile : D) * VCPR;      // 16-byte chunks of a V tile
  constexpr int VPT = (VCHN + NTH - 1) / NTH;
  // register-staged tiles: two K and two V buffers in one array; LDS-loaded
  // tiles: three stages of each, separate arrays (the compiler then tells
  // the stages apart and does not wait for a stage's loads before reading
  // another one)
  __shared__ __attribute__((aligned(16))) unsigned char smem[DMA ? 16 : 2 * KT_BYTES + 2 * VT_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char smk0[DMA ? KT_BYTES : 16];
  __shared__ __attribute__((aligned(16))) unsigned char smk1[DMA ? KT_BYTES : 16];
  __shared__ __attribute__((aligned(16))) unsigned char smk2[DMA ? KT_BYTES : 16];
  __shared__ __attribute__((aligned(16))) unsigned char smv0[DMA ? VT_BYTES : 16];
  __shared__ __attribute__((aligned(16))) unsigned char smv1[DMA ? VT_BYTES : 16];
  __shared__ __attribute__((aligned(16))) unsigned char smv2[DMA ? VT_BYTES : 16];

  const int nqt = Npad / WGQ;
  int bh, qt;
  map_workgroup(blockIdx.x, BH, nqt, CAUSAL, bh, qt);
  const int q0 = qt * WGQ;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = PP ? wave >> 2 : 0;            // 0 or 1: which half of the ping-pong
  const int wrow0 = q0 + grp * 128 + (wave & 3) * 32;   // first query row of this wave
  const int qrow = wrow0 + l32;

  // Q of this lane's query (16 bytes per score matrix op: 16 INT8 codes, or
  // 8 fp16 values): the B operand of the score MFMAs, kept in registers. The
  // INT8 codes are zero-padded to Npad rows; fp16 Q is read as given, with
  // zeros for rows >= N.
  v4i qf[NQF];
  uint4 qraw[QIN ? 2 * NQF : 1];   // fp16 Q of this lane: channels c*32 + g*16 .. +15 in qraw[2c], qraw[2c+1]
  if (QIN && qin) {
    const bool live = qrow < N;
    const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(qsrc) +
                                                     (static_cast<size_t>(bh) * N + (live ? qrow : 0)) * D + g * 16);
#pragma unroll
    for (int c = 0; c < NQF; ++c) {
      qraw[2 * c] = live ? qp[c * 4] : make_uint4(0, 0, 0, 0);
      qraw[2 * c + 1] = live ? qp[c * 4 + 1] : make_uint4(0, 0, 0, 0);
    }
  } else if (F16) {
    const bool live = qrow < N;
    const unsigned char* qp = static_cast<const unsigned char*>(qsrc) +
                              (static_cast<size_t>(bh) * N + (live ? qrow : 0)) * D * 2 + g * 16;
#pragma unroll
    for (int c = 0; c < NQF; ++c) {
      qf[c] = v4i{0, 0, 0, 0};
      if (live) qf[c] = *reinterpret_cast<const v4i*>(qp + c * 32);
    }
  } else {
    const int8_t* qp = static_cast<const int8_t*>(qsrc) + (static_cast<size_t>(bh) * Npad + qrow) * D + g * 16;
#pragma unroll
    for (int c = 0; c < NQF; ++c) qf[c] = *reinterpret_cast<const v4i*>(qp + c * 32);
  }
  // Q scale: one per block of qblk rows (a wave never straddles two), or per row.
  // K scale: one per 64-key block (= one key tile), or one per key.
  float sq = 1.f;
  const float* ksh = nullptr;
  if (!F16) {
    const int nqs = Npad / qblk;
    if (!(QIN && qin)) sq = qs[static_cast<size_t>(bh) * nqs + (PERTOK ? qrow : wrow0 / qblk)];
    const int nks = PERTOK ? Npad : Npad / kKTile;
    ksh = ks + static_cast<size_t>(bh) * nks;
  }

  int nkt = (N + kKTile - 1) / kKTile;
  if (CAUSAL) nkt = min(nkt, (q0 + WGQ) / kKTile);

  // K: INT8 codes zero-padded to Npad rows, or fp16 K as given ([N, d] per head).
  const unsigned char* kbase = static_cast<const unsigned char*>(ksrc) +
                               static_cast<size_t>(bh) * (F16 ? N : Npad) * D * EB;
  // V: fp16 as given ([N, d] per head), or INT8 V^T codes zero-padded to Npad keys.
  const unsigned char* vbase = static_cast<const unsigned char*>(vsrc) + static_cast<size_t>(bh) * (VRM ? N * 2 : Npad) * D;
  // d = 128: the tile loads are buffer loads (per-lane offset fixed for the
  // loop, the tile's offset in a scalar register; +1% at d = 128, -1.4% at
  // d = 64, where plain global loads are kept)
  const auto rk = buffer_rsrc(kbase, static_cast<unsigned>(F16 ? N : Npad) * (D * EB));
  const auto rv = buffer_rsrc(vbase, static_cast<unsigned>(D) * (VRM ? N * 2 : Npad));

  // Loading: every thread moves at most KPT 16-byte K chunks and VPT V^T chunks
  // per tile, global -> registers at the start of a period, registers -> LDS
  // at its end. K rows go to their permuted LDS rows.
  const bool kload_last = (tid + NTH * (KPT - 1)) < KCHN;
  int kg[KPT], kl[KPT], krw[KPT];
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const int i = tid + NTH * u, row = i / (D * EB / 16), col = i % (D * EB / 16);
    kg[u] = row * D * EB + col * 16;
    const int lr = lds_row_of_key(row);
    kl[u] = lr * KROW + (KSWZ ? (col ^ ((lr >> KSH) & (KCPR - 1))) : col) * 16;
    krw[u] = row;
  }
  int vg[VPT], vls[VPT];
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int i = tid + NTH * u, row = i / VCPR, col = i % VCPR;
    vg[u] = row * (VRM ? D * 2 : Npad) + col * 16;
    vls[u] = row * VROW + col * 16;
  }
  const bool vload_last = (tid + NTH * (VPT - 1)) < VCHN;
  unsigned kr[4 * KPT], vr[4 * VPT];
  const int ka = l32 * KROW + g * 16;   // score A operand: K row l32 of each 32-key half
  // with DMA: the A operand of score matrix op c (data chunk 2c + g of row
  // l32; the swizzle of row t * 32 + l32 is that of row l32)
  int kc[NQF];
#pragma unroll
  for (int c = 0; c < NQF; ++c) kc[c] = l32 * KROW + (((2 * c + g) ^ ((l32 >> KSH) & (KCPR - 1))) * 16);
  // P.V A operand (channel l32 of a 32-channel tile, keys g*32 + 8c .. +7):
  // INT8 V^T row l32; or, from row-major fp16 V, two transposing reads of 4
  // keys each. In such a read, lane i of each 16-lane group receives element
  // i % 4 of the 8 bytes addressed by lane 4j + i / 4 as its element j; so the
  // lane at position r of its group addresses key row r / 4 and channels
  // 16 h + 4 (r % 4) .. +3 (h: which half of the 32 channels), and every lane
  // receives channel 16 h + (its position) for 4 consecutive keys.
  const int va = VRM ? (g * 32 + ((lane & 15) >> 2)) * VROW + ((lane >> 4) & 1) * 32 + (lane & 3) * 8
                     : l32 * VROW + g * 32;
  // with DMA: the same read for 32-channel tile dt, in its swizzled segment
  // (the rows this lane addresses, g*32 + 8c + (lane & 15)/4 (+4), share the
  // swizzle of row (lane & 15)/4)
  int vdt[NC];
#pragma unroll
  for (int dt = 0; dt < NC; ++dt)
    vdt[dt] = (g * 32 + ((lane & 15) >> 2)) * VROW + ((dt ^ ((((lane & 15) >> 2) >> VSH) & (VSEG - 1))) * 64) +
              ((lane >> 4) & 1) * 32 + (lane & 3) * 8;

  v16f o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[c][i] = 0.f;
  float m = -INFINITY, l = 0.f, alpha = 1.f;
  // INT8 P.V: fp32 O^T against reference m0 (of), and the reference under
  // which the int32 sum in o was accumulated (mpv)
  v16f of[PV8 ? NC : 1];
#pragma unroll
  for (int c = 0; c < (PV8 ? NC : 1); ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) of[c][i] = 0.f;
  float m0 = 0.f, mpv = -INFINITY;
  v16i s[2];
  v8h pf[4];   // fp16 P, keys g*32 + c*8 .. +7 in pf[c]
  v4i pq[2];   // INT8 form: round(127 P), keys g*32 + u*16 .. +15 in pq[u]

#define SAGE_LOAD_K(J_)                                                                          \
  _Pragma("unroll") for (int u = 0; u < KPT; ++u) {                                              \
    if (u < KPT - 1 || kload_last) {                                                             \
      v4u t_ = {0u, 0u, 0u, 0u};                                                                 \
      /* INT8 codes are padded; fp16 K rows >= N read as zeros (their scores are masked) */     \
      if (!F16 || (J_) * kKTile + krw[u] < N) {                                                  \
        if (D == 128)                                                                            \
          t_ = __builtin_amdgcn_raw_buffer_load_b128(rk, kg[u], (J_) * (kKTile * D * EB), 0);    \
        else                                                                                     \
          t_ = *reinterpret_cast<const v4u*>(kbase + static_cast<size_t>(J_) * kKTile * D * EB + kg[u]); \
      }                                                                                          \
      kr[4 * u] = t_[0]; kr[4 * u + 1] = t_[1]; kr[4 * u + 2] = t_[2]; kr[4 * u + 3] = t_[3];   \
    }                                                                                            \
  }
#define SAGE_LOAD_V(J_)                                                                          \
  _Pragma("unroll") for (int u = 0; u < VPT; ++u) {                                              \
    if (u < VPT - 1 || vload_last) {                                                             \
      v4u t_ = {0u, 0u, 0u, 0u};                                                                 \
      /* INT8 V^T codes are padded; fp16 V rows >= N lie past the buffer's range, */            \
      /* which reads them as zeros (their P is 0) without a branch */                           \
      if (VRM) {                                                                                 \
        t_ = __builtin_amdgcn_raw_buffer_load_b128(rv, vg[u] + (J_) * (kKTile * D * 2), 0, 0);   \
      } else {                                                                                   \
        t_ = (D == 128) ? __builtin_amdgcn_raw_buffer_load_b128(rv, vg[u], (J_) * kKTile, 0)     \
                        : *reinterpret_cast<const v4u*>(vbase + (J_) * kKTile + vg[u]);          \
      }                                                                                          \
      vr[4 * u] = t_[0]; vr[4 * u + 1] = t_[1]; vr[4 * u + 2] = t_[2]; vr[4 * u + 3] = t_[3];   \
    }                                                                                            \
  }
#define SAGE_STORE_K(KB_)                                                                        \
  _Pragma("unroll") for (int u = 0; u < KPT; ++u) {                                              \
    if (u < KPT - 1 || kload_last)                                                               \
      *reinterpret_cast<uint4*>(smem + (KB_) + kl[u]) =                                          \
          make_uint4(kr[4 * u], kr[4 * u + 1], kr[4 * u + 2], kr[4 * u + 3]);                    \
  }
#define SAGE_STORE_V(VB_)                                                                        \
  _Pragma("unroll") for (int u = 0; u < VPT; ++u) {                                              \
    if (u < VPT - 1 || vload_last)                                                               \
      *reinterpret_cast<uint4*>(smem + (VB_) + vls[u]) =                                         \
          make_uint4(vr[4 * u], vr[4 * u + 1], vr[4 * u + 2], vr[4 * u + 3]);                    \
  }

  // S^T = K Q^T for key tile J_ from the K buffer KB_: INT8 MFMA (exact int32)
  // or, for fp16 Q and K, the FP16 MFMA (fp32 accumulation; the fp32 bits are
  // kept in the same registers). Both read 16 bytes of K per lane and matrix op
  // at the same LDS offsets. All K operands are read up front so the matrix ops
  // issue back to back.
#define SAGE_SCORES(KB_)                                                                         \
  do {                                                                                           \
    v4i ka_[2 * NQF];                                                                            \
    _Pragma("unroll") for (int t = 0; t < 2; ++t)                                                \
      _Pragma("unroll") for (int c = 0; c < NQF; ++c)                                            \
        ka_[t * NQF + c] = *reinterpret_cast<const v4i*>((KB_) + (KSWZ ? kc[c] : ka + c * 32) + t * 32 * KROW); \
    _Pragma("unroll") for (int t = 0; t < 2; ++t) {                                              \
      _Pragma("unroll") for (int i = 0; i < 16; ++i) s[t][i] = 0;                                \
      _Pragma("unroll") for (int c = 0; c < NQF; ++c) {                                          \
        if (F16)                                                                                 \
          s[t] = __builtin_bit_cast(v16i, __builtin_amdgcn_mfma_f32_32x32x16_f16(                \
                     __builtin_bit_cast(v8h, ka_[t * NQF + c]), __builtin_bit_cast(v8h, qf[c]),  \
                     __builtin_bit_cast(v16f, s[t]), 0, 0, 0));                                  \
        else                                                                                     \
          s[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka_[t * NQF + c], qf[c], s[t], 0, 0, 0); \
      }                                                                                          \
    }                                                                                            \
    /* issue order: 4 LDS reads ahead, then one read per matrix op */                           \
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);                                           \
    _Pragma("unroll") for (int u = 0; u < 2 * NQF - 4; ++u) {                                    \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);                                         \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);                                         \
    }                                                                                            \
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);                                           \
  } while (0)

  // O^T = alpha * O^T + V^T P^T from the V buffer VB_ (FP16 MFMA, FP32
  // accumulation). The rescale by the last softmax's alpha is done here, in the
  // matrix phase, so the softmax phase never touches the O registers. In the
  // INT8 form O^T holds int32 sums (in the same registers), each 32-channel
  // tile takes two INT8 matrix ops (32 keys each) instead of four, and a moved
  // max flushes the int32 sums into the fp32 accumulator (of) instead of
  // rescaling them: the first matrix op of each tile then starts from zero.
#define SAGE_VA(VB_, DT_, C_)                                                                    \
  (VRM ? lds_read_tr_v8h((VB_) + (DMA ? vdt[DT_] : va + (DT_) * 64) + (C_) * 8 * VROW, 4 * VROW)    \
       : *reinterpret_cast<const v8h*>((VB_) + va + (DT_) * 32 * VROW + (C_) * 16))
#define SAGE_PV_MMA(VB_, Z_)                                                                     \
  do {                                                                                           \
    v8h va_[2][RPV];                                                                             \
    _Pragma("unroll") for (int c = 0; c < RPV; ++c)                                              \
      va_[0][c] = SAGE_VA(VB_, 0, c);                                                            \
    _Pragma("unroll") for (int dt = 0; dt < NC; ++dt) {                                          \
      if (dt + 1 < NC) {                                                                         \
        _Pragma("unroll") for (int c = 0; c < RPV; ++c) va_[(dt + 1) & 1][c] = SAGE_VA(VB_, dt + 1, c); \
      }                                                                                          \
      _Pragma("unroll") for (int c = 0; c < RPV; ++c) {                                          \
        if (PV8) {                                                                               \
          const v16i z_ = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};                      \
          o[dt] = __builtin_bit_cast(v16f, __builtin_amdgcn_mfma_i32_32x32x32_i8(                \
                      __builtin_bit_cast(v4i, va_[dt & 1][c]), pq[c],                            \
                      ((Z_) && c == 0) ? z_ : __builtin_bit_cast(v16i, o[dt]), 0, 0, 0));        \
        } else {                                                                                 \
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va_[dt & 1][c], pf[c], o[dt], 0, 0, 0); \
        }                                                                                        \
      }                                                                                          \
    }                                                                                            \
    __builtin_amdgcn_sched_group_barrier(0x100, RPV * VRD, 2);                                   \
    _Pragma("unroll") for (int u = 0; u < RPV * NC - RPV; ++u) {                                 \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);                                         \
      __builtin_amdgcn_sched_group_barrier(0x100, VRD, 2);                                       \
    }                                                                                            \
    __builtin_amdgcn_sched_group_barrier(0x008, RPV, 2);                                         \
  } while (0)
#define SAGE_PV(VB_)                                                                             \
  do {                                                                                           \
    if (PV8) {                                                                                   \
      if (__ballot(alpha != 1.f)) {                                                              \
        /* flush: of += float(int32 sum) * 2^(mpv - m0), moving m0 up to mpv */                 \
        /* first if that factor would leave the fp32 range guard */                             \
        if (__ballot(mpv - m0 > kRebase)) {                                                      \
          const float r_ = (mpv - m0 > kRebase) ? __builtin_amdgcn_exp2f(m0 - mpv) : 1.f;        \
          m0 = (mpv - m0 > kRebase) ? mpv : m0;                                                  \
          _Pragma("unroll") for (int c = 0; c < NC; ++c)                                         \
            _Pragma("unroll") for (int i = 0; i < 16; ++i) of[c][i] *= r_;                       \
        }                                                                                        \
        const float f_ = __builtin_amdgcn_exp2f(mpv - m0);                                       \
        _Pragma("unroll") for (int c = 0; c < NC; ++c)                                           \
          _Pragma("unroll") for (int i = 0; i < 16; ++i)                                         \
            of[PV8 ? c : 0][i] = __builtin_fmaf(static_cast<float>(__float_as_int(o[c][i])), f_, of[PV8 ? c : 0][i]); \
        _Pragma("unroll") for (int c = 0; c < NC; ++c)                                           \
          _Pragma("unroll") for (int i = 0; i < 16; ++i) o[c][i] = 0.f;                          \
      }                                                                                          \
      SAGE_PV_MMA(VB_, false);                                                                   \
    } else {                                                                                     \
      if (__ballot(alpha != 1.f)) {                                                              \
        _Pragma("unroll") for (int c = 0; c < NC; ++c)                                           \
          _Pragma("unroll") for (int i = 0; i < 16; ++i) o[c][i] *= alpha;                       \
      }                                                                                          \
      SAGE_PV_MMA(VB_, false);                                                                   \
    }                                                                                            \
  } while (0)

  // Softmax of key tile J_ on the scores in s: dequantize to base-2 logits,
  // mask, move the reference max if needed (rescaling l now and O in the next
  // P.V), P = exp2(S - m), row sum, P -> fp16 in pf (keys g*32 + c*8 .. +7 in
  // pf[c]), as a plain per-score sequence (an in-place form with tree row
  // maxima measured slower once each wave group's period sequence is compiled
  // on its own).
  // INT8 form: the exponent offset nm_ = log2(127) - m is lowered by whole
  // ulps until the tile's largest exponent Y_ (the same expression the
  // values use) is at most log2(127), so every weight round(127 P) stays <= 127
  // whatever the rounding of nm_ and of the row max (the excess is below 1.5
  // ulps of nm_: two steps suffice).
#define SAGE_CAP_P8(Y_)                                                                          \
  do {                                                                                           \
    if (PV8) {                                                                                   \
      if ((Y_) > PLOG) nm_ = below_ulp(nm_);                                                     \
      if ((Y_) > PLOG) nm_ = below_ulp(nm_);                                                     \
    }                                                                                            \
  } while (0)

  // INT8 form of P: the 32 values 127 P of this lane (GETP_ reads value E_)
  // rounded to integers (v_cvt_pk_u8_f32 rounds to nearest even; 0 <= 127 P
  // <= 127 up to the exp2 rounding) and packed four per word into pq; rsum_
  // is their sum, four bytes per v_dot4_i32_i8 in two chains.
#define SAGE_PACK_P8(GETP_)                                                                      \
  float rsum_;                                                                                   \
  do {                                                                                           \
    _Pragma("unroll") for (int w_ = 0; w_ < 8; ++w_) {                                           \
      unsigned x_ = 0;                                                                           \
      _Pragma("unroll") for (int b_ = 0; b_ < 4; ++b_) {                                         \
        const int E_ = 4 * w_ + b_;                                                              \
        x_ = __builtin_amdgcn_cvt_pk_u8_f32(GETP_, b_, x_);                                      \
      }                                                                                          \
      pq[w_ >> 2][w_ & 3] = static_cast<int>(x_);                                                \
    }                                                                                            \
    int r0_ = 0, r1_ = 0;                                                                        \
    _Pragma("unroll") for (int u_ = 0; u_ < 2; ++u_) {                                           \
      r0_ = __builtin_amdgcn_sdot4(pq[u_][0], 0x01010101, r0_, false);                           \
      r1_ = __builtin_amdgcn_sdot4(pq[u_][1], 0x01010101, r1_, false);                           \
      r0_ = __builtin_amdgcn_sdot4(pq[u_][2], 0x01010101, r0_, false);                           \
      r1_ = __builtin_amdgcn_sdot4(pq[u_][3], 0x01010101, r1_, false);                           \
    }                                                                                            \
    rsum_ = static_cast<float>(r0_ + r1_);                                                       \
  } while (0)

#define SAGE_SOFTMAX_SEQ(J_, KS_)                                                                    \
  do {                                                                                           \
    const int j_ = (J_);                                                                         \
    const bool masked_ = (CAUSAL && (j_ * kKTile + kKTile - 1 > wrow0)) || (j_ * kKTile + kKTile > N); \
    const int kb_ = j_ * kKTile + g * 32;                                                        \
    float p[32];                                                                                 \
    float mt_, mnew_;                                                                            \
    bool need_;                                                                                  \
    if (PERTOK) {                                                                                \
      const float scq_ = sq * sl2;                                                               \
      const float4* k4_ = reinterpret_cast<const float4*>(ksh + kb_);                            \
      _Pragma("unroll") for (int u = 0; u < 8; ++u) {                                            \
        const float4 kk_ = k4_[u];                                                               \
        const float kv_[4] = {kk_.x, kk_.y, kk_.z, kk_.w};                                       \
        _Pragma("unroll") for (int r = 0; r < 4; ++r) {                                          \
          const int e = 4 * u + r;                                                               \
          p[e] = static_cast<float>(s[e >> 4][e & 15]) * scq_ * kv_[r];                          \
        }                                                                                        \
      }                                                                                          \
      if (masked_) {                                                                             \
        _Pragma("unroll") for (int e = 0; e < 32; ++e) {                                         \
          const int key = kb_ + e;                                                               \
          if ((CAUSAL && key > qrow) || key >= N) p[e] = -INFINITY;                              \
        }                                                                                        \
      }                                                                                          \
      float mx_ = p[0];                                                                          \
      _Pragma("unroll") for (int e = 1; e < 32; ++e) mx_ = fmaxf(mx_, p[e]);                     \
      mt_ = pair_max(mx_);                                                                       \
      need_ = mt_ > m + SLACK;                                                               \
      mnew_ = need_ ? mt_ : m;                                                                   \
      float nm_ = PLOG - mnew_;                                                                  \
      SAGE_CAP_P8(mt_ + nm_);                                                                    \
      _Pragma("unroll") for (int e = 0; e < 32; ++e) p[e] = __builtin_amdgcn_exp2f(p[e] + nm_);  \
    } else if (F16) {                                                                            \
      /* fp32 scores (bits in s): the max is taken before the sm_scale * log2(e) */             \
      /* factor, which is > 0, and the factor is applied in the fma */                          \
      const float sc_ = sl2;                                                                     \
      if (masked_) {                                                                             \
        _Pragma("unroll") for (int e = 0; e < 32; ++e) {                                         \
          const int key = kb_ + e;                                                               \
          if ((CAUSAL && key > qrow) || key >= N) s[e >> 4][e & 15] = __float_as_int(-INFINITY); \
        }                                                                                        \
      }                                                                                          \
      float mx_ = __int_as_float(s[0][0]);                                                       \
      _Pragma("unroll") for (int e = 1; e < 32; ++e) mx_ = fmaxf(mx_, __int_as_float(s[e >> 4][e & 15])); \
      mx_ = pair_max(mx_);                                                                       \
      mt_ = (mx_ == -INFINITY) ? -INFINITY : mx_ * sc_;                                          \
      need_ = mt_ > m + SLACK;                                                               \
      mnew_ = need_ ? mt_ : m;                                                                   \
      float nm_ = PLOG - mnew_;                                                                  \
      SAGE_CAP_P8(__builtin_fmaf(mx_, sc_, nm_));                                                \
      if (masked_) {                                                                             \
        _Pragma("unroll") for (int e = 0; e < 32; ++e) {                                         \
          const float x_ = __int_as_float(s[e >> 4][e & 15]);                                    \
          p[e] = (x_ == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(x_, sc_, nm_)); \
        }                                                                                        \
      } else {                                                                                   \
        _Pragma("unroll") for (int e = 0; e < 32; ++e)                                           \
          p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(__int_as_float(s[e >> 4][e & 15]), sc_, nm_)); \
      }                                                                                          \
    } else {                                                                                     \
      /* one scale per (query block, key tile): the max of the integer scores, */               \
      /* scaled once, is the max of the dequantized scores (the scale is >= 0) */               \
      const float sc_ = sq * (KS_) * sl2;                                                        \
      if (masked_) {                                                                             \
        _Pragma("unroll") for (int e = 0; e < 32; ++e) {                                         \
          const int key = kb_ + e;                                                               \
          if ((CAUSAL && key > qrow) || key >= N) s[e >> 4][e & 15] = INT_MIN;                   \
        }                                                                                        \
        int mi_ = s[0][0];                                                                       \
        _Pragma("unroll") for (int e = 1; e < 32; ++e) mi_ = max(mi_, s[e >> 4][e & 15]);        \
        mi_ = pair_max_i(mi_);                                                                   \
        mt_ = (mi_ == INT_MIN) ? -INFINITY : static_cast<float>(mi_) * sc_;                      \
        need_ = mt_ > m + SLACK;                                                             \
        mnew_ = need_ ? mt_ : m;                                                                 \
        float nm_ = PLOG - mnew_;                                                                \
        SAGE_CAP_P8(__builtin_fmaf(static_cast<float>(mi_), sc_, nm_));                          \
        _Pragma("unroll") for (int e = 0; e < 32; ++e) {                                         \
          const float x_ = __builtin_fmaf(static_cast<float>(s[e >> 4][e & 15]), sc_, nm_);     \
          p[e] = (s[e >> 4][e & 15] == INT_MIN) ? 0.f : __builtin_amdgcn_exp2f(x_);             \
        }                                                                                        \
      } else {                                                                                   \
        int mi_ = s[0][0];                                                                       \
        _Pragma("unroll") for (int e = 1; e < 32; ++e) mi_ = max(mi_, s[e >> 4][e & 15]);        \
        mi_ = pair_max_i(mi_);                                                                   \
        mt_ = static_cast<float>(mi_) * sc_;                                                     \
        need_ = mt_ > m + SLACK;                                                             \
        mnew_ = need_ ? mt_ : m;                                                                 \
        float nm_ = PLOG - mnew_;                                                                \
        SAGE_CAP_P8(__builtin_fmaf(static_cast<float>(mi_), sc_, nm_));                          \
        _Pragma("unroll") for (int e = 0; e < 32; ++e)                                           \
          p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(static_cast<float>(s[e >> 4][e & 15]), sc_, nm_)); \
      }                                                                                          \
    }                                                                                            \
    const float alpha_ = need_ ? __builtin_amdgcn_exp2f(m - mnew_) : 1.f;                       \
    if (PV8) {                                                                                   \
      SAGE_PACK_P8(p[E_]);                                                                       \
      l = l * alpha_ + rsum_;                                                                    \
    } else {                                                                                     \
      _Pragma("unroll") for (int c = 0; c < 4; ++c)                                              \
        _Pragma("unroll") for (int e = 0; e < 8; e += 2) {                                       \
          /* a pair per v_cvt_pk_f16_f32 (round to nearest even) */                             \
          const v2h h_ = __builtin_convertvector((v2f){p[c * 8 + e], p[c * 8 + e + 1]}, v2h);  \
          pf[c][e] = h_[0];                                                                      \
          pf[c][e + 1] = h_[1];                                                                  \
        }                                                                                        \
      /* row sum of the fp16 P that multiplies V: two products per v_dot2_f32_f16 */            \
      float rs0_ = 0.f, rs1_ = 0.f;                                                              \
      _Pragma("unroll") for (int c = 0; c < 4; ++c)                                              \
        _Pragma("unroll") for (int e = 0; e < 8; e += 4) {                                       \
          rs0_ = __builtin_amdgcn_fdot2(v2h{pf[c][e], pf[c][e + 1]}, kOnes2, rs0_, false);      \
          rs1_ = __builtin_amdgcn_fdot2(v2h{pf[c][e + 2], pf[c][e + 3]}, kOnes2, rs1_, false);  \
        }                                                                                        \
      l = l * alpha_ + (rs0_ + rs1_);                                                            \
    }                                                                                            \
    mpv = m;                                                                                     \
    m = mnew_;                                                                                   \
    alpha = alpha_;                                                                              \
  } while (0)

#define SAGE_SOFTMAX(J_, KS_)                                                                    \
  do {                                                                                           \
    SAGE_SOFTMAX_SEQ(J_, KS_);                                                                   \
  } while (0)

  // One period of the ping-pong. Key tile jp_ is in K buffer KB_, tile jp_-1
  // in V buffer VBP_ (buffer offsets are per-period values; every LDS access
  // is a per-period base plus an immediate). Phase A: group 0 runs its matrix
  // ops (P.V of tile jp_-1, scores of tile jp_) while group 1 runs its softmax
  // of tile jp_-1; phase B swaps the roles. Tiles jp_+1 (K, clamped to the
  // last tile) and jp_ (V) are staged meanwhile into the free buffers KBN_ and
  // VBC_. The first (jp_ = 0) and last (jp_ = nkt) periods are peeled, so the
  // steady-state loop has no conditional work and no register copies.
  // Score register (t, i) of lane group g holds key g*32 + t*16 + i of the tile
  // (the permuted K rows), for query wrow0 + l32.
#define SAGE_DUMP_S(J_)                                                                          \
  do {                                                                                           \
    if (DUMP && (J_) == dkt && bh == dbh && qt == dqt) {                                         \
      _Pragma("unroll") for (int t = 0; t < 2; ++t)                                              \
        _Pragma("unroll") for (int i = 0; i < 16; ++i)                                           \
          dump[(wave * 32 + l32) * kKTile + g * 32 + t * 16 + i] = s[t][i];                      \
    }                                                                                            \
  } while (0)
#define SAGE_PHASE_MATRIX(HAS_PV_, HAS_K_, KB_, VBP_)                                                     \
  __builtin_amdgcn_s_setprio(1);                                                                 \
  if (HAS_PV_) { SAGE_PV(VBP_); }                                                                \
  __builtin_amdgcn_sched_barrier(0);                                                             \
  if (HAS_K_) { SAGE_SCORES(KB_); SAGE_DUMP_S(jp_); }                                            \
  __builtin_amdgcn_s_setprio(0);
#define SAGE_PERIOD(J_, KB_, KBN_, VBC_, VBP_, FIRST_, LAST_, G_)                                \
  do {                                                                                           \
    const int jp_ = (J_);                                                                        \
    /* per-block K scale of tile jp_, loaded a phase before group 0's softmax */                \
    /* uses it; group 1's softmax of tile jp_ - 1 uses the one of the last period */           \
    const float ksn_ = (SM == kScoresInt8Block) ? ksh[min(jp_, nkt - 1)] : 0.f;                 \
    if (!(LAST_)) {                                                                              \
      SAGE_LOAD_K(min(jp_ + 1, nkt - 1))                                                         \
      SAGE_LOAD_V(jp_)                                                                           \
    }                                                                                            \
    if ((G_) == 0) {                                                                             \
      SAGE_PHASE_MATRIX(!(FIRST_), !(LAST_), smem + (KB_), smem + (VBP_))                        \
    } else if (!(FIRST_)) {                                                                      \
      SAGE_SOFTMAX(jp_ - 1, ksp);                                                                \
    }                                                                                            \
    if (PP) __syncthreads();  /* the ping-pong's phase switch */                                 \
    if ((G_) == 1) {                                                                             \
      SAGE_PHASE_MATRIX(!(FIRST_), !(LAST_), smem + (KB_), smem + (VBP_))                        \
    } else if (!(LAST_)) {                                                                       \
      SAGE_SOFTMAX(jp_, ksn_);                                                                   \
    }                                                                                            \
    if (!(LAST_)) {                                                                              \
      SAGE_STORE_K(KBN_)                                                                         \
      SAGE_STORE_V(VBC_)                                                                         \
    }                                                                                            \
    __syncthreads();                                                                             \
    ksp = ksn_;                                                                                  \
  } while (0)

  float ksp = 0.f;
  if (!DMA) {
    SAGE_LOAD_K(0)
    SAGE_STORE_K(KB0)
    // Drain every outstanding load here (Q fragments included): otherwise the
    // counter-based waits inside the loop cannot tell the Q loads are done and
    // wait on the tile prefetch before each period's score MFMAs.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // The period sequence, compiled once per wave group (the group's phase order
    // is then fixed in the code: no register copies where the two orders would
    // otherwise merge; 3-16% faster). Both groups pass the same barriers in the
    // same order.
#define SAGE_PERIODS(G_)                                                                         \
  do {                                                                                           \
    SAGE_PERIOD(0, KB0, KB1, VB0, VB1, true, false, G_);                                         \
    /* INT8 P.V: the fp32 accumulator's reference is the first tile's max */                    \
    m0 = m;                                                                                      \
    int jt = 1;                                                                                  \
    for (; jt + 1 < nkt; jt += 2) {                                                              \
      SAGE_PERIOD(jt, KB1, KB0, VB1, VB0, false, false, G_);                                     \
      SAGE_PERIOD(jt + 1, KB0, KB1, VB0, VB1, false, false, G_);                                 \
    }                                                                                            \
    if (jt < nkt) SAGE_PERIOD(jt, KB1, KB0, VB1, VB0, false, false, G_);                         \
    const int odd = nkt & 1;                                                                     \
    SAGE_PERIOD(nkt, odd ? KB1 : KB0, odd ? KB0 : KB1, odd ? VB1 : VB0, odd ? VB0 : VB1, false, true, G_); \
  } while (0)
    if (grp == 0) SAGE_PERIODS(0);
    else SAGE_PERIODS(1);
  } else {
    // Three LDS stages per operand: key tile t in K stage t % 3, value tile t
    // in V stage t % 3. Period jp_ reads K(jp_) and V(jp_ - 1) and issues the
    // loads of K(jp_ + 2) and V(jp_ + 1) (clamped to the last tile; a
    // clamped copy lands in a stage nobody reads again), which then have two
    // periods to arrive: at the end of a period each wave waits only for the
    // loads it issued before that period. Each wave instruction fills 1 KiB of
    // a stage (lane l: bytes 16 l .. +15); every lane's source is the 16 bytes
    // the padded, permuted tile layout puts there (pad bytes: a repeat of the
    // row's first chunk). Rows past N read as zeros by the buffer's range check.
    constexpr int KI = KT_BYTES / 1024, VI = VT_BYTES / 1024;   // wave instructions per tile
    // the loads are spread over all waves when that gives each the same
    // count, else over the first wave group only (a compile-time set in the
    // period sequence, which is compiled per group): every issuing wave then
    // waits for a constant count
    constexpr int NW = ((KI + VI) % (NTH / 64) == 0 && KI % (NTH / 64) == 0) ? NTH / 64 : NTH / 128;
    static_assert(!DMA || (KI % NW == 0 && VI % NW == 0), "tile loads split evenly over the issuing waves");
    constexpr int NVMC = KI / NW + VI / NW;   // loads per issuing wave and period
    const bool issuer = wave < NW;
    static_assert(!DMA || (KT_BYTES % 1024 == 0 && VT_BYTES % 1024 == 0), "tiles fill whole wave instructions");
    constexpr int KIW = (KI + NW - 1) / NW, VIW = (VI + NW - 1) / NW;
    constexpr int KDATA = D * EB, VDATA = D * 2;   // data bytes per K / V row
    static_assert(!DMA || (KROW == KDATA && VROW == VDATA), "unpadded rows");
    int kdo[KIW], vdo[VIW];
    int nvm = 0;   // this wave's tile load instructions per period
#pragma unroll
    for (int u = 0; u < KIW; ++u) {
      const int b = (wave + NW * u) * 1024 + lane * 16, row = b / KROW, q = (b % KROW) / 16;
      kdo[u] = key_of_lds_row(row) * KDATA + ((q ^ ((row >> KSH) & (KCPR - 1))) * 16);
      nvm += (wave + NW * u < KI) ? 1 : 0;
    }
#pragma unroll
    for (int u = 0; u < VIW; ++u) {
      const int b = (wave + NW * u) * 1024 + lane * 16, row = b / VROW, q = (b % VROW) / 16;
      vdo[u] = row * VDATA + ((((q >> 2) ^ ((row >> VSH) & (VSEG - 1))) * 4 + (q & 3)) * 16);
      nvm += (wave + NW * u < VI) ? 1 : 0;
    }
    nvm = issuer ? NVMC : 0;
#define SAGE_SK(I_) ((I_) == 0 ? smk0 : ((I_) == 1 ? smk1 : smk2))
#define SAGE_SV(I_) ((I_) == 0 ? smv0 : ((I_) == 1 ? smv1 : smv2))
#define SAGE_DMA_K(J_, ST_)                                                                      \
    _Pragma("unroll") for (int u = 0; u < KIW; ++u) {                                            \
      if (wave + NW * u < KI)                                                                    \
        lds_dma16(rk, SAGE_SK(ST_) + (wave + NW * u) * 1024, kdo[u], (J_) * (kKTile * KDATA));   \
    }
#define SAGE_DMA_V(J_, ST_)                                                                      \
    _Pragma("unroll") for (int u = 0; u < VIW; ++u) {                                            \
      if (wave + NW * u < VI)                                                                    \
        lds_dma16(rv, SAGE_SV(ST_) + (wave + NW * u) * 1024, vdo[u], (J_) * (kKTile * VDATA));   \
    }
  // end of a period: this wave's loads issued before it have landed (the ones
  // issued in it may still be in flight), then the barrier; the acquire fence
  // keeps the next period's LDS reads behind it (a release fence would wait
  // for every load in flight)
#define SAGE_END_BARRIER(N_)                                                                     \
  do {                                                                                           \
    wait_vmcnt(N_);                                                                              \
    __builtin_amdgcn_s_barrier();                                                                \
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");                              \
  } while (0)
  // Period jp_ with K stage SK_ = jp_ % 3 (a compile-time constant): reads
  // K(jp_) from stage SK_ and V(jp_ - 1) from stage (SK_ + 2) % 3; loads
  // K(jp_ + 2) into stage (SK_ + 2) % 3 (K(jp_ - 1)'s, read in the last
  // period) and V(jp_ + 1) into stage (SK_ + 1) % 3 (V(jp_ - 2)'s).
#define SAGE_PERIOD_DMA(J_, SK_, FIRST_, LAST_, G_)                                              \
  do {                                                                                           \
    const int jp_ = (J_);                                                                        \
    const float ksn_ = (SM == kScoresInt8Block) ? ksh[min(jp_, nkt - 1)] : 0.f;                 \
    if (!(LAST_) && ((G_) == 0 || NW == NTH / 64)) {                                             \
      SAGE_DMA_K(min(jp_ + 2, nkt - 1), ((SK_) + 2) % 3)                                         \
      SAGE_DMA_V(min(jp_ + 1, nkt - 1), ((SK_) + 1) % 3)                                         \
    }                                                                                            \
    if ((G_) == 0) {                                                                             \
      SAGE_PHASE_MATRIX(!(FIRST_), !(LAST_), SAGE_SK(SK_), SAGE_SV(((SK_) + 2) % 3))             \
    } else if (!(FIRST_)) {                                                                      \
      SAGE_SOFTMAX(jp_ - 1, ksp);                                                                \
    }                                                                                            \
    /* the ping-pong's phase switch: it orders no LDS data (the loads in */                     \
    /* flight write stages nobody reads in this period) */                                      \
    __builtin_amdgcn_s_barrier();                                                                \
    if ((G_) == 1) {                                                                             \
      SAGE_PHASE_MATRIX(!(FIRST_), !(LAST_), SAGE_SK(SK_), SAGE_SV(((SK_) + 2) % 3))             \
    } else if (!(LAST_)) {                                                                       \
      SAGE_SOFTMAX(jp_, ksn_);                                                                   \
    }                                                                                            \
    /* K(jp_ + 1) and V(jp_), issued a period earlier, must have landed */                      \
    if (!(LAST_)) SAGE_END_BARRIER(((G_) == 0 || NW == NTH / 64) ? NVMC : 0);                   \
    ksp = ksn_;                                                                                  \
  } while (0)
    // prologue: K(0) -> stage 0, K(1) -> stage 1, V(0) -> stage 0; the Q
    // fragments and K(0) must have landed before period 0
    if (issuer) {
      SAGE_DMA_K(0, 0)
      SAGE_DMA_K(min(1, nkt - 1), 1)
      SAGE_DMA_V(0, 0)
    }
    __shared__ float qmax_w[QIN ? 8 : 1];   // max |Q| of each wave's 32 rows
    if (QIN && qin) {
      float mq = 0.f;
#pragma unroll
      for (int u = 0; u < 2 * NQF; ++u) {
        const unsigned w4[4] = {qraw[u].x, qraw[u].y, qraw[u].z, qraw[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          mq = fmaxf(mq, fabsf(static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w4[j] & 0xffffu)))));
          mq = fmaxf(mq, fabsf(static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w4[j] >> 16)))));
        }
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) mq = fmaxf(mq, __shfl_xor(mq, off, 64));
      if (lane == 0) qmax_w[wave] = mq;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    }
    SAGE_END_BARRIER(nvm);   // nvm = this wave's K(1) + V(0) instructions
    if (QIN && qin) {
      // the Q block of this wave: qblk / 32 consecutive waves (qblk is 128 or 64)
      const int nw = qblk >> 5, b0 = wave & -nw;
      float a = fmaxf(qmax_w[b0], qmax_w[b0 + 1]);
      if (nw == 4) a = fmaxf(a, fmaxf(qmax_w[b0 + 2], qmax_w[b0 + 3]));
      // every lane read the same words: a scalar, so that the choice of the
      // quotient below is one branch for the wave, not one per element
      a = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, a)));
      const float sb = a / 127.0f;
      const auto codes = [&](auto code) {
#pragma unroll
        for (int c = 0; c < NQF; ++c) {
          unsigned w[16];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const unsigned w4[4] = {qraw[2 * c + h].x, qraw[2 * c + h].y, qraw[2 * c + h].z, qraw[2 * c + h].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              w[h * 8 + 2 * j] = code(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w4[j] & 0xffffu)));
              w[h * 8 + 2 * j + 1] = code(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w4[j] >> 16)));
            }
          }
          qf[c] = v4i{static_cast<int>(pack_low_bytes(w[0], w[1], w[2], w[3])),
                      static_cast<int>(pack_low_bytes(w[4], w[5], w[6], w[7])),
                      static_cast<int>(pack_low_bytes(w[8], w[9], w[10], w[11])),
                      static_cast<int>(pack_low_bytes(w[12], w[13], w[14], w[15]))};
        }
      };
      if (sb >= kMarksteinMinScale) {
        const float y = 1.0f / sb;
        codes([&](_Float16 x) { return int8_code_bits_h(x, sb, y); });
      } else {
        codes([&](_Float16 x) { return int8_code_bits_div(static_cast<float>(x), sb); });
      }
      sq = sb;
    }
#define SAGE_PERIODS_DMA(G_)                                                                     \
  do {                                                                                           \
    SAGE_PERIOD_DMA(0, 0, true, false, G_);                                                      \
    int jt = 1;                                                                                  \
    for (; jt + 2 < nkt; jt += 3) {                                                              \
      SAGE_PERIOD_DMA(jt, 1, false, false, G_);                                                  \
      SAGE_PERIOD_DMA(jt + 1, 2, false, false, G_);                                              \
      SAGE_PERIOD_DMA(jt + 2, 0, false, false, G_);                                              \
    }                                                                                            \
    if (jt < nkt) SAGE_PERIOD_DMA(jt, 1, false, false, G_);                                      \
    if (jt + 1 < nkt) SAGE_PERIOD_DMA(jt + 1, 2, false, false, G_);                              \
    const int sl = nkt % 3;                                                                      \
    if (sl == 0) SAGE_PERIOD_DMA(nkt, 0, false, true, G_);                                       \
    else if (sl == 1) SAGE_PERIOD_DMA(nkt, 1, false, true, G_);                                  \
    else SAGE_PERIOD_DMA(nkt, 2, false, true, G_);                                               \
    /* no load may still be writing this workgroup's LDS when it ends */                        \
    wait_vmcnt(0);                                                                               \
  } while (0)
    if (grp == 0) SAGE_PERIODS_DMA(0);
    else SAGE_PERIODS_DMA(1);
#undef SAGE_PERIODS_DMA
#undef SAGE_PERIOD_DMA
#undef SAGE_END_BARRIER
#undef SAGE_DMA_V
#undef SAGE_DMA_K
#undef SAGE_SV
#undef SAGE_SK
  }
#undef SAGE_PERIODS
#undef SAGE_PHASE_MATRIX
#undef SAGE_DUMP_S
#undef SAGE_PERIOD
#undef SAGE_SOFTMAX
#undef SAGE_SOFTMAX_SEQ
#undef SAGE_PACK_P8
#undef SAGE_CAP_P8
#undef SAGE_PV
#undef SAGE_PV_MMA
#undef SAGE_VA
#undef SAGE_SCORES
#undef SAGE_STORE_V
#undef SAGE_STORE_K
#undef SAGE_LOAD_V
#undef SAGE_LOAD_K

  // epilogue: O = O^T / l, rows >= N are padding and are not stored
  const float lsum = pair_sum(l);
  const float inv = 1.f / lsum;
  // the row log-sum-exp for a backward pass: m is the reference max and l the
  // row sum against it, both in log2 units of the scaled scores
  if (!PV8 && lse != nullptr && g == 0 && qrow < N)
    lse[static_cast<size_t>(bh) * N + qrow] = (m + __log2f(lsum)) * 0.693147180559945309f;
  const float f0 = PV8 ? __builtin_amdgcn_exp2f(m0 - m) : 1.f;  // of's reference against the final max
  if (qrow < N) {
    _Float16* orow = out + (static_cast<size_t>(bh) * N + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < NC; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v4h h;
        if (PV8) {
          // sums of weight * code against the final max: the fp32 part (against
          // m0) and the int32 part; channel c's value is code * scale[c]
          const float4 vs4 = *reinterpret_cast<const float4*>(vsc + static_cast<size_t>(bh) * D + dt * 32 + r * 8 + g * 4);
          const float vsv[4] = {vs4.x, vs4.y, vs4.z, vs4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float sum = __builtin_fmaf(of[PV8 ? dt : 0][r * 4 + i], f0,
                                             static_cast<float>(__float_as_int(o[dt][r * 4 + i])));
            h[i] = static_cast<_Float16>(sum * (vsv[i] * inv));
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) h[i] = static_cast<_Float16>(o[dt][r * 4 + i] * inv);
        }
        *reinterpret_cast<v4h*>(orow + dt * 32 + r * 8 + g * 4) = h;
      }
  }
}

hipError_t launch_attn_int8(const AttnArgs& a, const void* q, const void* k, const void* vt,
                            const float* qs, const float* ks, const float* vs, hipStream_t s) {
  // modes: 0 Q128/K64, 1 Q64/K64, 3 per token, 4 FP16, 6 Q128/K64 + INT8 P.V, 7 per token + INT8 P.V
  const bool tok = a.mode == 3 || a.mode == 7;
  const int qblk = tok ? 1 : (a.mode == 1 ? 64 : 128);
  const int sm = tok ? kScoresInt8Token : (a.mode == 4 ? kScoresF16 : kScoresInt8Block);
  const bool pv8 = mode_pv_int8(a.mode);
  auto* o = static_cast<_Float16*>(a.out);
#define SAGE_LAUNCH(D_, C_, S_, P_)                                                                  \
  do {                                                                                               \
    constexpr bool pp_ = attn_pingpong(D_, S_, P_, false);                                           \
    const dim3 grid_(a.BH * (a.Npad / (pp_ ? kWGQ : kWGQ / 2))), block_(pp_ ? 512 : 256);            \
    attn_int8_kernel<D_, C_, S_, P_><<<grid_, block_, 0, s>>>(q, k, vt, qs, ks, vs, o, a.N, a.Npad,  \
                                                              qblk, a.sl2, a.BH, nullptr, 0, 0, 0,   \
                                                              a.lse, a.qin ? 1 : 0);                 \
  } while (0)
#define SAGE_LAUNCH_SM(D_, C_)                                                    \
  do {                                                                            \
    if (sm == kScoresF16) SAGE_LAUNCH(D_, C_, kScoresF16, false);                 \
    else if (sm == kScoresInt8Token) {                                            \
      if (pv8) SAGE_LAUNCH(D_, C_, kScoresInt8Token, true);                       \
      else SAGE_LAUNCH(D_, C_, kScoresInt8Token, false);                          \
    } else {                                                                      \
      if (pv8) SAGE_LAUNCH(D_, C_, kScoresInt8Block, true);                       \
      else SAGE_LAUNCH(D_, C_, kScoresInt8Block, false);                          \
    }                                                                             \
  } while (0)
  if (a.d == 128) {
    if (a.causal) SAGE_LAUNCH_SM(128, true); else SAGE_LAUNCH_SM(128, false);
  } else {
    if (a.causal) SAGE_LAUNCH_SM(64, true); else SAGE_LAUNCH_SM(64, false);
  }
#undef SAGE_LAUNCH_SM
#undef SAGE_LAUNCH
  return hipGetLastError();
}

hipError_t launch_attn_int8_dump(const AttnArgs& a, const void* q, const void* k, const void* vt,
                                 const float* qs, const float* ks, int* dump, int dbh, int dqt, int dkt,
                                 hipStream_t s) {
  const int nqt = a.Npad / kWGQ;
  const dim3 grid(a.BH * nqt), block(512);
  const bool tok = a.mode == 3;
  const int qblk = tok ? 1 : (a.mode == 1 ? 64 : 128);
  auto* o = static_cast<_Float16*>(a.out);
#define SAGE_LAUNCH_DUMP(D_, S_)                                                                          \
  attn_int8_kernel<D_, false, S_, false, true><<<grid, block, 0, s>>>(q, k, vt, qs, ks, nullptr, o, a.N, a.Npad, \
                                                                       qblk, a.sl2, a.BH, dump, dbh, dqt, dkt)
  if (a.d == 128) {
    if (tok) SAGE_LAUNCH_DUMP(128, kScoresInt8Token); else SAGE_LAUNCH_DUMP(128, kScoresInt8Block);
  } else {
    if (tok) SAGE_LAUNCH_DUMP(64, kScoresInt8Token); else SAGE_LAUNCH_DUMP(64, kScoresInt8Block);
  }
#undef SAGE_LAUNCH_DUMP
  return hipGetLastError();
}

}  // namespace sage
