// INT8 attention backward pass for gfx950 (CDNA4).
//
// The 8-bit backward of "SageAttention3: Microscaling FP4 Attention for
// Inference and An Exploration of 8-Bit Training" (abstract; the trainable
// attention is INT8 on the scifaro.com page of related papers), laid out as
// FlashAttention-2's backward, which the SageAttention page's "Experimental
// setup" names as the base: the scores are recomputed from the forward's Q and
// K codes, P = exp(S - L) from the forward's row log-sum-exp L, and
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO o O),  dS = P o (dP - D),
//   dQ = sm_scale dS K_s,  dK = sm_scale dS^T Q,
// every product on v_mfma_i32_32x32x32_i8 with int32 accumulation:
//   * S: the forward's codes (Q per 128- or 64-token block, K_s per 64 keys);
//   * dP: dO per 64-token block, V per token (one scale per key);
//   * dV, dK, dQ: P and dS quantized per aligned 32 x 32 tile of the N x N
//     matrices (a = max|x| over the tile, s = a / 127, code = rint(x / s)), so
//     each product sums one tile exactly in int32 and the tile's partial is
//     scaled and added in fp32.
//
// Work decomposition
//   * Tiles are loaded straight into LDS (buffer loads with an LDS
//     destination) and double-buffered: a tile's loads are issued before the
//     previous tile's work and waited for after it.
//   * bwd_dkdv_kernel: a workgroup owns 128 keys of one head (4 waves x 32)
//     and walks the query tiles (64 queries, two 32-query sub-blocks). Per
//     sub-block a wave computes S and dP for its 32 keys x 32 queries (K and V
//     codes of its keys are the B operands, kept in registers; Q and dO rows
//     come from LDS), P and dS in registers, their tile codes, then
//     dV^T += dO^T P and dK^T += Q^T dS with the transposed Q and dO codes
//     from LDS as A operands.
//   * bwd_dq_kernel: a workgroup owns 128 queries (4 waves x 32) and walks the
//     key tiles; per 32-key sub-block a wave computes S^T and dP^T (Q and dO
//     codes of its queries in registers, K and V rows from LDS), dS and its
//     tile codes, and dQ^T += K^T dS^T.
//   * Both kernels form P and dS with the same fp32 expressions, so the two
//     quantize every dS tile identically.
//   * The first product's A rows are read in a permuted order (row r of the
//     32-row operand holds index perm32(r)) so that the accumulator register i
//     of lane group g holds index g*16 + i: the 16 codes of a lane are then,
//     byte for byte, the B operand of the second product, whose A operand
//     reads 16 consecutive indices at offset g*16.
#include "sage_internal.h"

#include <math.h>

namespace sage {

namespace {

constexpr int kBT = 64;    // loop tile: queries (dK/dV) or keys (dQ)
constexpr int kBW = 128;   // rows of the fixed dimension per workgroup (4 waves x 32)
constexpr float kLog2e = 1.4426950408889634f;

// Index held by row r of a 32-row A operand: the accumulator layout puts row
// (i/4)*8 + g*4 + i%4 in register i of lane group g, and this makes that
// index g*16 + i.
__device__ __forceinline__ int perm32(int r) { return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3); }

// Waits until none of this wave's vector memory operations is outstanding
// (s_waitcnt with only the vmcnt field set, so LDS and scalar counters are
// left alone).
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0xF70); }

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// lds + 16 l (buffer_load_dwordx4 with an LDS destination; the LDS address is
// wave-uniform). A non-template helper: the host-side pass of a kernel
// template that names this builtin drops the kernel.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Maximum over the 64 lanes: DPP within each row of 16 (neighbour swaps, then
// the half-row and row mirrors), one lane shuffle between the two rows of a
// half, and the swap of the wave's halves.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));
  x = fmaxf(x, dpp_f32<0x4E>(x));
  x = fmaxf(x, dpp_f32<0x141>(x));
  x = fmaxf(x, dpp_f32<0x140>(x));
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Tile maximum of |x| over a 32 x 32 tile held as one accumulator (16 values
// per lane), and its scale s = fp32(a / 127) with the multiplier r ~ 1 / s
// (0 for an all-zero tile).
__device__ __forceinline__ float tile_scale(const float (&x)[16], float& r) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(x[i]));
  const float a = wave_max(m);
  const float s = a / 127.0f;
  // the codes only need x / s to within a few ulps (a code that close to a
  // rounding boundary may round either way), so v_rcp_f32 serves
  r = s > 0.f ? __builtin_amdgcn_rcpf(s) : 0.f;
  return s;
}

// INT8 codes rint(x * r) of a tile whose values are >= 0 (P), register i in
// byte i: v_cvt_pk_u8_f32 rounds to nearest even (0 <= x r <= 127).
__device__ __forceinline__ float tile_codes_nonneg(const float (&x)[16], v4i& codes) {
  float r;
  const float s = tile_scale(x, r);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    unsigned word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) word = __builtin_amdgcn_cvt_pk_u8_f32(x[w * 4 + b] * r, b, word);
    codes[w] = static_cast<int>(word);
  }
  return s;
}

// Signed codes: rint(x * r) (|x r| <= 127), offset by 128 to an exact integer in
// [1, 255], packed by v_cvt_pk_u8_f32, and the offset taken back per byte
// (XOR 0x80 turns c + 128 into the two's complement byte of c).
__device__ __forceinline__ float tile_codes_signed(const float (&x)[16], v4i& codes) {
  float r;
  const float s = tile_scale(x, r);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    unsigned word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) word = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_rintf(x[w * 4 + b] * r) + 128.f, b, word);
    codes[w] = static_cast<int>(word ^ 0x80808080u);
  }
  return s;
}

// ---------------------------------------------------------------------------
// Row terms: (L2, D) per query row, L2 = L * log2(e) from the forward's
// natural-log L, D = sum_c dO_c O_c (products of fp16 values are exact in fp32,
// summed in fp64, rounded once). Rows >= N: L2 = +inf (P = 0), D = 0.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_rows_kernel(const _Float16* __restrict__ o, const _Float16* __restrict__ dout,
                                                       const float* __restrict__ lse, float2* __restrict__ ld,
                                                       int N, int Npad, int BH) {
  constexpr int LPR = D / 8;          // lanes per row, 8 channels (16 bytes) each
  constexpr int RPB = 256 / LPR;      // rows per workgroup
  const long long total = static_cast<long long>(BH) * Npad;
  const long long r = static_cast<long long>(blockIdx.x) * RPB + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  const bool in = r < total;
  const int bh = in ? static_cast<int>(r / Npad) : 0, n = in ? static_cast<int>(r % Npad) : 0;
  const bool live = in && n < N;
  const size_t row = static_cast<size_t>(bh) * N + n;
  double acc = 0.0;
  if (live) {
    const v8h a = *reinterpret_cast<const v8h*>(o + row * D + c * 8);
    const v8h b = *reinterpret_cast<const v8h*>(dout + row * D + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += static_cast<double>(static_cast<float>(a[e]) * static_cast<float>(b[e]));
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off, 64);
  if (in && c == 0) ld[r] = live ? make_float2(lse[row] * kLog2e, static_cast<float>(acc)) : make_float2(INFINITY, 0.f);
}

// ---------------------------------------------------------------------------
// Transposed copies of INT8 codes: src [BH, Npad, D] -> dst [BH, D, Npad],
// 64 tokens per workgroup through LDS; blockIdx.y picks one of three jobs.
// ---------------------------------------------------------------------------
struct TJob {
  const int8_t* src;
  int8_t* dst;
};
template <int D>
__global__ __launch_bounds__(256) void transpose_codes_kernel(TJob j0, TJob j1, TJob j2, int Npad) {
  const TJob J = blockIdx.y == 0 ? j0 : (blockIdx.y == 1 ? j1 : j2);
  constexpr int ROW = D + 4;
  __shared__ unsigned char t[64 * ROW];
  const int ntile = Npad / 64;
  const int bh = blockIdx.x / ntile, n0 = (blockIdx.x % ntile) * 64;
  const unsigned char* src = reinterpret_cast<const unsigned char*>(J.src) + (static_cast<size_t>(bh) * Npad + n0) * D;
  for (int i = threadIdx.x; i < 64 * D / 4; i += 256) {
    const int row = i / (D / 4), col = i % (D / 4);
    *reinterpret_cast<unsigned*>(t + row * ROW + col * 4) = *reinterpret_cast<const unsigned*>(src + row * D + col * 4);
  }
  __syncthreads();
  unsigned char* dst = reinterpret_cast<unsigned char*>(J.dst) + static_cast<size_t>(bh) * D * Npad + n0;
  for (int i = threadIdx.x; i < D * 16; i += 256) {
    const int ch = i / 16, q = i % 16;  // 4 tokens 4q .. 4q+3 of channel ch
    unsigned w = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) w |= static_cast<unsigned>(t[(q * 4 + b) * ROW + ch]) << (8 * b);
    *reinterpret_cast<unsigned*>(dst + static_cast<size_t>(ch) * Npad + q * 4) = w;
  }
}

// Arguments shared by the two gradient kernels. Codes are zero-padded to
// Npad rows; transposed codes are [BH, D, Npad].
struct BwdArgs {
  const int8_t* qc; const int8_t* qt; const float* qs; int qblk;  // Q codes, Q^T codes, scales [BH, Npad/qblk]
  const int8_t* kc; const int8_t* kt; const float* ks;            // K_s codes, K_s^T codes, scales [BH, Npad/64]
  const int8_t* vc; const float* vs;                              // V codes, scales [BH, Npad] (per token)
  const int8_t* gc; const int8_t* gt; const float* gs;            // dO codes, dO^T codes, scales [BH, Npad/64]
  const float2* ld;                                               // (L2, D) per row [BH, Npad]
  float* dq; float* dk; float* dv;                                // fp32 [BH, N, D]
  int N, Npad, BH;
  float sl2, sm;                                                  // sm_scale * log2(e), sm_scale
};

// Workgroup id -> (head, 128-row block), heads spread contiguously over the
// 8 XCDs (dispatch is round-robin over XCDs by id % 8) so a head's tiles stay
// in one XCD's L2.
__device__ __forceinline__ void map_wg(int id, int BH, int nblk, int& bh, int& blk) {
  const int total = BH * nblk;
  const int per = (total + 7) / 8;
  const int x = id % 8, k = id / 8;
  int lin = x * per + k;
  if (total % 8 != 0 || lin >= total) lin = id;  // uneven split: plain order
  bh = lin / nblk;
  blk = lin % nblk;
}

// ---------------------------------------------------------------------------
// Tile staging shared by the two gradient kernels: every tile (64 rows of d
// code bytes, or d rows of 64 code bytes for a transposed tile) is loaded
// straight into LDS by buffer loads with an LDS destination (one wave
// instruction = 1 KiB, lane l's 16 bytes at +16 l), double-buffered: the
// next tile's loads are issued before the current tile's work and waited for
// at its end, so they need no staging registers. Rows are unpadded; the
// 16-byte chunks are permuted within each row (XOR swizzle) so that the
// matrix ops' LDS reads stay free of bank conflicts: in a row-major tile,
// chunk c of row r sits at position c ^ swz_rm(r), chosen for the reads of
// rows perm32(l32) (16 lanes of a read phase hit 16 distinct 16-byte bank
// groups of the 256-byte bank line); in a transposed tile (64-byte rows),
// at c ^ swz_tr(r), for reads of 16 consecutive rows.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int swz_rm(int r) {
  return D == 128 ? (((r >> 1) & 3) | (((r >> 4) & 1) << 2)) : (((r >> 2) & 1) | (((r >> 4) & 1) << 1));
}
__device__ __forceinline__ int swz_tr(int r) { return (r >> 2) & 3; }

// End of a tile: this wave's loads of the next tile have landed, every wave is
// past its reads of the current stage; the acquire fence keeps the next
// tile's LDS reads behind the barrier (a release fence would also wait for
// loads in flight).
__device__ __forceinline__ void tile_barrier() {
  wait_vmcnt0();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(BwdArgs a, const float* __restrict__ qsp,
                                                            const float* __restrict__ ksp,
                                                            const float* __restrict__ vsp,
                                                            const float* __restrict__ gsp) {
  constexpr int NCH = D / 32;        // 32-channel chunks
  constexpr int TB = kBT * D;        // bytes of a tile (row-major or transposed)
  constexpr int NI = TB / 4096;      // load instructions per wave and tile (4 waves x 1 KiB)
  constexpr int CPR = D / 16;        // 16-byte chunks per row-major row
  static_assert(TB % 4096 == 0, "tiles fill whole wave instructions");
  __shared__ __attribute__((aligned(16))) unsigned char sq0[TB], sq1[TB], sg0[TB], sg1[TB];
  __shared__ __attribute__((aligned(16))) unsigned char sqt0[TB], sqt1[TB], sgt0[TB], sgt1[TB];
  __shared__ __attribute__((aligned(16))) float2 sld0[128], sld1[128];

  const int Npad = a.Npad, N = a.N;
  const int nkb = Npad / kBW;
  int bh, kblk;
  map_wg(blockIdx.x, a.BH, nkb, bh, kblk);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k0w = kblk * kBW + wave * 32;   // first key of this wave
  const int key = k0w + l32;

  // B operands of S and dP: this lane's key, 16 channels per matrix op
  v4i kb[NCH], vb[NCH];
  {
    const int8_t* kp = a.kc + (static_cast<size_t>(bh) * Npad + key) * D + g * 16;
    const int8_t* vp = a.vc + (static_cast<size_t>(bh) * Npad + key) * D + g * 16;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      kb[c] = *reinterpret_cast<const v4i*>(kp + c * 32);
      vb[c] = *reinterpret_cast<const v4i*>(vp + c * 32);
    }
  }
  // the scales are read through restrict-qualified kernel arguments: the
  // compiler then loads the per-tile ones with scalar loads, which do not
  // count against (and wait for) the tile loads in flight
  const float skw = ksp[static_cast<size_t>(bh) * (Npad / 64) + k0w / 64];
  const float svk = vsp[static_cast<size_t>(bh) * Npad + key];
  const float* qsh = qsp + static_cast<size_t>(bh) * (Npad / a.qblk);
  const float* gsh = gsp + static_cast<size_t>(bh) * (Npad / 64);

  v16f dkf[NCH], dvf[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) dkf[c][i] = dvf[c][i] = 0.f;

  const int qt_begin = CAUSAL ? (kblk * kBW) / kBT : 0;
  const int qt_end = (N + kBT - 1) / kBT;
  const auto rq = buffer_rsrc(a.qc + static_cast<size_t>(bh) * Npad * D, static_cast<unsigned>(Npad) * D);
  const auto rg = buffer_rsrc(a.gc + static_cast<size_t>(bh) * Npad * D, static_cast<unsigned>(Npad) * D);
  const auto rqt = buffer_rsrc(a.qt + static_cast<size_t>(bh) * D * Npad, static_cast<unsigned>(Npad) * D);
  const auto rgt = buffer_rsrc(a.gt + static_cast<size_t>(bh) * D * Npad, static_cast<unsigned>(Npad) * D);
  const auto rld = buffer_rsrc(a.ld + static_cast<size_t>(bh) * Npad, static_cast<unsigned>(Npad) * 8);
  // per-lane sources of this wave's load instructions (tile offset added per tile)
  int rmo[NI], tro[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int i = (wave * NI + u) * 64 + lane;
    const int rr = i / CPR, rp = i % CPR;
    rmo[u] = rr * D + ((rp ^ swz_rm<D>(rr)) * 16);
    const int tr = i / 4, tp = i % 4;
    tro[u] = tr * Npad + ((tp ^ swz_tr(tr)) * 16);
  }
  // LDS read offsets: S / dP A operands (rows perm32(l32) of each 32-row
  // half), and the transposed A operands (channel rows l32 of each 32-channel
  // chunk, for either 32-row half)
  int aro[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int r = perm32(l32);
    aro[c] = r * D + (((2 * c + g) ^ swz_rm<D>(r)) * 16);
  }
  const int tsw = swz_tr(l32);

  // stage ST_ (0 or 1, a compile-time constant: the stages are distinct
  // arrays, so the compiler's wait before an LDS read covers only the loads
  // into the stage being read)
#define SAGE_STG(A0_, A1_, ST_) ((ST_) == 0 ? (A0_) : (A1_))
#define SAGE_LOAD_Q(ST_, QT_)                                                                       \
  do {                                                                                              \
    const int q0_ = (QT_) * kBT;                                                                    \
    _Pragma("unroll") for (int u = 0; u < NI; ++u) {                                                \
      const int at_ = (wave * NI + u) * 1024;                                                       \
      lds_dma16(rq, SAGE_STG(sq0, sq1, ST_) + at_, rmo[u] + q0_ * D, 0);                            \
      lds_dma16(rg, SAGE_STG(sg0, sg1, ST_) + at_, rmo[u] + q0_ * D, 0);                            \
      lds_dma16(rqt, SAGE_STG(sqt0, sqt1, ST_) + at_, tro[u] + q0_, 0);                             \
      lds_dma16(rgt, SAGE_STG(sgt0, sgt1, ST_) + at_, tro[u] + q0_, 0);                             \
    }                                                                                               \
    /* (L2, D) of rows q0 .. q0+127 (the second half unused; past Npad: zeros) */                  \
    lds_dma16(rld, reinterpret_cast<unsigned char*>(SAGE_STG(sld0, sld1, ST_)), q0_ * 8 + lane * 16, 0); \
  } while (0)

#define SAGE_TILE_Q(ST_, QT_)                                                                                 \
  do {                                                                                                       \
    const int q0 = (QT_) * kBT;                                                                               \
_Pragma("unroll 1")                                                                                               \
    for (int sb = 0; sb < 2; ++sb) {                                                                          \
      const int qb = q0 + sb * 32;  /* first query of the sub-block */                                        \
      if (CAUSAL && k0w > qb + 31) continue;  /* every key of the wave is above every query */                \
      const int tao = l32 * kBT + (((2 * sb + g) ^ tsw) * 16);                                                \
      v16i s, dp;                                                                                             \
_Pragma("unroll")                                                                                             \
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0;                                                          \
_Pragma("unroll")                                                                                             \
      for (int c = 0; c < NCH; ++c) {                                                                         \
        s = __builtin_amdgcn_mfma_i32_32x32x32_i8(*reinterpret_cast<const v4i*>(SAGE_STG(sq0, sq1, ST_) + sb * 32 * D + aro[c]), kb[c], s, 0, 0, 0);\
        dp = __builtin_amdgcn_mfma_i32_32x32x32_i8(*reinterpret_cast<const v4i*>(SAGE_STG(sg0, sg1, ST_) + sb * 32 * D + aro[c]), vb[c], dp, 0, 0, 0);\
      }                                                                                                       \
      const float sqb = qsh[qb / a.qblk];                                                                     \
      const float gsb = gsh[qb / 64];                                                                         \
      const float cs = (sqb * skw) * a.sl2;                                                                   \
      const float gsv = gsb * svk;                                                                            \
  /* masking only in sub-blocks with keys >= N or above the diagonal */                                       \
      const bool masked = k0w + 31 >= N || (CAUSAL && k0w + 31 > qb);                                         \
      float p[16], ds[16];                                                                                    \
_Pragma("unroll")                                                                                             \
      for (int i = 0; i < 16; ++i) {                                                                          \
        const float2 lq = SAGE_STG(sld0, sld1, ST_)[sb * 32 + g * 16 + i];                                    \
        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(static_cast<float>(s[i]), cs, -lq.x));                   \
        ds[i] = __builtin_fmaf(static_cast<float>(dp[i]), gsv, -lq.y);                                        \
      }                                                                                                       \
      if (masked) {                                                                                           \
_Pragma("unroll")                                                                                             \
        for (int i = 0; i < 16; ++i)                                                                          \
          if (key >= N || (CAUSAL && key > qb + g * 16 + i)) p[i] = 0.f;                                      \
      }                                                                                                       \
_Pragma("unroll")                                                                                             \
      for (int i = 0; i < 16; ++i) ds[i] *= p[i];                                                             \
      v4i pc, dsc;                                                                                            \
      const float sp = tile_codes_nonneg(p, pc);                                                              \
      const float sds = tile_codes_signed(ds, dsc);                                                           \
      const float fv = sp * gsb;                                                                              \
      const float fk = (sds * sqb) * a.sm;                                                                    \
_Pragma("unroll")                                                                                             \
      for (int c = 0; c < NCH; ++c) {                                                                         \
        v16i zv, zk;                                                                                          \
_Pragma("unroll")                                                                                             \
        for (int i = 0; i < 16; ++i) zv[i] = zk[i] = 0;                                                       \
        zv = __builtin_amdgcn_mfma_i32_32x32x32_i8(*reinterpret_cast<const v4i*>(SAGE_STG(sgt0, sgt1, ST_) + c * 32 * kBT + tao), pc, zv, 0, 0, 0);\
        zk = __builtin_amdgcn_mfma_i32_32x32x32_i8(*reinterpret_cast<const v4i*>(SAGE_STG(sqt0, sqt1, ST_) + c * 32 * kBT + tao), dsc, zk, 0, 0, 0);\
_Pragma("unroll")                                                                                             \
        for (int i = 0; i < 16; ++i) {                                                                        \
          dvf[c][i] = __builtin_fmaf(static_cast<float>(zv[i]), fv, dvf[c][i]);                               \
          dkf[c][i] = __builtin_fmaf(static_cast<float>(zk[i]), fk, dkf[c][i]);                               \
        }                                                                                                     \
      }                                                                                                       \
    }                                                                                                         \
  } while (0)

  if (qt_begin < qt_end) SAGE_LOAD_Q(0, qt_begin);
  tile_barrier();
  for (int qt = qt_begin; qt < qt_end; qt += 2) {
    if (qt + 1 < qt_end) SAGE_LOAD_Q(1, qt + 1);
    SAGE_TILE_Q(0, qt);
    tile_barrier();
    if (qt + 1 >= qt_end) break;
    if (qt + 2 < qt_end) SAGE_LOAD_Q(0, qt + 2);
    SAGE_TILE_Q(1, qt + 1);
    tile_barrier();
  }
#undef SAGE_TILE_Q
#undef SAGE_LOAD_Q

  // dV^T and dK^T: lane = key, register i of chunk c = channel c*32 + (i/4)*8 + g*4 + i%4
  if (key < N) {
    float* dvr = a.dv + (static_cast<size_t>(bh) * N + key) * D;
    float* dkr = a.dk + (static_cast<size_t>(bh) * N + key) * D;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ch = c * 32 + r * 8 + g * 4;
        *reinterpret_cast<float4*>(dvr + ch) = make_float4(dvf[c][r * 4], dvf[c][r * 4 + 1], dvf[c][r * 4 + 2], dvf[c][r * 4 + 3]);
        *reinterpret_cast<float4*>(dkr + ch) = make_float4(dkf[c][r * 4], dkf[c][r * 4 + 1], dkf[c][r * 4 + 2], dkf[c][r * 4 + 3]);
      }
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a, const float* __restrict__ qsp,
                                                         const float* __restrict__ ksp,
                                                         const float* __restrict__ vsp,
                                                         const float* __restrict__ gsp) {
  constexpr int NCH = D / 32;
  constexpr int TB = kBT * D;
  constexpr int NI = TB / 4096;
  constexpr int CPR = D / 16;
  static_assert(TB % 4096 == 0, "tiles fill whole wave instructions");
  __shared__ __attribute__((aligned(16))) unsigned char sk0[TB], sk1[TB], sv0[TB], sv1[TB], skt0[TB], skt1[TB];
  __shared__ __attribute__((aligned(16))) float ssv0[256], ssv1[256];

  const int Npad = a.Npad, N = a.N;
  const int nqb = Npad / kBW;
  int bh, qblk;
  map_wg(blockIdx.x, a.BH, nqb, bh, qblk);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q0w = qblk * kBW + wave * 32;   // first query of this wave
  const int query = q0w + l32;

  // B operands of S^T and dP^T: this lane's query
  v4i qb[NCH], gb[NCH];
  {
    const int8_t* qp = a.qc + (static_cast<size_t>(bh) * Npad + query) * D + g * 16;
    const int8_t* gp = a.gc + (static_cast<size_t>(bh) * Npad + query) * D + g * 16;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      qb[c] = *reinterpret_cast<const v4i*>(qp + c * 32);
      gb[c] = *reinterpret_cast<const v4i*>(gp + c * 32);
    }
  }
  const float sqw = qsp[static_cast<size_t>(bh) * (Npad / a.qblk) + q0w / a.qblk];
  const float gsw = gsp[static_cast<size_t>(bh) * (Npad / 64) + q0w / 64];
  const float2 lq = a.ld[static_cast<size_t>(bh) * Npad + query];
  const float* ksh = ksp + static_cast<size_t>(bh) * (Npad / 64);

  v16f dqf[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqf[c][i] = 0.f;

  int kt_end = (N + kBT - 1) / kBT;
  if (CAUSAL) kt_end = min(kt_end, (qblk * kBW + kBW) / kBT);
  const auto rk = buffer_rsrc(a.kc + static_cast<size_t>(bh) * Npad * D, static_cast<unsigned>(Npad) * D);
  const auto rv = buffer_rsrc(a.vc + static_cast<size_t>(bh) * Npad * D, static_cast<unsigned>(Npad) * D);
  const auto rkt = buffer_rsrc(a.kt + static_cast<size_t>(bh) * D * Npad, static_cast<unsigned>(Npad) * D);
  const auto rvs = buffer_rsrc(vsp + static_cast<size_t>(bh) * Npad, static_cast<unsigned>(Npad) * 4);
  int aro[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int r = perm32(l32);
    aro[c] = r * D + (((2 * c + g) ^ swz_rm<D>(r)) * 16);
  }
  const int tsw = swz_tr(l32);

  auto load_tile = [&](unsigned char* dk_, unsigned char* dv_, unsigned char* dkt_, float* dsv_, int kt) __attribute__((always_inline)) {
    const int k0 = kt * kBT;
    // this lane's source chunks, recomputed per tile (a few VALU instructions
    // instead of registers held across the loop; the empty asm keeps the
    // compiler from hoisting them out of it)
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int i = (wave * NI + u) * 64 + ln;
      const int rr = i / CPR, rp = i % CPR, tr = i / 4, tp = i % 4;
      const int rmo = rr * D + ((rp ^ swz_rm<D>(rr)) * 16);
      const int tro = tr * Npad + ((tp ^ swz_tr(tr)) * 16);
      const int at = (wave * NI + u) * 1024;
      lds_dma16(rk, dk_ + at, rmo + k0 * D, 0);
      lds_dma16(rv, dv_ + at, rmo + k0 * D, 0);
      lds_dma16(rkt, dkt_ + at, tro + k0, 0);
    }
    // V scales of keys k0 .. k0+255 (the first 64 used; past Npad: zeros)
    lds_dma16(rvs, reinterpret_cast<unsigned char*>(dsv_), k0 * 4 + lane * 16, 0);
  };

  auto tile = [&](const unsigned char* sk, const unsigned char* sv, const unsigned char* skt, const float* ssv,
                  int kt) __attribute__((always_inline)) {
    const int k0 = kt * kBT;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int kb0 = k0 + sb * 32;                   // first key of the sub-block
      if (CAUSAL && kb0 > q0w + 31) continue;
      const int tao = l32 * kBT + (((2 * sb + g) ^ tsw) * 16);
      v16i s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        s = __builtin_amdgcn_mfma_i32_32x32x32_i8(*reinterpret_cast<const v4i*>(sk + sb * 32 * D + aro[c]), qb[c], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_i32_32x32x32_i8(*reinterpret_cast<const v4i*>(sv + sb * 32 * D + aro[c]), gb[c], dp, 0, 0, 0);
      }
      const float skb = ksh[kb0 / 64];
      const float cs = (sqw * skb) * a.sl2;
      const bool masked = kb0 + 31 >= N || (CAUSAL && kb0 + 31 > q0w);
      float ds[16];
      float pv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float gsv = gsw * ssv[sb * 32 + g * 16 + i];
        pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(static_cast<float>(s[i]), cs, -lq.x));
        ds[i] = __builtin_fmaf(static_cast<float>(dp[i]), gsv, -lq.y);
      }
      if (masked) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kj = kb0 + g * 16 + i;
          if (kj >= N || (CAUSAL && kj > query)) pv[i] = 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) ds[i] *= pv[i];
      v4i dsc;
      const float sds = tile_codes_signed(ds, dsc);
      const float fq = (sds * skb) * a.sm;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        v16i z;
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = 0;
        z = __builtin_amdgcn_mfma_i32_32x32x32_i8(*reinterpret_cast<const v4i*>(skt + c * 32 * kBT + tao), dsc, z, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) dqf[c][i] = __builtin_fmaf(static_cast<float>(z[i]), fq, dqf[c][i]);
      }
    }
  };

  if (kt_end > 0) load_tile(sk0, sv0, skt0, ssv0, 0);
  tile_barrier();
  for (int kt = 0; kt < kt_end; kt += 2) {
    if (kt + 1 < kt_end) load_tile(sk1, sv1, skt1, ssv1, kt + 1);
    tile(sk0, sv0, skt0, ssv0, kt);
    tile_barrier();
    if (kt + 1 >= kt_end) break;
    if (kt + 2 < kt_end) load_tile(sk0, sv0, skt0, ssv0, kt + 2);
    tile(sk1, sv1, skt1, ssv1, kt + 1);
    tile_barrier();
  }

  if (query < N) {
    float* dqr = a.dq + (static_cast<size_t>(bh) * N + query) * D;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<float4*>(dqr + c * 32 + r * 8 + g * 4) =
            make_float4(dqf[c][r * 4], dqf[c][r * 4 + 1], dqf[c][r * 4 + 2], dqf[c][r * 4 + 3]);
  }
}

}  // namespace

hipError_t launch_attn_bwd(const BwdLaunch& b, hipStream_t s) {
  const int BH = b.BH, N = b.N, Npad = b.Npad, d = b.d;
  {
    const long long rows = static_cast<long long>(BH) * Npad;
    const int rpb = 256 / (d / 8);
    const dim3 grid(static_cast<unsigned>((rows + rpb - 1) / rpb));
    if (d == 128) bwd_rows_kernel<128><<<grid, 256, 0, s>>>(b.o, b.dout, b.lse, b.ld, N, Npad, BH);
    else bwd_rows_kernel<64><<<grid, 256, 0, s>>>(b.o, b.dout, b.lse, b.ld, N, Npad, BH);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const TJob j0{b.qc, b.qt}, j1{b.kc, b.kt}, j2{b.gc, b.gt};
    const dim3 grid(BH * (Npad / 64), 3);
    if (d == 128) transpose_codes_kernel<128><<<grid, 256, 0, s>>>(j0, j1, j2, Npad);
    else transpose_codes_kernel<64><<<grid, 256, 0, s>>>(j0, j1, j2, Npad);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BwdArgs a;
  a.qc = b.qc; a.qt = b.qt; a.qs = b.qs; a.qblk = b.qblk;
  a.kc = b.kc; a.kt = b.kt; a.ks = b.ks;
  a.vc = b.vc; a.vs = b.vs;
  a.gc = b.gc; a.gt = b.gt; a.gs = b.gs;
  a.ld = b.ld; a.dq = b.dq; a.dk = b.dk; a.dv = b.dv;
  a.N = N; a.Npad = Npad; a.BH = BH; a.sl2 = b.sl2; a.sm = b.sm;
  const dim3 grid(BH * (Npad / kBW)), block(256);
#define SAGE_BWD(D_, C_)                                  \
  do {                                                    \
    bwd_dkdv_kernel<D_, C_><<<grid, block, 0, s>>>(a, a.qs, a.ks, a.vs, a.gs);    \
    bwd_dq_kernel<D_, C_><<<grid, block, 0, s>>>(a, a.qs, a.ks, a.vs, a.gs);      \
  } while (0)
  if (d == 128) {
    if (b.causal) SAGE_BWD(128, true); else SAGE_BWD(128, false);
  } else {
    if (b.causal) SAGE_BWD(64, true); else SAGE_BWD(64, false);
  }
#undef SAGE_BWD
  return hipGetLastError();
}

}  // namespace sage
