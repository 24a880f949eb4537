// Fused microscaled-FP4 attention kernel for gfx950 (CDNA4).
//
// The SageAttention3 abstract's idea (attention with microscaled FP4
// operands on FP4 matrix units) on CDNA4's block-scaled MFMA
// v_mfma_scale_f32_32x32x64_f8f6f4: Q, the mean-smoothed K, V and the softmax
// P are E2M1 with one E8M0 exponent per 32 elements of the contraction
// dimension (d for Q K^T, keys for P V), accumulation in FP32.
//
// Same decomposition as the INT8 kernel: 4 waves x 32 query rows per
// workgroup, 64-key tiles in LDS (double-buffered), scores computed as
// S^T = K Q^T so each lane owns one query column; the permuted K row
// placement leaves lane group g holding keys g*32 .. g*32+31 of the tile,
// which is exactly one MX block of P for the B operand of O^T = V^T P^T. P is
// therefore quantized in registers: block max (in-lane), shared exponent
// e = floor(log2 max) - 2, and v_cvt_scalef32_pk_fp4_f32 (RNE, saturating)
// for the E2M1 codes.
#include "sage_internal.h"

#include <math.h>

namespace sage {

namespace {

typedef short v2s __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lds_row_of_key4(int k) {
  const int g = k >> 5, t = (k >> 4) & 1, i = k & 15;
  return t * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
}

// The next float below x (x finite).
__device__ __forceinline__ float below_ulp4(float x) {
  if (x == 0.f) return -0x1p-149f;
  return __uint_as_float(__float_as_uint(x) + (x > 0.f ? 0xffffffffu : 1u));
}

// Maxima of scores use the NaN-propagating maximum: the same result as fmaxf
// on finite and infinite values, without the quieting of possible signaling
// NaNs that fmaxf costs on matrix-op results.
__device__ __forceinline__ float max4(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float pair_max4(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max4(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum4(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void map_workgroup4(int bid, int BH, int nqt, bool causal, int& bh, int& qt) {
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

// 32x32x64 FP4 x FP4 block-scaled MFMA; the scale exponents are byte SEL of sa
// and of sb (the matrix op's op_sel picks the byte: checked on the GPU).
template <int SEL>
__device__ __forceinline__ v16f mfma_fp4(const v4i a, const v4i b, unsigned sa, unsigned sb, v16f c) {
  const v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  const v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, SEL, static_cast<int>(sa), SEL,
                                                          static_cast<int>(sb));
}

}  // namespace

// PV8: P and V in MX-FP8 (E4M3) instead of MXFP4 (the accuracy variant; Q and
// K_s stay MXFP4). The P.V matrix op then takes 32 bytes of each operand per
// lane (format code 0 = E4M3), laid out (measured on the GPU) as keys g*16 ..
// g*16+15 and 32 + g*16 .. 32+g*16+15 for lane group g, with the block scale
// of keys 32b .. 32b+31 taken from lane group b.
// Two workgroups per CU; three for the MX-FP8 P.V instance at d = 64, which
// fits in 168 registers (+9% at the video_dit shape; the FP4 one spills there
// and measured 13% slower).
template <int D, bool CAUSAL, bool PV8>
__global__ __launch_bounds__(256, (D == 64 && PV8) ? 3 : 2) void attn_mxfp4_kernel(
    const uint8_t* __restrict__ q4, const uint8_t* __restrict__ qe, const uint8_t* __restrict__ k4,
    const uint8_t* __restrict__ ke, const uint8_t* __restrict__ v4, const uint8_t* __restrict__ ve,
    _Float16* __restrict__ out, int N, int Npad, float sl2, int BH) {
  constexpr int NC = D / 64;         // 64-channel steps of the score contraction
  constexpr int NE = D / 32;         // exponent bytes per Q / K row
  constexpr int NT = D / 32;         // 32-row tiles of O^T
  // The K and V^T rows are unpadded and their 16-byte chunks are permuted
  // within the row (XOR swizzle), so that the 16 lanes of one LDS access
  // phase hit distinct banks both when a tile is stored (lanes write whole
  // rows) and when the matrix ops read it (lanes read one chunk of 16
  // consecutive rows). At d = 64 a K row is 32 bytes and the rows one store
  // phase writes (keys 8q .. 8q+7) would share bank slots, so K rows are
  // also placed in a permuted slot order within each group of 16. The MX-FP8
  // P.V instance at d = 64 keeps padded rows instead: the swizzle's address
  // registers would not fit its 168 (three workgroups per CU).
  constexpr bool SWZ = !(PV8 && D == 64);
  constexpr int KROW = SWZ ? D / 2 : D / 2 + 16;   // LDS bytes per K row
  constexpr int VTB = PV8 ? 64 : 32;  // bytes of one V^T row per key tile (64 keys)
  constexpr int VROW = SWZ ? VTB : VTB + 16;       // LDS bytes per V^T row
  constexpr int KT_BYTES = kKTile * KROW;
  constexpr int KS_BYTES = kKTile * 8;  // per K row: its exponent word, and the word >> 8
  constexpr int VT_BYTES = D * VROW;
  constexpr int VS_BYTES = D * 8;       // per V^T row: likewise
  constexpr int BUF = KT_BYTES + KS_BYTES + VT_BYTES + VS_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF];
  // LDS slot of K row p, and the position of data chunk c of K row p / V^T row r
  const auto kslot = [](int p) { return (SWZ && D == 64) ? p ^ (((p >> 3) & 1) << 2) : p; };
  const auto kpos = [](int p, int c) { return !SWZ ? c : D == 128 ? (c ^ ((p >> 2) & 3)) : (c ^ ((p >> 3) & 1)); };
  const auto vpos = [](int r, int c) { return !SWZ ? c : PV8 ? (c ^ ((r >> 2) & 3)) : (c ^ ((r >> 3) & 1)); };

  const int nqt = Npad / kQTile;
  int bh, qt;
  map_workgroup4(blockIdx.x, BH, nqt, CAUSAL, bh, qt);
  const int q0 = qt * kQTile;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int qrow = q0 + wave * 32 + l32;
  const size_t row_q = static_cast<size_t>(bh) * Npad + qrow;

  v4i qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) qf[c] = *reinterpret_cast<const v4i*>(q4 + row_q * (D / 2) + c * 32 + g * 16);
  unsigned qsw;  // exponent bytes of this query row, shifted so block c*2+g sits at byte 2c
  if (NE == 4) qsw = *reinterpret_cast<const unsigned*>(qe + row_q * 4);
  else qsw = *reinterpret_cast<const uint16_t*>(qe + row_q * 2);
  qsw >>= 8 * g;

  int nkt = (N + kKTile - 1) / kKTile;
  if (CAUSAL) nkt = min(nkt, (q0 + kQTile) / kKTile);

  const uint8_t* kb4 = k4 + static_cast<size_t>(bh) * Npad * (D / 2);
  const uint8_t* kbe = ke + static_cast<size_t>(bh) * Npad * NE;
  const int vrb = PV8 ? Npad : Npad / 2;  // bytes per V^T row in HBM
  const uint8_t* vb4 = v4 + static_cast<size_t>(bh) * D * vrb;
  const uint8_t* vbe = ve + static_cast<size_t>(bh) * D * (Npad / 32);
  // the tile loads are buffer loads: a per-lane offset fixed for the whole loop
  // and the tile's offset in a scalar register
  const auto rk4 = buffer_rsrc(kb4, static_cast<unsigned>(Npad) * (D / 2));
  const auto rke = buffer_rsrc(kbe, static_cast<unsigned>(Npad) * NE);
  const auto rv4 = buffer_rsrc(vb4, static_cast<unsigned>(D) * vrb);
  const auto rve = buffer_rsrc(vbe, static_cast<unsigned>(D) * (Npad / 32));

  // staging registers, two sets (tiles are loaded two iterations ahead): one
  // 16-byte K chunk, one K exponent word, one 16-byte V^T chunk, one V^T exponent pair
  constexpr int KCHUNKS = kKTile * D / 32;  // 16-byte chunks per K tile (256 or 128)
  constexpr int VCPR = VTB / 16;            // 16-byte chunks per V^T row of a tile
  constexpr int VCHUNKS = D * VCPR;         // 16-byte chunks per V^T tile
  constexpr int VPT4 = (VCHUNKS + 255) / 256;
  unsigned kr[2][4], vr[2][4 * VPT4];
  unsigned ksr[2] = {0, 0}, vsr[2] = {0, 0};
  // per-lane byte offsets of this thread's chunks within a tile (every thread
  // loads; threads beyond a tile's chunk count repeat an in-bounds chunk)
  int k_off, ke_off, ve_off, v_off[VPT4];
  {
    const int i = tid % KCHUNKS;
    k_off = (i / (D / 32)) * (D / 2) + (i % (D / 32)) * 16;
    ke_off = (tid % kKTile) * NE;
    ve_off = (tid % D) * (Npad / 32);
#pragma unroll
    for (int u = 0; u < VPT4; ++u) {
      const int c = (tid + 256 * u) % VCHUNKS;
      v_off[u] = (c / VCPR) * vrb + (c % VCPR) * 16;
    }
  }
// Global loads of tile J_ (clamped to the last tile, so the loop issues them
  // unconditionally) into staging set S_. Every thread loads (threads beyond a
  // tile's chunk count repeat an in-bounds chunk and do not store it): the code
  // stays branch-free, so the compiler's counter waits before the LDS stores
  // wait only for the loads they need, not for the newer prefetch.
#define SAGE_GLOAD4(J_, S_)                                                                          \
  do {                                                                                               \
    const int jj_ = min((J_), nkt - 1);                                                              \
    {                                                                                                \
      const auto t_ = __builtin_amdgcn_raw_buffer_load_b128(rk4, k_off, jj_ * (kKTile * D / 2), 0);  \
      kr[S_][0] = t_[0]; kr[S_][1] = t_[1]; kr[S_][2] = t_[2]; kr[S_][3] = t_[3];                    \
    }                                                                                                \
    ksr[S_] = (NE == 4) ? __builtin_amdgcn_raw_buffer_load_b32(rke, ke_off, jj_ * (kKTile * NE), 0)   \
                        : static_cast<unsigned>(__builtin_amdgcn_raw_buffer_load_b16(rke, ke_off,   \
                                                                                  jj_ * (kKTile * NE), 0)); \
    _Pragma("unroll") for (int u_ = 0; u_ < VPT4; ++u_) {                                           \
      const auto t_ = __builtin_amdgcn_raw_buffer_load_b128(rv4, v_off[u_], jj_ * VTB, 0);           \
      vr[S_][4 * u_] = t_[0]; vr[S_][4 * u_ + 1] = t_[1]; vr[S_][4 * u_ + 2] = t_[2]; vr[S_][4 * u_ + 3] = t_[3]; \
    }                                                                                                \
    vsr[S_] = __builtin_amdgcn_raw_buffer_load_b16(rve, ve_off, jj_ * 2, 0);                          \
  } while (0)
#define SAGE_SWRITE4(BUF_, S_)                                                                       \
  do {                                                                                               \
    unsigned char* kt_ = smem + (BUF_) * BUF;                                                        \
    unsigned char* ks_ = kt_ + KT_BYTES;                                                             \
    unsigned char* vl_ = ks_ + KS_BYTES;                                                             \
    unsigned char* vs_ = vl_ + VT_BYTES;                                                             \
    if (tid < KCHUNKS) {                                                                             \
      const int row_ = lds_row_of_key4(tid / (D / 32)), col_ = tid % (D / 32);                       \
      *reinterpret_cast<uint4*>(kt_ + kslot(row_) * KROW + kpos(row_, col_) * 16) =                  \
          make_uint4(kr[S_][0], kr[S_][1], kr[S_][2], kr[S_][3]);                                    \
    }                                                                                                \
    if (tid < kKTile) *reinterpret_cast<uint2*>(ks_ + lds_row_of_key4(tid) * 8) = make_uint2(ksr[S_], ksr[S_] >> 8); \
    _Pragma("unroll") for (int u_ = 0; u_ < VPT4; ++u_) {                                           \
      const int i_ = tid + 256 * u_;                                                                 \
      if (i_ < VCHUNKS) {                                                                            \
        const int row_ = i_ / VCPR, col_ = i_ % VCPR;                                                \
        *reinterpret_cast<uint4*>(vl_ + row_ * VROW + vpos(row_, col_) * 16) =                       \
            make_uint4(vr[S_][4 * u_], vr[S_][4 * u_ + 1], vr[S_][4 * u_ + 2], vr[S_][4 * u_ + 3]);  \
      }                                                                                              \
    }                                                                                                \
    if (tid < D) *reinterpret_cast<uint2*>(vs_ + tid * 8) = make_uint2(vsr[S_], vsr[S_] >> 8);      \
  } while (0)

  // o[NT] is the row sum: the quantized P times a block of ones, accumulated
  // and rescaled with O^T (every one of its rows holds l of the lane's query)
  v16f o[NT + 1];
#pragma unroll
  for (int c = 0; c < NT + 1; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[c][i] = 0.f;
  float m = -INFINITY;
  // the block of ones of the row-sum matrix op (E2M1 1.0 = 0x2, E4M3 1.0 =
  // 0x38 in every element), kept in registers (asm values are not
  // rematerialized for every tile), except where the 8 registers of the E4M3
  // block would not fit (MX-FP8 P.V at d = 64, three workgroups per CU)
  constexpr bool KEEP8 = PV8 && D == 128;
  v4i ones4;
  v8i ones8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (KEEP8) asm volatile("v_mov_b32 %0, 0x38383838" : "=v"(ones8[i]));
    else ones8[i] = 0x38383838;
    if (i < 4) {
      if (PV8) ones4[i] = 0;
      else asm volatile("v_mov_b32 %0, 0x22222222" : "=v"(ones4[i]));
    }
  }

  // One key tile (J_) from LDS buffer BUF_: scores, softmax, P quantization, P.V.
#define SAGE_TILE4(J_, BUF_)                                                                         \
  do {                                                                                               \
    const int j = (J_);                                                                              \
    const int buf = (BUF_);                                                                          \
    const unsigned char* kt = smem + buf * BUF;                                                     \
    const unsigned char* ksl = kt + KT_BYTES;                                                       \
    const unsigned char* vl = ksl + KS_BYTES;                                                       \
    const unsigned char* vsl = vl + VT_BYTES;                                                       \
                                                                                                    \
    /* S^T = K_s Q^T on the block-scaled FP4 MFMA (scores come out dequantized) */                  \
    v16f s[2];                                                                                      \
_Pragma("unroll")                                                                                   \
    for (int t = 0; t < 2; ++t) {                                                                   \
_Pragma("unroll")                                                                                   \
      for (int i = 0; i < 16; ++i) s[t][i] = 0.f;                                                   \
      const int krow = t * 32 + l32;                                                                \
      const unsigned ksw = *reinterpret_cast<const unsigned*>(ksl + krow * 8 + g * 4);              \
_Pragma("unroll")                                                                                   \
      for (int c = 0; c < NC; ++c) {                                                                \
        const v4i a = *reinterpret_cast<const v4i*>(kt + kslot(krow) * KROW + kpos(krow, c * 2 + g) * 16); \
        /* block c*2+g of the K row and of the Q row: byte 2c of ksw and qsw */                     \
        s[t] = (c == 0) ? mfma_fp4<0>(a, qf[c], ksw, qsw, s[t]) : mfma_fp4<2>(a, qf[c], ksw, qsw, s[t]); \
      }                                                                                             \
    }                                                                                               \
                                                                                                    \
    /* softmax on the raw scores: the max is taken before the sm_scale * log2(e) */                \
    /* factor (> 0), which one fma per score applies with the max subtraction */                    \
    float p[32];                                                                                    \
_Pragma("unroll")                                                                                   \
    for (int t = 0; t < 2; ++t)                                                                     \
_Pragma("unroll")                                                                                   \
      for (int i = 0; i < 16; ++i) p[t * 16 + i] = s[t][i];                                         \
    const bool diag = CAUSAL && (j * kKTile + kKTile - 1 > q0 + wave * 32);                         \
    const bool tail = (j * kKTile + kKTile > N);                                                    \
    if (diag || tail) {                                                                             \
      const int kb = j * kKTile + g * 32;                                                           \
_Pragma("unroll")                                                                                   \
      for (int e = 0; e < 32; ++e) {                                                                \
        const int key = kb + e;                                                                     \
        if ((CAUSAL && key > qrow) || key >= N) p[e] = -INFINITY;                                   \
      }                                                                                             \
    }                                                                                               \
                                                                                                    \
    float lmx = p[0];                                                                               \
_Pragma("unroll")                                                                                   \
    for (int e = 1; e < 32; ++e) lmx = max4(lmx, p[e]);                                             \
    const float mxr = pair_max4(lmx);                                                               \
    float mx = mxr * sl2;                                                                           \
    /* round the new reference down when the product rounded up: the row's */                      \
    /* largest score then gets P >= 1 (its exact value is 1), so the block */                       \
    /* exponent of P cannot drop a binade below the exact one */                                    \
    if (__builtin_fmaf(mxr, sl2, -mx) < 0.f) mx = below_ulp4(mx);                                   \
    /* P is formed against the running max, so its MX codes are the method's */                    \
    const bool need = mx > m;                                                                       \
    const float mnew = need ? mx : m;                                                               \
    const float alpha = need ? __builtin_amdgcn_exp2f(m - mnew) : 1.f;                              \
    const float nm = -mnew;                                                                         \
_Pragma("unroll")                                                                                   \
    for (int e = 0; e < 32; ++e) p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(p[e], sl2, nm));     \
    /* the block max of P is the P of the lane's largest score: the same fma and */                 \
    /* exp2 on the same operands (0 for a fully masked lane) */                                     \
    const float pmax = __builtin_amdgcn_exp2f(__builtin_fmaf(lmx, sl2, nm));                        \
    m = mnew;                                                                                       \
                                                                                                    \
    /* MX-quantize this lane's 32 P values (one block of 32 keys): */                              \
    /* e = floor(log2 pmax) - 2 (E2M1) or - 8 (E4M3), floored at -126 */                            \
    /* (blocks below 2^-118 are negligible). E4M3 values past 448 saturate */                       \
    /* (the conversion itself would give NaN). */                                                   \
    unsigned pe8 = 127;                                                                             \
    float pscale = 1.f;                                                                             \
    if (pmax > 0.f) {                                                                               \
      const int E = static_cast<int>(__float_as_uint(pmax) >> 23);                                  \
      const int e = max(E - (PV8 ? 135 : 129), -126);                                               \
      pe8 = static_cast<unsigned>(e + 127);                                                         \
      pscale = __uint_as_float(pe8 << 23);                                                          \
    }                                                                                               \
    v8i pq;                                                                                         \
    if (PV8) {                                                                                      \
      const float plim = 448.f * pscale;                                                            \
      _Pragma("unroll") for (int w = 0; w < 8; ++w) {                                               \
        /* both halves are written below: no zeroing */                                           \
        v2s r = __builtin_nondeterministic_value(r);                                                \
        r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, fminf(p[4 * w], plim), fminf(p[4 * w + 1], plim), pscale, false); \
        r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, fminf(p[4 * w + 2], plim), fminf(p[4 * w + 3], plim), pscale, true); \
        pq[w] = __builtin_bit_cast(int, r);                                                         \
      }                                                                                             \
      /* the FP8 operand of the matrix op takes keys g*16 .. +15 in bytes 0-15 and */               \
      /* 32 + g*16 .. +15 in bytes 16-31 (the block scale of keys 32b .. 32b+31 */                 \
      /* comes from lane group b): swap keys 16-31 of group 0 with 32-47 of group 1 */              \
      _Pragma("unroll") for (int w = 0; w < 4; ++w) {                                               \
        const auto x_ = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(pq[w]),              \
                                                         static_cast<unsigned>(pq[4 + w]), false, false); \
        pq[w] = static_cast<int>(x_[0]);                                                            \
        pq[4 + w] = static_cast<int>(x_[1]);                                                        \
      }                                                                                             \
    } else {                                                                                        \
      _Pragma("unroll") for (int w = 0; w < 4; ++w) {                                               \
        unsigned r = __builtin_nondeterministic_value(r);  /* all four bytes are written below */  \
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, p[8 * w + 0], p[8 * w + 1], pscale, 0);     \
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, p[8 * w + 2], p[8 * w + 3], pscale, 1);     \
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, p[8 * w + 4], p[8 * w + 5], pscale, 2);     \
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, p[8 * w + 6], p[8 * w + 7], pscale, 3);     \
        pq[w] = static_cast<int>(r);                                                                \
      }                                                                                             \
      pq[4] = pq[5] = pq[6] = pq[7] = 0;                                                            \
    }                                                                                               \
                                                                                                    \
    if (__ballot(need)) {                                                                           \
_Pragma("unroll")                                                                                   \
      for (int c = 0; c < NT; ++c)                                                                  \
_Pragma("unroll")                                                                                   \
        for (int i = 0; i < 16; ++i) o[c][i] *= alpha;                                              \
      /* every row of the row-sum product holds l; only register 0 is read */                       \
      o[NT][0] *= alpha;                                                                            \
    }                                                                                               \
_Pragma("unroll")                                                                                   \
    for (int dt = 0; dt < NT; ++dt) {                                                               \
      const int vrow = dt * 32 + l32;                                                               \
      const unsigned vsw = *reinterpret_cast<const unsigned*>(vsl + vrow * 8 + g * 4);              \
      if (PV8) {                                                                                    \
        /* keys g*16 .. +15 and 32 + g*16 .. +15 of the tile (see the P swap) */                    \
        const v4i a0 = *reinterpret_cast<const v4i*>(vl + vrow * VROW + vpos(vrow, g) * 16);        \
        const v4i a1 = *reinterpret_cast<const v4i*>(vl + vrow * VROW + vpos(vrow, 2 + g) * 16);    \
        const v8i a8 = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};                    \
        o[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, pq, o[dt], 0, 0, 0,            \
                                                                static_cast<int>(vsw), 0,           \
                                                                static_cast<int>(pe8));             \
      } else {                                                                                      \
        const v4i a = *reinterpret_cast<const v4i*>(vl + vrow * VROW + vpos(vrow, g) * 16);         \
        o[dt] = mfma_fp4<0>(a, v4i{pq[0], pq[1], pq[2], pq[3]}, vsw, pe8, o[dt]);                   \
      }                                                                                             \
    }                                                                                               \
    /* row sum of the quantized P: ones (E4M3 0x38 or E2M1 0x2, scale 2^0) times P */              \
    if (PV8) {                                                                                      \
      o[NT] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones8, pq, o[NT], 0, 0, 0, 127, 0,   \
                                                              static_cast<int>(pe8));               \
    } else {                                                                                        \
      o[NT] = mfma_fp4<0>(ones4, v4i{pq[0], pq[1], pq[2], pq[3]}, 127u, pe8, o[NT]);              \
    }                                                                                               \
  } while (0)

  // Tiles are loaded into registers two iterations ahead (two staging sets)
  // and stored to LDS one iteration ahead (two LDS buffers), so a tile's
  // global loads have a whole iteration to arrive before they are stored.
  SAGE_GLOAD4(0, 0);
  SAGE_SWRITE4(0, 0);
  SAGE_GLOAD4(1, 1);
  lds_barrier();
  int j2 = 0;
  for (; j2 + 1 < nkt; j2 += 2) {
    SAGE_GLOAD4(j2 + 2, 0);
    SAGE_TILE4(j2, 0);
    SAGE_SWRITE4(1, 1);
    lds_barrier();
    SAGE_GLOAD4(j2 + 3, 1);
    SAGE_TILE4(j2 + 1, 1);
    SAGE_SWRITE4(0, 0);   /* tile min(j2 + 2, nkt - 1): unused after the last tile */
    lds_barrier();
  }
  if (j2 < nkt) SAGE_TILE4(j2, 0);
#undef SAGE_TILE4
#undef SAGE_GLOAD4
#undef SAGE_SWRITE4

  const float inv = 1.f / o[NT][0];
  if (qrow < N) {
    _Float16* orow = out + (static_cast<size_t>(bh) * N + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < NT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v4h h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = static_cast<_Float16>(o[dt][r * 4 + i] * inv);
        *reinterpret_cast<v4h*>(orow + dt * 32 + r * 8 + g * 4) = h;
      }
  }
}

hipError_t launch_attn_mxfp4(const AttnArgs& a, const uint8_t* q4, const uint8_t* qe,
                             const uint8_t* k4, const uint8_t* ke, const uint8_t* v4,
                             const uint8_t* ve, hipStream_t s) {
  const int nqt = a.Npad / kQTile;
  const dim3 grid(a.BH * nqt), block(256);
  auto* o = static_cast<_Float16*>(a.out);
  const bool pv8 = (a.mode == 5);
#define SAGE_LAUNCH4(D_, C_, P_) \
  attn_mxfp4_kernel<D_, C_, P_><<<grid, block, 0, s>>>(q4, qe, k4, ke, v4, ve, o, a.N, a.Npad, a.sl2, a.BH)
#define SAGE_LAUNCH4_PV(D_, C_)                         \
  do {                                                  \
    if (pv8) SAGE_LAUNCH4(D_, C_, true);                \
    else SAGE_LAUNCH4(D_, C_, false);                   \
  } while (0)
  if (a.d == 128) {
    if (a.causal) SAGE_LAUNCH4_PV(128, true); else SAGE_LAUNCH4_PV(128, false);
  } else {
    if (a.causal) SAGE_LAUNCH4_PV(64, true); else SAGE_LAUNCH4_PV(64, false);
  }
#undef SAGE_LAUNCH4_PV
#undef SAGE_LAUNCH4
  return hipGetLastError();
}

}  // namespace sage
