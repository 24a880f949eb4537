// Fused INT8 attention kernel for gfx950 (CDNA4).
//
// Computes, per head, O = softmax(sm_scale * dequant(Qc Kc^T)) V from the
// INT8 codes and per-block scales of Q and the mean-smoothed K, with P and V
// in FP16 for P.V (SageAttention page, "Approach" and summary paragraph) and
// the softmax taken online over key tiles, FlashAttention-2 style ("Experimental
// setup: builds on FlashAttention-2 ... online softmax").
//
// Work decomposition
//   * one workgroup = 4 waves = 128 query rows of one head; wave w owns rows
//     q0 + 32w .. q0 + 32w + 31; key tiles of 64 keys are staged in LDS
//     (double-buffered) and shared by the 4 waves.
//   * scores are computed transposed, S^T = K Q^T, on v_mfma_i32_32x32x32_i8:
//     in the 32x32 accumulator layout every lane owns one query column
//     (lane % 32) and 16 key rows, so the row max and row sum of the softmax
//     are in-lane reductions plus one swap between lanes l and l + 32.
//   * K rows are placed in LDS in a permuted order so that, after the score
//     MFMA, lane group g = lane / 32 holds exactly keys g*32 .. g*32+31 of the
//     tile, in order. Those fp32 values, rounded to fp16, are already the
//     B operand of O^T = V^T P^T on v_mfma_f32_32x32x16_f16: no shuffle and no
//     LDS round trip for P.
//   * O^T accumulates in fp32 (CDNA4's FP16 matrix op accumulates in FP32; the
//     page reports no accuracy difference between FP16 and FP32 accumulators).
//   * softmax in base 2: the dequantization scale s_q * s_k * sm_scale * log2(e)
//     is one fp32 multiply per score; P = exp2(S - m) on v_exp_f32.
//   * causal: key tiles wholly above the workgroup's last query are skipped;
//     masking runs only on tiles that cross the diagonal or the ragged tail.
#include "sage_internal.h"

#include <math.h>

namespace sage {

namespace {

// LDS row (0..63) holding key k of a 64-key tile. Row t*32 + r feeds row r of
// score MFMA t; its accumulator register i of lane group g is row
// (i/4)*8 + g*4 + i%4, and the placement below makes that key g*32 + t*16 + i.
__device__ __forceinline__ int lds_row_of_key(int k) {
  const int g = k >> 5, t = (k >> 4) & 1, i = k & 15;
  return t * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
}

// Combines a per-lane value with the one in lane l ^ 32 (same query column).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

template <int D, bool CAUSAL, bool PERTOK>
__global__ __launch_bounds__(256, 2) void attn_int8_kernel(
    const int8_t* __restrict__ qc, const int8_t* __restrict__ kc, const _Float16* __restrict__ vt,
    const float* __restrict__ qs, const float* __restrict__ ks, _Float16* __restrict__ out, int N,
    int Npad, int qblk, float sl2, int BH) {
  constexpr int NC = D / 32;            // 32-channel chunks of the score contraction
  constexpr int KROW = D + 16;          // LDS bytes per K row (16 bytes of padding)
  constexpr int VROW = kKTile * 2 + 16; // LDS bytes per V^T row
  constexpr int KT_BYTES = kKTile * KROW;
  constexpr int VT_BYTES = D * VROW;
  constexpr int BUF = KT_BYTES + VT_BYTES;
  constexpr int KCH = kKTile * D / 16 / 256;  // 16-byte K chunks per thread per tile
  constexpr int VCH = D * 8 / 256;            // 16-byte V^T chunks per thread per tile
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF];

  const int nqt = Npad / kQTile;
  int bh, qt;
  map_workgroup(blockIdx.x, BH, nqt, CAUSAL, bh, qt);
  const int q0 = qt * kQTile;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int qrow = q0 + wave * 32 + l32;

  // Q codes of this lane's query: the B operand of the score MFMAs, kept in registers.
  v4i qf[NC];
  {
    const int8_t* qp = qc + (static_cast<size_t>(bh) * Npad + qrow) * D + g * 16;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = *reinterpret_cast<const v4i*>(qp + c * 32);
  }
  // Q scale: one per block of qblk rows (a wave never straddles two), or per row.
  const int nqs = Npad / qblk;
  const float sq = qs[static_cast<size_t>(bh) * nqs + (PERTOK ? qrow : (q0 + wave * 32) / qblk)];
  // K scale: one per 64-key block (= one key tile), or one per key.
  const int nks = PERTOK ? Npad : Npad / kKTile;
  const float* ksh = ks + static_cast<size_t>(bh) * nks;

  int nkt = (N + kKTile - 1) / kKTile;
  if (CAUSAL) nkt = min(nkt, (q0 + kQTile) / kKTile);

  const int8_t* kbase = kc + static_cast<size_t>(bh) * Npad * D;
  const _Float16* vbase = vt + static_cast<size_t>(bh) * D * Npad;
  // Global -> register staging of one key tile (K codes and V^T), then
  // register -> LDS. The K rows go to their permuted LDS rows. (Arrays of
  // scalars, not of uint4, so the compiler keeps them in registers.)
  unsigned kr[4 * KCH], vr[4 * VCH];
#define SAGE_GLOAD(J_)                                                                               \
  do {                                                                                               \
    _Pragma("unroll") for (int u = 0; u < KCH; ++u) {                                                \
      const int i_ = tid + 256 * u, row_ = i_ / (D / 16), col_ = i_ % (D / 16);                      \
      const uint4 t_ = *reinterpret_cast<const uint4*>(kbase + static_cast<size_t>((J_) * kKTile + row_) * D + \
                                                       col_ * 16);                                   \
      kr[4 * u] = t_.x; kr[4 * u + 1] = t_.y; kr[4 * u + 2] = t_.z; kr[4 * u + 3] = t_.w;           \
    }                                                                                                \
    _Pragma("unroll") for (int u = 0; u < VCH; ++u) {                                                \
      const int i_ = tid + 256 * u, row_ = i_ >> 3, col_ = i_ & 7;                                   \
      const uint4 t_ = *reinterpret_cast<const uint4*>(vbase + static_cast<size_t>(row_) * Npad +    \
                                                       (J_) * kKTile + col_ * 8);                    \
      vr[4 * u] = t_.x; vr[4 * u + 1] = t_.y; vr[4 * u + 2] = t_.z; vr[4 * u + 3] = t_.w;           \
    }                                                                                                \
  } while (0)
#define SAGE_SWRITE(BUF_)                                                                            \
  do {                                                                                               \
    unsigned char* kt_ = smem + (BUF_) * BUF;                                                        \
    unsigned char* vl_ = kt_ + KT_BYTES;                                                             \
    _Pragma("unroll") for (int u = 0; u < KCH; ++u) {                                                \
      const int i_ = tid + 256 * u, row_ = i_ / (D / 16), col_ = i_ % (D / 16);                      \
      *reinterpret_cast<uint4*>(kt_ + lds_row_of_key(row_) * KROW + col_ * 16) =                     \
          make_uint4(kr[4 * u], kr[4 * u + 1], kr[4 * u + 2], kr[4 * u + 3]);                        \
    }                                                                                                \
    _Pragma("unroll") for (int u = 0; u < VCH; ++u) {                                                \
      const int i_ = tid + 256 * u, row_ = i_ >> 3, col_ = i_ & 7;                                   \
      *reinterpret_cast<uint4*>(vl_ + row_ * VROW + col_ * 16) =                                     \
          make_uint4(vr[4 * u], vr[4 * u + 1], vr[4 * u + 2], vr[4 * u + 3]);                        \
    }                                                                                                \
  } while (0)

  v16f o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[c][i] = 0.f;
  float m = -INFINITY, l = 0.f;

  SAGE_GLOAD(0);
  SAGE_SWRITE(0);
  __syncthreads();

  for (int j = 0; j < nkt; ++j) {
    const int buf = j & 1;
    if (j + 1 < nkt) SAGE_GLOAD(j + 1);
    const unsigned char* kt = smem + buf * BUF;
    const unsigned char* vl = kt + KT_BYTES;

    // S^T = K Q^T for keys j*64 .. j*64+63 (two 32-key halves t)
    v16i s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[t][i] = 0;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const v4i a = *reinterpret_cast<const v4i*>(kt + (t * 32 + l32) * KROW + c * 32 + g * 16);
        s[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qf[c], s[t], 0, 0, 0);
      }
    }

    // dequantize into base-2 logits; p[t*16+i] is key j*64 + g*32 + t*16 + i
    float p[32];
    if (PERTOK) {
      const float sc = sq * sl2;
      const float4* k4 = reinterpret_cast<const float4*>(ksh + j * kKTile + g * 32);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float4 kk = k4[u];
        const int e = 4 * u;
        p[e] = static_cast<float>(s[e >> 4][e & 15]) * sc * kk.x;
        p[e + 1] = static_cast<float>(s[(e + 1) >> 4][(e + 1) & 15]) * sc * kk.y;
        p[e + 2] = static_cast<float>(s[(e + 2) >> 4][(e + 2) & 15]) * sc * kk.z;
        p[e + 3] = static_cast<float>(s[(e + 3) >> 4][(e + 3) & 15]) * sc * kk.w;
      }
    } else {
      const float sc = sq * ksh[j] * sl2;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) p[t * 16 + i] = static_cast<float>(s[t][i]) * sc;
    }
    const bool diag = CAUSAL && (j * kKTile + kKTile - 1 > q0 + wave * 32);
    const bool tail = (j * kKTile + kKTile > N);
    if (diag || tail) {
      const int kb = j * kKTile + g * 32;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int key = kb + e;
        if ((CAUSAL && key > qrow) || key >= N) p[e] = -INFINITY;
      }
    }

    // online softmax (base 2)
    float mx = p[0];
#pragma unroll
    for (int e = 1; e < 32; ++e) mx = fmaxf(mx, p[e]);
    mx = pair_max(mx);
    const float mnew = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      p[e] = __builtin_amdgcn_exp2f(p[e] - mnew);
      rs += p[e];
    }
    l = l * alpha + rs;
    m = mnew;

    // P -> fp16 (RNE); pf[c] holds keys g*32 + c*8 .. +7
    v8h pf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[c][e] = static_cast<_Float16>(p[c * 8 + e]);

    // O^T = alpha * O^T + V^T P^T
    if (__ballot(alpha != 1.f)) {  // wave-uniform: skip when no row max moved
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[c][i] *= alpha;
    }
#pragma unroll
    for (int dt = 0; dt < NC; ++dt) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const v8h a = *reinterpret_cast<const v8h*>(vl + (dt * 32 + l32) * VROW + (g * 32 + c * 8) * 2);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[c], o[dt], 0, 0, 0);
      }
    }

    if (j + 1 < nkt) SAGE_SWRITE(buf ^ 1);
    __syncthreads();
  }

  // epilogue: O = O^T / l, rows >= N are padding and are not stored
  const float inv = 1.f / pair_sum(l);
  if (qrow < N) {
    _Float16* orow = out + (static_cast<size_t>(bh) * N + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < NC; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v4h h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = static_cast<_Float16>(o[dt][r * 4 + i] * inv);
        *reinterpret_cast<v4h*>(orow + dt * 32 + r * 8 + g * 4) = h;
      }
  }
}

#undef SAGE_GLOAD
#undef SAGE_SWRITE

hipError_t launch_attn_int8(const AttnArgs& a, const int8_t* qc, const int8_t* kc, const void* vt,
                            const float* qs, const float* ks, hipStream_t s) {
  const int nqt = a.Npad / kQTile;
  const dim3 grid(a.BH * nqt), block(256);
  const int qblk = (a.mode == 0) ? 128 : (a.mode == 1 ? 64 : 1);
  const bool pt = (a.mode == 3);
  const auto* v = static_cast<const _Float16*>(vt);
  auto* o = static_cast<_Float16*>(a.out);
#define SAGE_LAUNCH(D_, C_, P_) \
  attn_int8_kernel<D_, C_, P_><<<grid, block, 0, s>>>(qc, kc, v, qs, ks, o, a.N, a.Npad, qblk, a.sl2, a.BH)
  if (a.d == 128) {
    if (a.causal) { if (pt) SAGE_LAUNCH(128, true, true); else SAGE_LAUNCH(128, true, false); }
    else { if (pt) SAGE_LAUNCH(128, false, true); else SAGE_LAUNCH(128, false, false); }
  } else {
    if (a.causal) { if (pt) SAGE_LAUNCH(64, true, true); else SAGE_LAUNCH(64, true, false); }
    else { if (pt) SAGE_LAUNCH(64, false, true); else SAGE_LAUNCH(64, false, false); }
  }
#undef SAGE_LAUNCH
  return hipGetLastError();
}

}  // namespace sage
