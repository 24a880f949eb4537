// Quantization kernels for gfx950: the K channel mean, per-block INT8 codes,
// the transposed fp16 V used by the INT8 attention kernel, per-channel INT8 V
// for its INT8 P.V variant, and MXFP4
// (E2M1 + E8M0) codes. All of them are HBM-streaming kernels: 16-byte
// coalesced loads and stores, one pass over each input.
//
// Method (SageAttention page, "Approach"): subtract the mean of K across
// tokens (softmax is unchanged because every score row shifts by q.mu), then
// quantize Q and the smoothed K to INT8 with per-block or per-token scales.
// MXFP4 (SageAttention3 abstract; the MX format of its reference list):
// 32 elements share one power-of-two scale, elements are E2M1.
#include "sage_internal.h"

namespace sage {

// ---------------------------------------------------------------------------
// K channel mean: exact and order-independent. Every fp16 value is an integer
// multiple of 2^-24, so K * 2^24 is an integer below 2^41 and sums exactly in
// int64. mu = fp32(fp64(sum) * 2^-24 / N): one correctly rounded fp64
// division and one RNE conversion, identical however the sum was split.
// A thread first adds its own tokens in fp64: a sum of n such values is a
// multiple of 2^-24 below n * 2^16, exactly representable (53-bit
// significand) while n <= 8192, so every one of those additions is exact and
// the thread's sum, times 2^24, converts to the same int64 as the integer
// sum; n <= ksum_rows_per_thread(N) <= 4096 for every accepted N. Three VALU
// instructions per element (two widenings and the fp64 add) instead of an
// integer decode with a variable 64-bit shift.
// ---------------------------------------------------------------------------

// One 256-thread block of the column sums: chunk `bid` (head bid / nchunk).
template <int D>
__device__ __forceinline__ void ksum_partial_block(const uint16_t* __restrict__ k, long long* __restrict__ part,
                                                   int N, int chunk, int nchunk, int bid, long long (*red)[9]) {
  constexpr int TPR = D / 8;      // threads per token row, 8 channels (16 bytes) each
  constexpr int RPP = 256 / TPR;  // token rows per pass
  const int bh = bid / nchunk, ci = bid % nchunk;
  const int tid = threadIdx.x, cg = tid % TPR;
  const int n0 = ci * chunk, n1 = min(N, n0 + chunk);
  const uint16_t* src = k + static_cast<size_t>(bh) * N * D + cg * 8;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int n = n0 + tid / TPR; n < n1; n += RPP) {
    const uint4 raw = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(n) * D);
    const unsigned w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += static_cast<double>(static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[j] & 0xffffu))));
      acc[2 * j + 1] += static_cast<double>(static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[j] >> 16))));
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red[tid][j] = static_cast<long long>(acc[j] * 0x1p24);
  __syncthreads();
  if (tid < D) {
    const int g = tid / 8, j = tid % 8;
    long long s = 0;
    for (int r = 0; r < RPP; ++r) s += red[r * TPR + g][j];
    part[(static_cast<size_t>(bh) * nchunk + ci) * D + tid] = s;
  }
}

template <int D>
__global__ __launch_bounds__(256) void ksum_partial_kernel(const uint16_t* __restrict__ k,
                                                           long long* __restrict__ part, int N,
                                                           int chunk, int nchunk) {
  __shared__ long long red[256][9];
  ksum_partial_block<D>(k, part, N, chunk, nchunk, blockIdx.x, red);
}

// mu from the partial sums: one block per (head, 32 channels), so that a
// head's chunks are added by 8 groups of 32 threads in parallel (a short
// chain of dependent loads per thread), then the 8 results by one group.
constexpr int kMeanCh = 32;
template <int D>
__global__ __launch_bounds__(256) void kmean_kernel(const long long* __restrict__ part,
                                                    float* __restrict__ mu_ws,
                                                    float* __restrict__ mu_out, int N, int nchunk) {
  constexpr int G = 256 / kMeanCh;  // chunk groups reduced in parallel
  __shared__ long long red[256];
  const int bh = blockIdx.x / (D / kMeanCh);
  const int cl = threadIdx.x % kMeanCh, c = (blockIdx.x % (D / kMeanCh)) * kMeanCh + cl, grp = threadIdx.x / kMeanCh;
  long long s = 0;
  for (int i = grp; i < nchunk; i += G) s += part[(static_cast<size_t>(bh) * nchunk + i) * D + c];
  red[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x < kMeanCh) {
    long long t = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) t += red[g * kMeanCh + cl];  // integer: order is irrelevant
    const float mu = static_cast<float>((static_cast<double>(t) * 0x1p-24) / static_cast<double>(N));
    mu_ws[static_cast<size_t>(bh) * D + c] = mu;
    if (mu_out) mu_out[static_cast<size_t>(bh) * D + c] = mu;
  }
}

hipError_t launch_kmean(const void* k, long long* ksum, float* kmean_ws, float* kmean_out, int BH,
                        int N, int d, int chunk, int nchunk, hipStream_t s) {
  const auto* kk = static_cast<const uint16_t*>(k);
  if (d == 128) {
    ksum_partial_kernel<128><<<BH * nchunk, 256, 0, s>>>(kk, ksum, N, chunk, nchunk);
    kmean_kernel<128><<<BH * (128 / kMeanCh), 256, 0, s>>>(ksum, kmean_ws, kmean_out, N, nchunk);
  } else {
    ksum_partial_kernel<64><<<BH * nchunk, 256, 0, s>>>(kk, ksum, N, chunk, nchunk);
    kmean_kernel<64><<<BH * (64 / kMeanCh), 256, 0, s>>>(ksum, kmean_ws, kmean_out, N, nchunk);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-block INT8 quantization. A workgroup owns 128 token rows of one head.
// Per block of `blk` rows: a = max|x|, s = fp32(a / 127) (IEEE division),
// code = rint(fp32(x / s)) (ties to even); a = 0 gives s = 0 and zero codes.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void unpack8(const uint4 raw, float* x) {
  const unsigned w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[j] & 0xffffu)));
    x[2 * j + 1] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[j] >> 16)));
  }
}

// x from the lane the DPP control CTRL names (all rows and banks enabled).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// fp32(v) - mu for the 8 fp16 values in raw, one mixed-precision fma each:
// v is widened inside the fma and multiplied by `one` (an fp16 1.0 the
// compiler cannot see as a constant, so it keeps the fma form), which is exact,
// so the result is the single rounding of fp32(v) - mu.
__device__ __forceinline__ void unpack8_sub(const uint4 raw, const float* mu, _Float16 one, float* x) {
  const unsigned w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const _Float16 lo = __builtin_bit_cast(_Float16, static_cast<uint16_t>(w[j] & 0xffffu));
    const _Float16 hi = __builtin_bit_cast(_Float16, static_cast<uint16_t>(w[j] >> 16));
    x[2 * j] = __builtin_fmaf(static_cast<float>(lo), static_cast<float>(one), -mu[2 * j]);
    x[2 * j + 1] = __builtin_fmaf(static_cast<float>(hi), static_cast<float>(one), -mu[2 * j + 1]);
  }
}

// One 256-thread block of a quantization job: TR-row tile `bid` (head bid /
// J.ntile), TR = 128 or 64 (64-row tiles hold half the registers, for jobs
// with blocks of at most 64 rows).
template <int D, int TR = kQTile>
__device__ __forceinline__ void int8_quant_block(const Int8Job& J, int N, int bid, float* rmax, float* bmax) {
  static_assert(TR == 128 || TR == 64, "tile rows");
  constexpr int TPR = D / 8;         // threads per row
  constexpr int RPP = 256 / TPR;     // rows per pass
  constexpr int NP = TR / RPP;       // passes per tile
  const int bh = bid / J.ntile, tile = bid % J.ntile;
  const int tid = threadIdx.x, cg = tid % TPR, rl = tid / TPR;
  const int row0 = tile * TR;
  const uint16_t* src = static_cast<const uint16_t*>(J.src) + static_cast<size_t>(bh) * N * D + cg * 8;

  float mu[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (J.mu) {
    const float4* m4 = reinterpret_cast<const float4*>(J.mu + static_cast<size_t>(bh) * D + cg * 8);
    const float4 a = m4[0], b = m4[1];
    mu[0] = a.x; mu[1] = a.y; mu[2] = a.z; mu[3] = a.w;
    mu[4] = b.x; mu[5] = b.y; mu[6] = b.z; mu[7] = b.w;
  }

  // the tile stays in registers as fp16 (4 registers per 8 values); the fp32
  // values x - mu are formed once for the maxima and again for the codes
  uint4 raw[NP];
  float lm[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int row = row0 + p * RPP + rl;
    raw[p] = row < N ? *reinterpret_cast<const uint4*>(src + static_cast<size_t>(row) * D) : make_uint4(0, 0, 0, 0);
  }
  // x = fp32(v) - mu (one RNE subtraction; mu = 0 if off), zero for rows >= N
  // (only the last tile of a head can hold such rows)
  _Float16 one = 1;
  asm volatile("" : "+v"(one));
  const bool full = row0 + TR <= N;
  auto values = [&](int p, float* x) {
    unpack8_sub(raw[p], mu, one, x);
    if (!full) {
      const bool live = row0 + p * RPP + rl < N;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = live ? x[e] : 0.f;
    }
  };
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    float x[8];
    values(p, x);
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
    // max over the TPR consecutive lanes that share this row, by DPP lane
    // swaps: pairs, then quad halves, then the two quads of each 8 lanes
    // (half-row mirror), then the two halves of each 16 (row mirror)
    m = fmaxf(m, dpp_f32<0xB1>(m));
    m = fmaxf(m, dpp_f32<0x4E>(m));
    m = fmaxf(m, dpp_f32<0x141>(m));
    if (TPR == 16) m = fmaxf(m, dpp_f32<0x140>(m));
    lm[p] = m;
  }
  // an empty asm that claims to change the raw registers: the compiler then
  // forms x - mu again below instead of keeping all 8 * NP fp32 values live
#pragma unroll
  for (int p = 0; p < NP; ++p) asm volatile("" : "+v"(raw[p].x), "+v"(raw[p].y), "+v"(raw[p].z), "+v"(raw[p].w));

  const int blk = J.blk;
  float s[NP];
  if (blk == 1) {
#pragma unroll
    for (int p = 0; p < NP; ++p) s[p] = lm[p] / 127.0f;
  } else {
#pragma unroll
    for (int p = 0; p < NP; ++p)
      if (cg == 0) rmax[p * RPP + rl] = lm[p];
    __syncthreads();
    // block maxima by one wave: lane i holds rows i and i + 64, then a
    // butterfly over the lanes of each block (blk is a power of two, <= TR)
    if (tid < 64) {
      float m0 = rmax[tid], m1 = TR == 128 ? rmax[tid + 64] : 0.f;
      if (blk >= 128) m0 = m1 = fmaxf(m0, m1);
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        if (off < blk) {
          m0 = fmaxf(m0, __shfl_xor(m0, off, 64));
          m1 = fmaxf(m1, __shfl_xor(m1, off, 64));
        }
      }
      if (tid % blk == 0) {
        bmax[tid / blk] = m0;
        if (TR == 128 && blk < 128) bmax[(tid + 64) / blk] = m1;
      }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < NP; ++p) s[p] = bmax[(p * RPP + rl) / blk] / 127.0f;
  }

#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int row = row0 + p * RPP + rl;
    if (row < J.code_rows) {
      const float sp = s[p];
      float x[8];
      values(p, x);
      unsigned w[8];
      if (sp >= kMarksteinMinScale) {
        const float y = 1.0f / sp;
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = int8_code_bits(x[e], sp, y);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = int8_code_bits_div(x[e], sp);
      }
      *reinterpret_cast<uint2*>(J.codes + (static_cast<size_t>(bh) * J.code_rows + row) * D + cg * 8) =
          make_uint2(pack_low_bytes(w[0], w[1], w[2], w[3]), pack_low_bytes(w[4], w[5], w[6], w[7]));
    }
  }

  // scales
  if (blk == 1) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int row = row0 + p * RPP + rl;
      if (cg == 0 && row < J.nscale) J.scales[static_cast<size_t>(bh) * J.nscale + row] = s[p];
    }
  } else {
    const int nb = TR / blk;
    const int bi = tile * nb + tid;
    if (tid < nb && bi < J.nscale) J.scales[static_cast<size_t>(bh) * J.nscale + bi] = bmax[tid] / 127.0f;
  }
}

template <int D, int TR = kQTile>
__global__ __launch_bounds__(256) void int8_quant_kernel(Int8Job j0, Int8Job j1, int N) {
  __shared__ float rmax[kQTile];
  __shared__ float bmax[kQTile];
  int8_quant_block<D, TR>(blockIdx.y ? j1 : j0, N, blockIdx.x, rmax, bmax);
}

hipError_t launch_int8_quant(const Int8Job& j0, const Int8Job& j1, int BH, int N, int d, hipStream_t s) {
  // Both jobs cover the same rows per head, so they share the tile count.
  dim3 grid(BH * j0.ntile, 2);
  if (d == 128) int8_quant_kernel<128><<<grid, 256, 0, s>>>(j0, j1, N);
  else int8_quant_kernel<64><<<grid, 256, 0, s>>>(j0, j1, N);
  return hipGetLastError();
}

constexpr int kVTile = 64;  // tokens per INT8 V tile

// ---------------------------------------------------------------------------
// INT8 V for the INT8 P.V variant: one scale per (head, channel) over all
// tokens, a = max|V|, s = fp32(a / 127) (IEEE division), code =
// rint(fp32(V / s)) (ties to even), with the per-block rules above. Pass 1
// takes the channel maxima of chunks of tokens; pass 2 finishes the maxima,
// writes the scales and the codes transposed, V^T [BH, d, ldv] int8 with
// tokens >= N zero. |V| is compared on the fp16 bit patterns with the sign
// cleared, which orders finite values like their magnitudes.
// ---------------------------------------------------------------------------

template <int D>
__device__ __forceinline__ void vmax_partial_block(const uint16_t* __restrict__ v, unsigned* __restrict__ part,
                                                   int N, int chunk, int nchunk, int bid, unsigned (*red)[9]) {
  constexpr int TPR = D / 8;      // threads per token row, 8 channels (16 bytes) each
  constexpr int RPP = 256 / TPR;  // token rows per pass
  const int bh = bid / nchunk, ci = bid % nchunk;
  const int tid = threadIdx.x, cg = tid % TPR;
  const int n0 = ci * chunk, n1 = min(N, n0 + chunk);
  const uint16_t* src = v + static_cast<size_t>(bh) * N * D + cg * 8;
  unsigned acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int n = n0 + tid / TPR; n < n1; n += RPP) {
    const uint4 raw = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(n) * D);
    const unsigned w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] = max(acc[2 * j], w[j] & 0x7fffu);
      acc[2 * j + 1] = max(acc[2 * j + 1], (w[j] >> 16) & 0x7fffu);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red[tid][j] = acc[j];
  __syncthreads();
  if (tid < D) {
    const int g = tid / 8, j = tid % 8;
    unsigned m = 0;
    for (int r = 0; r < RPP; ++r) m = max(m, red[r * TPR + g][j]);
    part[(static_cast<size_t>(bh) * nchunk + ci) * D + tid] = m;
  }
}

template <int D>
__global__ __launch_bounds__(256) void vmax_partial_kernel(const uint16_t* __restrict__ v,
                                                           unsigned* __restrict__ part, int N,
                                                           int chunk, int nchunk) {
  __shared__ unsigned red[256][9];
  vmax_partial_block<D>(v, part, N, chunk, nchunk, blockIdx.x, red);
}

template <int D>
__device__ __forceinline__ void v_int8_block(const uint16_t* __restrict__ v, const unsigned* __restrict__ part,
                                             int8_t* __restrict__ codes, float* __restrict__ scales, int N,
                                             int nchunk, int ldv, int bid, uint16_t (*t)[D + 8], float* sc) {
  constexpr int TT = kVTile;  // tokens per tile
  constexpr int CPR = D / 8;  // 16-byte chunks per token row
  const int ntile = (ldv + TT - 1) / TT;
  const int bh = bid / ntile, tb = bid % ntile;
  const int tid = threadIdx.x;
  if (tid < D) {
    // the channel's partial maxima, eight independent loads at a time (a
    // chain of one load per chunk made long heads latency-bound)
    const unsigned* pp = part + static_cast<size_t>(bh) * nchunk * D + tid;
    unsigned m = 0;
    int i = 0;
    for (; i + 8 <= nchunk; i += 8) {
      unsigned r[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = pp[(i + j) * D];
#pragma unroll
      for (int j = 0; j < 8; ++j) m = max(m, r[j]);
    }
    for (; i < nchunk; ++i) m = max(m, pp[i * D]);
    const float a = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(m)));
    const float s = a / 127.0f;
    sc[tid] = s;
    if (tb == 0) scales[static_cast<size_t>(bh) * D + tid] = s;
  }
  const uint16_t* src = v + static_cast<size_t>(bh) * N * D;
#pragma unroll
  for (int u = 0; u < TT * CPR / 256; ++u) {
    const int i = tid + 256 * u, r = i / CPR, c8 = i % CPR;
    const int n = tb * TT + r;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (n < N) val = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(n) * D + c8 * 8);
    *reinterpret_cast<uint4*>(&t[r][c8 * 8]) = val;
  }
  __syncthreads();
  // every thread writes 16 consecutive tokens of one channel per pass
#pragma unroll
  for (int u = 0; u < D * (TT / 16) / 256; ++u) {
    const int i = tid + 256 * u, dd = i / (TT / 16), n16 = i % (TT / 16);
    const int n0 = tb * TT + n16 * 16;
    if (n0 >= ldv) continue;
    const float s = sc[dd];
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = static_cast<float>(__builtin_bit_cast(_Float16, t[n16 * 16 + j][dd]));
    unsigned w[16];
    if (s >= kMarksteinMinScale) {
      const float y = 1.0f / s;
#pragma unroll
      for (int j = 0; j < 16; ++j) w[j] = int8_code_bits(x[j], s, y);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) w[j] = int8_code_bits_div(x[j], s);
    }
    *reinterpret_cast<uint4*>(codes + (static_cast<size_t>(bh) * D + dd) * ldv + n0) =
        make_uint4(pack_low_bytes(w[0], w[1], w[2], w[3]), pack_low_bytes(w[4], w[5], w[6], w[7]),
                   pack_low_bytes(w[8], w[9], w[10], w[11]), pack_low_bytes(w[12], w[13], w[14], w[15]));
  }
}

template <int D>
__global__ __launch_bounds__(256) void v_int8_kernel(const uint16_t* __restrict__ v,
                                                     const unsigned* __restrict__ part,
                                                     int8_t* __restrict__ codes, float* __restrict__ scales,
                                                     int N, int nchunk, int ldv) {
  __shared__ uint16_t t[kVTile][D + 8];
  __shared__ float sc[D];
  v_int8_block<D>(v, part, codes, scales, N, nchunk, ldv, blockIdx.x, t, sc);
}

hipError_t launch_v_int8(const void* v, unsigned* part, int8_t* codes, float* scales, int BH, int N, int ldv,
                         int d, int chunk, int nchunk, hipStream_t s) {
  const auto* vv = static_cast<const uint16_t*>(v);
  const int grid = BH * ((ldv + 63) / 64);
  if (d == 128) {
    vmax_partial_kernel<128><<<BH * nchunk, 256, 0, s>>>(vv, part, N, chunk, nchunk);
    v_int8_kernel<128><<<grid, 256, 0, s>>>(vv, part, codes, scales, N, nchunk, ldv);
  } else {
    vmax_partial_kernel<64><<<BH * nchunk, 256, 0, s>>>(vv, part, N, chunk, nchunk);
    v_int8_kernel<64><<<grid, 256, 0, s>>>(vv, part, codes, scales, N, nchunk, ldv);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The prepare phase of the INT8 modes: (1) the K column sums and the Q codes
// share one grid, as neither depends on the other; (2) the K mean;
// (3) the K codes; for INT8 V, (4) its channel maxima and (5) its codes. The
// INT8 V passes keep launches of their own: in a shared grid their blocks are
// held to the occupancy of the quantization blocks' registers, which measured
// slower. Each block runs the same code as the standalone kernels.
// ---------------------------------------------------------------------------

constexpr int kPrepSmem = 256 * 9 * 8;  // the largest of the blocks' LDS needs

template <int D>
__global__ __launch_bounds__(256) void prep_int8_phase1_kernel(PrepInt8 P, int N, int n_ksum, int n_q) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kPrepSmem];
  const auto* k = static_cast<const uint16_t*>(P.k);
  int bid = blockIdx.x;
  if (bid < n_ksum) {
    ksum_partial_block<D>(k, P.ksum, N, P.chunk, P.nchunk, bid, reinterpret_cast<long long (*)[9]>(smem));
    return;
  }
  bid -= n_ksum;
  if (bid < n_q)
    int8_quant_block<D>(P.jq, N, bid, reinterpret_cast<float*>(smem), reinterpret_cast<float*>(smem) + kQTile);
}

hipError_t launch_prepare_int8(const PrepInt8& P, int BH, int N, int d, hipStream_t s) {
  const int n_ksum = P.smooth ? BH * P.nchunk : 0;
  const int n_q = BH * P.jq.ntile;   // 0 when the attention kernel quantizes Q itself
  // K codes in 64-row tiles (K blocks are 64 rows or one row): half the
  // registers of a 128-row tile, so twice the waves in flight
  Int8Job jk = P.jk;
  jk.ntile = P.jk.ntile * (kQTile / 64);
  const dim3 grid_k(BH * jk.ntile, 1);
  if (n_ksum + n_q > 0) {
    if (d == 128) prep_int8_phase1_kernel<128><<<n_ksum + n_q, 256, 0, s>>>(P, N, n_ksum, n_q);
    else prep_int8_phase1_kernel<64><<<n_ksum + n_q, 256, 0, s>>>(P, N, n_ksum, n_q);
  }
  if (P.smooth) {
    if (d == 128) kmean_kernel<128><<<BH * (128 / kMeanCh), 256, 0, s>>>(P.ksum, P.kmean, nullptr, N, P.nchunk);
    else kmean_kernel<64><<<BH * (64 / kMeanCh), 256, 0, s>>>(P.ksum, P.kmean, nullptr, N, P.nchunk);
  }
  if (d == 128) int8_quant_kernel<128, 64><<<grid_k, 256, 0, s>>>(jk, jk, N);
  else int8_quant_kernel<64, 64><<<grid_k, 256, 0, s>>>(jk, jk, N);
  if (P.vmax) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_v_int8(P.v, P.vmax, static_cast<int8_t*>(P.vt), P.vscale, BH, N, P.Npad, d, P.chunk, P.nchunk, s);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MXFP4: per 32-element block, e = floor(log2 max|x|) - 2 clamped to
// [-127, 127] (0 for an all-zero block), E8M0 byte e + 127, and every element
// the E2M1 value nearest to x * 2^-e with ties to the even code, saturating at
// 6. The E2M1 magnitudes are 0, .5, 1, 1.5, 2, 3, 4, 6; their midpoints .25,
// .75, 1.25, 1.75, 2.5, 3.5, 5 go down at even-below (.25, 1.25, 2.5, 5) and
// up at odd-below (.75, 1.75, 3.5), hence the mix of > and >= below.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  const int E = static_cast<int>((__float_as_uint(amax) >> 23) & 0xffu);  // amax >= 0
  const int e = E - 129;  // floor(log2 a) - 2 for a normal a
  return e < -127 ? -127 : e;
}

__device__ __forceinline__ unsigned e2m1_code(float x, int e) {
  const float y = ldexpf(fabsf(x), -e);  // exact power-of-two scaling
  const unsigned c = static_cast<unsigned>(y > 0.25f) + static_cast<unsigned>(y >= 0.75f) +
                     static_cast<unsigned>(y > 1.25f) + static_cast<unsigned>(y >= 1.75f) +
                     static_cast<unsigned>(y > 2.5f) + static_cast<unsigned>(y >= 3.5f) +
                     static_cast<unsigned>(y > 5.0f);
  return c | ((__float_as_uint(x) >> 28) & 8u);  // sign bit of x
}

// Quantizes 32 floats: 16 packed bytes (element 2i in the low nibble) + exponent byte.
// With a normal scale 2^e (e >= -126) the codes come from the hardware
// conversion v_cvt_scalef32_pk_fp4_f32 (x / 2^e, round to nearest even,
// saturating at 6, sign of x kept, first operand in the low nibble), two
// values per instruction; the comparison ladder above covers e = -127.
__device__ __forceinline__ uint4 mx_block(const float* x, unsigned& e8) {
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(x[i]));
  const int e = mx_exponent(a);
  e8 = static_cast<unsigned>(e + 127);
  unsigned w[4] = {0, 0, 0, 0};
  if (e >= -126) {
    const float scale = __uint_as_float(e8 << 23);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      unsigned r = 0;
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[8 * k + 0], x[8 * k + 1], scale, 0);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[8 * k + 2], x[8 * k + 3], scale, 1);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[8 * k + 4], x[8 * k + 5], scale, 2);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[8 * k + 6], x[8 * k + 7], scale, 3);
      w[k] = r;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) w[i / 8] |= e2m1_code(x[i], e) << (4 * (i % 8));
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// 256 consecutive 32-element row blocks of a job (one per thread), starting at block 256 * bid.
template <int D>
__device__ __forceinline__ void mx_rows_block(const MxRowJob& J, int BH, int N, int bid) {
  constexpr int NB = D / 32;  // blocks per row
  const long long gb = static_cast<long long>(bid) * 256 + threadIdx.x;
  const long long per_head = static_cast<long long>(J.rows) * NB;
  if (gb >= per_head * BH) return;
  const int bh = static_cast<int>(gb / per_head);
  const int rem = static_cast<int>(gb % per_head);
  const int row = rem / NB, db = rem % NB;
  float x[32];
  if (row < N) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(J.src) +
                                                    (static_cast<size_t>(bh) * N + row) * D + db * 32);
    if (J.mu) {
      const float* m = J.mu + static_cast<size_t>(bh) * D + db * 32;
      _Float16 one = 1;
      asm volatile("" : "+v"(one));
#pragma unroll
      for (int u = 0; u < 4; ++u) unpack8_sub(p[u], m + 8 * u, one, x + 8 * u);
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) unpack8(p[u], x + 8 * u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = 0.f;
  }
  unsigned e8;
  const uint4 packed = mx_block(x, e8);
  const size_t r = static_cast<size_t>(bh) * J.rows + row;
  *reinterpret_cast<uint4*>(J.fp4 + r * (D / 2) + db * 16) = packed;
  J.e8[r * NB + db] = static_cast<uint8_t>(e8);
}

template <int D>
__global__ __launch_bounds__(256) void mx_rows_kernel(MxRowJob j0, MxRowJob j1, int BH, int N) {
  mx_rows_block<D>(blockIdx.y ? j1 : j0, BH, N, blockIdx.x);
}

inline unsigned mx_rows_blocks(const MxRowJob& j, int BH, int d) {
  return static_cast<unsigned>((static_cast<long long>(BH) * j.rows * (d / 32) + 255) / 256);
}

hipError_t launch_mx_rows(const MxRowJob& j0, const MxRowJob& j1, int BH, int N, int d, hipStream_t s) {
  dim3 grid(mx_rows_blocks(j0, BH, d), 2);
  if (d == 128) mx_rows_kernel<128><<<grid, 256, 0, s>>>(j0, j1, BH, N);
  else mx_rows_kernel<64><<<grid, 256, 0, s>>>(j0, j1, BH, N);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MX-FP8 (E4M3 elements) for V, the accuracy variant of the FP4 path: per
// block of 32 tokens of one channel, e = floor(log2 max|x|) - 8 clamped to
// [-127, 127] (0 for an all-zero block), element = nearest E4M3 value to
// x * 2^-e with ties to even, saturating at 448. The rounding is the hardware
// conversion (v_cvt_scalef32_pk_fp8_f32: divides by the power-of-two scale,
// rounds to nearest even); it turns values past 448 into NaN, so they are
// clamped to +-448 * 2^e first.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int mx_exponent8(float amax) {
  if (!(amax > 0.f)) return 0;
  const int E = static_cast<int>((__float_as_uint(amax) >> 23) & 0xffu);
  const int e = E - 135;  // floor(log2 a) - 8 for a normal a
  return e < -127 ? -127 : e;
}

typedef short v2s_t __attribute__((ext_vector_type(2)));

// 32 floats -> 32 E4M3 bytes (element i in byte i) + exponent byte.
__device__ __forceinline__ void mx_block8(const float* x, uint4& lo, uint4& hi, unsigned& e8) {
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(x[i]));
  const int e = mx_exponent8(a);
  e8 = static_cast<unsigned>(e + 127);
  const float scale = ldexpf(1.f, e);
  const float lim = 448.f * scale;
  unsigned w[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    v2s_t r = {0, 0};
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, fminf(fmaxf(x[4 * k], -lim), lim),
                                                 fminf(fmaxf(x[4 * k + 1], -lim), lim), scale, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, fminf(fmaxf(x[4 * k + 2], -lim), lim),
                                                 fminf(fmaxf(x[4 * k + 3], -lim), lim), scale, true);
    w[k] = __builtin_bit_cast(unsigned, r);
  }
  lo = make_uint4(w[0], w[1], w[2], w[3]);
  hi = make_uint4(w[4], w[5], w[6], w[7]);
}

// V^T in MX blocks of 32 tokens per channel: one tile of TT tokens, every
// thread owns one (channel, 32-token block). Neighbouring threads own the
// blocks of one channel, so their code stores are contiguous. FP8: E4M3
// codes (one byte each), else packed E2M1.
template <int D, bool FP8>
__device__ __forceinline__ void mx_vt_block(const uint16_t* __restrict__ v, uint8_t* __restrict__ codes,
                                            uint8_t* __restrict__ e8, int N, int Nv, int bid, uint16_t (*t)[D + 2]) {
  constexpr int TT = 256 * 32 / D;  // tokens per tile
  constexpr int NBT = TT / 32;      // 32-token blocks per tile
  constexpr int CPR = D / 8;
  const int ntile = (Nv + TT - 1) / TT;
  const int bh = bid / ntile, tb = bid % ntile;
  const int tid = threadIdx.x;
  const uint16_t* src = v + static_cast<size_t>(bh) * N * D;
#pragma unroll
  for (int u = 0; u < TT * CPR / 256; ++u) {
    const int i = tid + 256 * u, r = i / CPR, c8 = i % CPR;
    const int n = tb * TT + r;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (n < N) val = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(n) * D + c8 * 8);
    const unsigned w[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      t[r][c8 * 8 + 2 * j] = static_cast<uint16_t>(w[j] & 0xffffu);
      t[r][c8 * 8 + 2 * j + 1] = static_cast<uint16_t>(w[j] >> 16);
    }
  }
  __syncthreads();
  const int c = tid / NBT, b = tid % NBT;
  const int n0 = tb * TT + b * 32;
  if (n0 >= Nv) return;
  float x[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = static_cast<float>(__builtin_bit_cast(_Float16, t[b * 32 + i][c]));
  unsigned eb;
  const size_t rowc = static_cast<size_t>(bh) * D + c;
  if (FP8) {
    uint4 lo, hi;
    mx_block8(x, lo, hi, eb);
    *reinterpret_cast<uint4*>(codes + rowc * Nv + n0) = lo;
    *reinterpret_cast<uint4*>(codes + rowc * Nv + n0 + 16) = hi;
  } else {
    *reinterpret_cast<uint4*>(codes + rowc * (Nv / 2) + n0 / 2) = mx_block(x, eb);
  }
  e8[rowc * (Nv / 32) + n0 / 32] = static_cast<uint8_t>(eb);
}

template <int D, bool FP8>
__global__ __launch_bounds__(256) void mx_vt_kernel(const uint16_t* __restrict__ v, uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ e8, int N, int Nv) {
  __shared__ uint16_t t[256 * 32 / D][D + 2];
  mx_vt_block<D, FP8>(v, codes, e8, N, Nv, blockIdx.x, t);
}

hipError_t launch_mx_vt8(const void* v, uint8_t* fp8, uint8_t* e8, int BH, int N, int Nv, int d, hipStream_t s) {
  const int TT = 256 * 32 / d;
  const int grid = BH * ((Nv + TT - 1) / TT);
  if (d == 128) mx_vt_kernel<128, true><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(v), fp8, e8, N, Nv);
  else mx_vt_kernel<64, true><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(v), fp8, e8, N, Nv);
  return hipGetLastError();
}

hipError_t launch_mx_vt(const void* v, uint8_t* fp4, uint8_t* e8, int BH, int N, int Nv, int d, hipStream_t s) {
  const int TT = 256 * 32 / d;
  const int grid = BH * ((Nv + TT - 1) / TT);
  if (d == 128) mx_vt_kernel<128, false><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(v), fp4, e8, N, Nv);
  else mx_vt_kernel<64, false><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(v), fp4, e8, N, Nv);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The prepare phase of the MXFP4 modes, like the INT8 one: (1) the K column
// sums, the Q codes and the V^T codes share one grid; (2) the K mean; (3) the
// K codes.
// ---------------------------------------------------------------------------

template <int D, bool FP8>
__global__ __launch_bounds__(256) void prep_mx_phase1_kernel(PrepMx P, int N, int n_ksum, int n_q) {
  static_assert(256 * 32 / D * (D + 2) * 2 <= kPrepSmem, "LDS");
  __shared__ __attribute__((aligned(16))) unsigned char smem[kPrepSmem];
  int bid = blockIdx.x;
  if (bid < n_ksum) {
    ksum_partial_block<D>(static_cast<const uint16_t*>(P.k), P.ksum, N, P.chunk, P.nchunk, bid,
                          reinterpret_cast<long long (*)[9]>(smem));
    return;
  }
  bid -= n_ksum;
  if (bid < n_q) {
    mx_rows_block<D>(P.jq, P.BH, N, bid);
    return;
  }
  bid -= n_q;
  mx_vt_block<D, FP8>(static_cast<const uint16_t*>(P.v), P.vt, P.vte8, N, P.Nv, bid,
                      reinterpret_cast<uint16_t (*)[D + 2]>(smem));
}

hipError_t launch_prepare_mx(const PrepMx& P, int N, int d, hipStream_t s) {
  const int BH = P.BH;
  const int n_ksum = P.smooth ? BH * P.nchunk : 0;
  const int n_q = static_cast<int>(mx_rows_blocks(P.jq, BH, d));
  const int TT = 256 * 32 / d;
  const int n_v = BH * ((P.Nv + TT - 1) / TT);
  const int grid = n_ksum + n_q + n_v;
#define SAGE_PHASE1(D_, F_) prep_mx_phase1_kernel<D_, F_><<<grid, 256, 0, s>>>(P, N, n_ksum, n_q)
  if (d == 128) { if (P.v_fp8) SAGE_PHASE1(128, true); else SAGE_PHASE1(128, false); }
  else { if (P.v_fp8) SAGE_PHASE1(64, true); else SAGE_PHASE1(64, false); }
#undef SAGE_PHASE1
  if (P.smooth) {
    if (d == 128) kmean_kernel<128><<<BH * (128 / kMeanCh), 256, 0, s>>>(P.ksum, P.kmean, nullptr, N, P.nchunk);
    else kmean_kernel<64><<<BH * (64 / kMeanCh), 256, 0, s>>>(P.ksum, P.kmean, nullptr, N, P.nchunk);
  }
  const dim3 grid_k(mx_rows_blocks(P.jk, BH, d), 1);
  if (d == 128) mx_rows_kernel<128><<<grid_k, 256, 0, s>>>(P.jk, P.jk, BH, N);
  else mx_rows_kernel<64><<<grid_k, 256, 0, s>>>(P.jk, P.jk, BH, N);
  return hipGetLastError();
}

}  // namespace sage
