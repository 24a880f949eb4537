// C ABI of the quantized-attention library (declared in include/sage_attn.h):
// argument validation, workspace sizing, device check and kernel dispatch.
// Every argument is validated before the first HIP runtime call, so argument
// errors are reported identically on hosts without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "sage_attn.h"
#include "sage_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

constexpr int kMaxN = 1 << 22;
static_assert(sage::ksum_rows_per_thread(kMaxN) <= 8192, "K column sums: fp64 running sums must stay exact");
// INT8 P.V: the int32 P.V sums are at most 127 * 127 * N and must stay below 2^31.
constexpr int kMaxNPv8 = 1 << 17;

int check_dims(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return fail(SAGE_ERR_INVALID_ARG, "B, H and N must be >= 1 (got %d, %d, %d)", B, H, N);
  if (N > kMaxN) return fail(SAGE_ERR_INVALID_ARG, "N = %d exceeds the supported maximum %d", N, kMaxN);
  if (d != 64 && d != 128) return fail(SAGE_ERR_UNSUPPORTED, "head dim d = %d is not supported (64 or 128)", d);
  const long long bh = static_cast<long long>(B) * H;
  if (bh > (1LL << 24)) return fail(SAGE_ERR_INVALID_ARG, "B*H = %lld is too large", bh);
  // the largest grid is B*H*Npad/128 workgroups and the largest tensor B*H*Npad*d bytes*2
  const long long rows = bh * sage::round_up(N, sage::kRowPad);
  if (rows / sage::kQTile > 0x7fffffffLL || rows > (1LL << 40) / d)
    return fail(SAGE_ERR_INVALID_ARG, "problem too large (B*H*N = %lld)", bh * N);
  return SAGE_OK;
}

int check_ptr(const void* p, const char* name, size_t align) {
  if (!p) return fail(SAGE_ERR_INVALID_ARG, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % align) return fail(SAGE_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
  return SAGE_OK;
}

int check_mode(int mode, bool attention) {
  if (mode & ~(SAGE_MODE_MASK | SAGE_FLAG_NO_SMOOTH | SAGE_FLAG_FUSED_Q))
    return fail(SAGE_ERR_UNSUPPORTED, "unknown flag bits in mode 0x%x", mode);
  const int lo = mode & SAGE_MODE_MASK;
  if (lo > SAGE_MODE_INT8_PV_PER_TOKEN) return fail(SAGE_ERR_UNSUPPORTED, "unknown mode %d", lo);
  if ((mode & SAGE_FLAG_FUSED_Q) && lo != SAGE_MODE_INT8_Q128_K64 && lo != SAGE_MODE_INT8_Q64_K64)
    return fail(SAGE_ERR_UNSUPPORTED, "SAGE_FLAG_FUSED_Q goes with the per-block INT8 modes %d and %d (got %d)",
                SAGE_MODE_INT8_Q128_K64, SAGE_MODE_INT8_Q64_K64, lo);
  (void)attention;
  return SAGE_OK;
}

// The fused pass: the per-block INT8 modes quantize Q inside the attention
// kernel (its prologue), so the prepare phase writes no Q codes. Below 64K
// token rows (B * H * N) the prologue costs more than the Q pass it saves
// (measured: 9% slower at 2 x 256 rows, 0.6-1.3% faster from 512K rows on).
constexpr long long kFusedQMinRows = 1 << 16;
int with_fused_q(int mode, int B, int H, int N) {
  const int lo = mode & SAGE_MODE_MASK;
  const bool fuse = (lo == SAGE_MODE_INT8_Q128_K64 || lo == SAGE_MODE_INT8_Q64_K64) &&
                    static_cast<long long>(B) * H * N >= kFusedQMinRows;
  return fuse ? (mode | SAGE_FLAG_FUSED_Q) : (mode & ~SAGE_FLAG_FUSED_Q);
}

// Device check: a HIP device must be current and be gfx950. Cached per device.
std::atomic<int> g_arch_ok[64];

int check_device() {
  int dev = -1;
  int count = 0;
  const hipError_t ce = hipGetDeviceCount(&count);
  if (ce != hipSuccess || count < 1) {
    (void)hipGetLastError();
    return fail(SAGE_ERR_NO_DEVICE, "no HIP device is visible (hipGetDeviceCount: %s, count %d)",
                hipGetErrorString(ce), count);
  }
  const hipError_t de = hipGetDevice(&dev);
  if (de != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(SAGE_ERR_NO_DEVICE, "no current HIP device (hipGetDevice: %s)", hipGetErrorString(de));
  }
  if (dev < 64) {
    const int st = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (st == 1) return SAGE_OK;
    if (st == 2) return fail(SAGE_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(SAGE_ERR_HIP, "hipGetDeviceProperties failed on device %d", dev);
  }
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  if (!ok) return fail(SAGE_ERR_UNSUPPORTED, "device %d is %s, the kernels are built for gfx950", dev, prop.gcnArchName);
  return SAGE_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SAGE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return SAGE_OK;
}

#define SAGE_TRY(expr)              \
  do {                              \
    const int rc_ = (expr);         \
    if (rc_ != SAGE_OK) return rc_; \
  } while (0)

unsigned char* at(void* base, size_t off) { return static_cast<unsigned char*>(base) + off; }
const unsigned char* at(const void* base, size_t off) { return static_cast<const unsigned char*>(base) + off; }

int validate_attn(int B, int H, int N, int d, int mode, const void* ws, size_t ws_bytes) {
  SAGE_TRY(check_dims(B, H, N, d));
  SAGE_TRY(check_mode(mode, true));
  if (sage::mode_pv_int8(mode & SAGE_MODE_MASK) && N > kMaxNPv8)
    return fail(SAGE_ERR_UNSUPPORTED, "N = %d exceeds %d, the limit of the INT8 P.V modes", N, kMaxNPv8);
  SAGE_TRY(check_ptr(ws, "workspace", 256));
  const sage::Layout L = sage::make_layout(static_cast<long long>(B) * H, N, d, mode & SAGE_MODE_MASK, true);
  if (ws_bytes < L.total)
    return fail(SAGE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, L.total);
  return SAGE_OK;
}

// Modes whose attention kernel reads the caller's fp16 V (all but the MXFP4
// and INT8 P.V modes, which read V codes from the workspace).
bool reads_fp16_v(int mode_lo) {
  return !(mode_lo == SAGE_MODE_MXFP4 || mode_lo == SAGE_MODE_MXFP4_FP8PV || sage::mode_pv_int8(mode_lo));
}

int check_scale(float sm_scale) {
  if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return fail(SAGE_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  return SAGE_OK;
}

int do_prepare(const void* q, const void* k, const void* v, int B, int H, int N, int d, int mode,
               void* ws, hipStream_t s) {
  const int BH = B * H;
  const int lo = mode & SAGE_MODE_MASK;
  const bool smooth = !(mode & SAGE_FLAG_NO_SMOOTH);
  const sage::Layout L = sage::make_layout(BH, N, d, lo, true);
  (void)hipGetLastError();
  float* mu = reinterpret_cast<float*>(at(ws, L.kmean));
  if (lo == SAGE_MODE_FP16)  // unquantized baseline: the attention kernel reads Q, K and V as given
    return SAGE_OK;
  if (lo == SAGE_MODE_MXFP4 || lo == SAGE_MODE_MXFP4_FP8PV) {
    sage::PrepMx P;
    P.BH = BH; P.k = k; P.v = v; P.ksum = reinterpret_cast<long long*>(at(ws, L.ksum)); P.kmean = mu;
    P.chunk = L.chunk; P.nchunk = L.nchunk; P.smooth = smooth;
    P.jq.src = q; P.jq.fp4 = at(ws, L.q_fp4); P.jq.e8 = at(ws, L.q_e8); P.jq.mu = nullptr; P.jq.rows = L.Npad;
    P.jk.src = k; P.jk.fp4 = at(ws, L.k_fp4); P.jk.e8 = at(ws, L.k_e8); P.jk.mu = smooth ? mu : nullptr; P.jk.rows = L.Npad;
    P.vt = at(ws, L.vt_fp4); P.vte8 = at(ws, L.vt_e8); P.Nv = L.Npad; P.v_fp8 = lo == SAGE_MODE_MXFP4_FP8PV;
    return hip_status(sage::launch_prepare_mx(P, N, d, s), "MXFP4 prepare kernels");
  }
  const bool per_token = lo == SAGE_MODE_INT8_PER_TOKEN || lo == SAGE_MODE_INT8_PV_PER_TOKEN;
  const int blk_q = per_token ? 1 : (lo == SAGE_MODE_INT8_Q64_K64 ? 64 : 128);
  const int blk_k = per_token ? 1 : 64;
  sage::PrepInt8 P;
  P.k = k; P.v = v; P.ksum = reinterpret_cast<long long*>(at(ws, L.ksum)); P.kmean = mu;
  P.chunk = L.chunk; P.nchunk = L.nchunk; P.smooth = smooth; P.Npad = L.Npad;
  P.jq.src = q; P.jq.codes = reinterpret_cast<int8_t*>(at(ws, L.q_codes)); P.jq.scales = reinterpret_cast<float*>(at(ws, L.q_scales));
  P.jq.mu = nullptr; P.jq.blk = blk_q; P.jq.code_rows = L.Npad; P.jq.nscale = L.Npad / blk_q;
  P.jq.ntile = (mode & SAGE_FLAG_FUSED_Q) ? 0 : L.Npad / sage::kQTile;   // 0: no Q codes
  P.jk.src = k; P.jk.codes = reinterpret_cast<int8_t*>(at(ws, L.k_codes)); P.jk.scales = reinterpret_cast<float*>(at(ws, L.k_scales));
  P.jk.mu = smooth ? mu : nullptr; P.jk.blk = blk_k; P.jk.code_rows = L.Npad; P.jk.nscale = L.Npad / blk_k; P.jk.ntile = L.Npad / sage::kQTile;
  if (sage::mode_pv_int8(lo)) {
    P.vt = at(ws, L.vt);
    P.vmax = reinterpret_cast<unsigned*>(at(ws, L.vmax));
    P.vscale = reinterpret_cast<float*>(at(ws, L.vscale));
  }
  return hip_status(sage::launch_prepare_int8(P, BH, N, d, s), "INT8 prepare kernels");
}

int do_compute(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d, int causal, float sm_scale,
               int mode, const void* ws, hipStream_t s, float* lse = nullptr) {
  const int BH = B * H;
  const int lo = mode & SAGE_MODE_MASK;
  const sage::Layout L = sage::make_layout(BH, N, d, lo, true);
  sage::AttnArgs a;
  a.BH = BH; a.N = N; a.Npad = L.Npad; a.d = d; a.causal = causal != 0;
  a.sl2 = static_cast<float>(static_cast<double>(sm_scale) * 1.4426950408889634);  // sm_scale * log2(e)
  a.mode = lo; a.out = out; a.lse = lse;
  (void)hipGetLastError();
  if (lo == SAGE_MODE_MXFP4 || lo == SAGE_MODE_MXFP4_FP8PV)
    return hip_status(sage::launch_attn_mxfp4(a, at(ws, L.q_fp4), at(ws, L.q_e8), at(ws, L.k_fp4), at(ws, L.k_e8),
                                              at(ws, L.vt_fp4), at(ws, L.vt_e8), s), "MXFP4 attention kernel");
  if (lo == SAGE_MODE_FP16)
    return hip_status(sage::launch_attn_int8(a, q, k, v, nullptr, nullptr, nullptr, s),
                      "FP16 attention kernel");
  a.qin = (mode & SAGE_FLAG_FUSED_Q) != 0;
  return hip_status(sage::launch_attn_int8(a, a.qin ? q : at(ws, L.q_codes), at(ws, L.k_codes),
                                           sage::mode_pv_int8(lo) ? at(ws, L.vt) : v,
                                           reinterpret_cast<const float*>(at(ws, L.q_scales)),
                                           reinterpret_cast<const float*>(at(ws, L.k_scales)),
                                           sage::mode_pv_int8(lo) ? reinterpret_cast<const float*>(at(ws, L.vscale))
                                                                  : nullptr, s),
                    "INT8 attention kernel");
}

// The training forward and the backward pass run the per-block INT8 modes.
int check_train_mode(int mode) {
  SAGE_TRY(check_mode(mode, true));
  const int lo = mode & SAGE_MODE_MASK;
  if (lo != SAGE_MODE_INT8_Q128_K64 && lo != SAGE_MODE_INT8_Q64_K64)
    return fail(SAGE_ERR_UNSUPPORTED, "mode %d: the training forward and the backward pass support the per-block "
                "INT8 modes %d and %d", lo, SAGE_MODE_INT8_Q128_K64, SAGE_MODE_INT8_Q64_K64);
  return SAGE_OK;
}

// Scratch of sage_attn_fwd_noalloc: the workspace of that entry point, a global
// of this code object, so each device the library runs on holds its own copy
// (allocated with the code object, kept until the process ends). Host code
// never uses the array's name as an address: the device address comes from
// hipGetSymbolAddress, taken once per device on the first call there.
static __device__ __align__(256) unsigned char scratch[SAGE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the current device.
int scratch_address(void** addr) {
  int dev = -1;
  SAGE_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SAGE_ERR_UNSUPPORTED, "device %d: the scratch table covers devices 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* a = nullptr;
    const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !a) {
      (void)hipGetLastError();
      return fail(SAGE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    }
    g_scratch_addr[dev] = a;
  }
  *addr = g_scratch_addr[dev];
  return SAGE_OK;
}

}  // namespace

extern "C" {

const char* sage_status_string(int status) {
  switch (status) {
    case SAGE_OK: return "SAGE_OK";
    case SAGE_ERR_INVALID_ARG: return "SAGE_ERR_INVALID_ARG";
    case SAGE_ERR_UNSUPPORTED: return "SAGE_ERR_UNSUPPORTED";
    case SAGE_ERR_WORKSPACE: return "SAGE_ERR_WORKSPACE";
    case SAGE_ERR_NO_DEVICE: return "SAGE_ERR_NO_DEVICE";
    case SAGE_ERR_HIP: return "SAGE_ERR_HIP";
    default: return "SAGE_ERR_UNKNOWN";
  }
}

const char* sage_last_error(void) { return g_err; }

size_t sage_attn_workspace_size(int B, int H, int N, int d, int mode) {
  if (check_dims(B, H, N, d) != SAGE_OK || check_mode(mode, true) != SAGE_OK) return 0;
  if (sage::mode_pv_int8(mode & SAGE_MODE_MASK) && N > kMaxNPv8) return 0;
  return sage::make_layout(static_cast<long long>(B) * H, N, d, mode & SAGE_MODE_MASK, true).total;
}

size_t sage_quant_workspace_size(int B, int H, int N, int d) {
  if (check_dims(B, H, N, d) != SAGE_OK) return 0;
  return sage::make_layout(static_cast<long long>(B) * H, N, d, 0, false).total;
}

int sage_attn_prepare(const void* q, const void* k, const void* v, int B, int H, int N, int d, int mode,
                      void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  SAGE_TRY(check_ptr(q, "q", 16));
  SAGE_TRY(check_ptr(k, "k", 16));
  SAGE_TRY(check_ptr(v, "v", 16));
  SAGE_TRY(validate_attn(B, H, N, d, mode, workspace, workspace_bytes));
  SAGE_TRY(check_device());
  return do_prepare(q, k, v, B, H, N, d, mode, workspace, static_cast<hipStream_t>(stream));
}

int sage_attn_compute(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
                      int causal, float sm_scale, int mode, const void* workspace, size_t workspace_bytes,
                      void* stream) {
  g_err[0] = 0;
  const int lo = mode & SAGE_MODE_MASK;
  if (lo == SAGE_MODE_FP16) {
    SAGE_TRY(check_ptr(q, "q", 16));
    SAGE_TRY(check_ptr(k, "k", 16));
  }
  if (mode & SAGE_FLAG_FUSED_Q) SAGE_TRY(check_ptr(q, "q", 16));
  if (reads_fp16_v(lo)) SAGE_TRY(check_ptr(v, "v", 16));
  SAGE_TRY(check_ptr(out, "out", 16));
  if (causal != 0 && causal != 1) return fail(SAGE_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  SAGE_TRY(check_scale(sm_scale));
  SAGE_TRY(validate_attn(B, H, N, d, mode, workspace, workspace_bytes));
  SAGE_TRY(check_device());
  return do_compute(q, k, v, out, B, H, N, d, causal, sm_scale, mode, workspace, static_cast<hipStream_t>(stream));
}

int sage_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
                  int causal, float sm_scale, int mode, void* workspace, size_t workspace_bytes,
                  void* stream) {
  g_err[0] = 0;
  SAGE_TRY(check_ptr(q, "q", 16));
  SAGE_TRY(check_ptr(k, "k", 16));
  SAGE_TRY(check_ptr(v, "v", 16));
  SAGE_TRY(check_ptr(out, "out", 16));
  if (causal != 0 && causal != 1) return fail(SAGE_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  SAGE_TRY(check_scale(sm_scale));
  SAGE_TRY(validate_attn(B, H, N, d, mode, workspace, workspace_bytes));
  SAGE_TRY(check_device());
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int fm = with_fused_q(mode, B, H, N);
  SAGE_TRY(do_prepare(q, k, v, B, H, N, d, fm, workspace, s));
  return do_compute(q, k, v, out, B, H, N, d, causal, sm_scale, fm, workspace, s);
}

int sage_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
                          int causal, float sm_scale, int mode, void* stream) {
  g_err[0] = 0;
  SAGE_TRY(check_ptr(q, "q", 16));
  SAGE_TRY(check_ptr(k, "k", 16));
  SAGE_TRY(check_ptr(v, "v", 16));
  SAGE_TRY(check_ptr(out, "out", 16));
  if (causal != 0 && causal != 1) return fail(SAGE_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  SAGE_TRY(check_scale(sm_scale));
  SAGE_TRY(check_dims(B, H, N, d));
  SAGE_TRY(check_mode(mode, true));
  if (sage::mode_pv_int8(mode & SAGE_MODE_MASK) && N > kMaxNPv8)
    return fail(SAGE_ERR_UNSUPPORTED, "N = %d exceeds %d, the limit of the INT8 P.V modes", N, kMaxNPv8);
  const size_t need = sage::make_layout(static_cast<long long>(B) * H, N, d, mode & SAGE_MODE_MASK, true).total;
  if (need > SAGE_NOALLOC_SCRATCH_BYTES)
    return fail(SAGE_ERR_WORKSPACE,
                "this problem needs %zu bytes of workspace; sage_attn_fwd_noalloc holds %zu "
                "(use sage_attn_fwd with a caller-provided workspace)",
                need, static_cast<size_t>(SAGE_NOALLOC_SCRATCH_BYTES));
  SAGE_TRY(check_device());
  void* ws = nullptr;
  SAGE_TRY(scratch_address(&ws));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int fm = with_fused_q(mode, B, H, N);
  SAGE_TRY(do_prepare(q, k, v, B, H, N, d, fm, ws, s));
  return do_compute(q, k, v, out, B, H, N, d, causal, sm_scale, fm, ws, s);
}

size_t sage_attn_bwd_workspace_size(int B, int H, int N, int d, int mode) {
  if (check_dims(B, H, N, d) != SAGE_OK || check_train_mode(mode) != SAGE_OK) return 0;
  return sage::make_bwd_layout(static_cast<long long>(B) * H, N, d, mode & SAGE_MODE_MASK).total;
}

int sage_attn_fwd_lse(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int N, int d,
                      int causal, float sm_scale, int mode, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  SAGE_TRY(check_ptr(q, "q", 16));
  SAGE_TRY(check_ptr(k, "k", 16));
  SAGE_TRY(check_ptr(v, "v", 16));
  SAGE_TRY(check_ptr(out, "out", 16));
  SAGE_TRY(check_ptr(lse, "lse", 4));
  if (causal != 0 && causal != 1) return fail(SAGE_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  SAGE_TRY(check_scale(sm_scale));
  SAGE_TRY(check_train_mode(mode));
  SAGE_TRY(validate_attn(B, H, N, d, mode, workspace, workspace_bytes));
  SAGE_TRY(check_device());
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int fm = with_fused_q(mode, B, H, N);
  SAGE_TRY(do_prepare(q, k, v, B, H, N, d, fm, workspace, s));
  return do_compute(q, k, v, out, B, H, N, d, causal, sm_scale, fm, workspace, s, lse);
}

int sage_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                  float* dq, float* dk, float* dv, int B, int H, int N, int d, int causal, float sm_scale, int mode,
                  void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  SAGE_TRY(check_ptr(q, "q", 16));
  SAGE_TRY(check_ptr(k, "k", 16));
  SAGE_TRY(check_ptr(v, "v", 16));
  SAGE_TRY(check_ptr(out, "out", 16));
  SAGE_TRY(check_ptr(dout, "dout", 16));
  SAGE_TRY(check_ptr(lse, "lse", 4));
  SAGE_TRY(check_ptr(dq, "dq", 16));
  SAGE_TRY(check_ptr(dk, "dk", 16));
  SAGE_TRY(check_ptr(dv, "dv", 16));
  if (causal != 0 && causal != 1) return fail(SAGE_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  SAGE_TRY(check_scale(sm_scale));
  SAGE_TRY(check_dims(B, H, N, d));
  SAGE_TRY(check_train_mode(mode));
  SAGE_TRY(check_ptr(workspace, "workspace", 256));
  const int BH = B * H;
  const int lo = mode & SAGE_MODE_MASK;
  const sage::BwdLayout L = sage::make_bwd_layout(BH, N, d, lo);
  if (workspace_bytes < L.total)
    return fail(SAGE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, L.total);
  SAGE_TRY(check_device());
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // the forward's codes of Q and K_s (same kernels, same layout), then V per
  // token and dO per 64 rows
  SAGE_TRY(do_prepare(q, k, v, B, H, N, d, mode & ~SAGE_FLAG_FUSED_Q, workspace, s));
  const int Npad = L.f.Npad;
  sage::Int8Job jv, jg;
  jv.src = v; jv.codes = reinterpret_cast<int8_t*>(at(workspace, L.vc)); jv.scales = reinterpret_cast<float*>(at(workspace, L.vs));
  jv.blk = 1; jv.code_rows = Npad; jv.nscale = Npad; jv.ntile = Npad / sage::kQTile;
  jg.src = dout; jg.codes = reinterpret_cast<int8_t*>(at(workspace, L.gc)); jg.scales = reinterpret_cast<float*>(at(workspace, L.gs));
  jg.blk = 64; jg.code_rows = Npad; jg.nscale = Npad / 64; jg.ntile = Npad / sage::kQTile;
  SAGE_TRY(hip_status(sage::launch_int8_quant(jv, jg, BH, N, d, s), "backward quantization kernel"));
  sage::BwdLaunch b;
  b.BH = BH; b.N = N; b.Npad = Npad; b.d = d; b.causal = causal != 0;
  b.qblk = lo == SAGE_MODE_INT8_Q64_K64 ? 64 : 128;
  b.sm = sm_scale;
  b.sl2 = static_cast<float>(static_cast<double>(sm_scale) * 1.4426950408889634);
  b.o = static_cast<const _Float16*>(out); b.dout = static_cast<const _Float16*>(dout); b.lse = lse;
  b.qc = reinterpret_cast<const int8_t*>(at(workspace, L.f.q_codes));
  b.kc = reinterpret_cast<const int8_t*>(at(workspace, L.f.k_codes));
  b.vc = reinterpret_cast<const int8_t*>(at(workspace, L.vc));
  b.gc = reinterpret_cast<const int8_t*>(at(workspace, L.gc));
  b.qt = reinterpret_cast<int8_t*>(at(workspace, L.qt));
  b.kt = reinterpret_cast<int8_t*>(at(workspace, L.kt));
  b.gt = reinterpret_cast<int8_t*>(at(workspace, L.gt));
  b.qs = reinterpret_cast<const float*>(at(workspace, L.f.q_scales));
  b.ks = reinterpret_cast<const float*>(at(workspace, L.f.k_scales));
  b.vs = reinterpret_cast<const float*>(at(workspace, L.vs));
  b.gs = reinterpret_cast<const float*>(at(workspace, L.gs));
  b.ld = reinterpret_cast<float2*>(at(workspace, L.ld));
  b.dq = dq; b.dk = dk; b.dv = dv;
  return hip_status(sage::launch_attn_bwd(b, s), "backward kernels");
}

int sage_attn_dump_scores(const void* v, void* out, int B, int H, int N, int d, float sm_scale, int mode,
                          const void* workspace, size_t workspace_bytes, int bh, int q_tile, int k_tile,
                          int32_t* s_out, void* stream) {
  g_err[0] = 0;
  SAGE_TRY(check_ptr(v, "v", 16));
  SAGE_TRY(check_ptr(out, "out", 16));
  SAGE_TRY(check_ptr(s_out, "s_out", 16));
  SAGE_TRY(check_scale(sm_scale));
  SAGE_TRY(validate_attn(B, H, N, d, mode, workspace, workspace_bytes));
  const int lo = mode & SAGE_MODE_MASK;
  if (lo != SAGE_MODE_INT8_Q128_K64 && lo != SAGE_MODE_INT8_Q64_K64 && lo != SAGE_MODE_INT8_PER_TOKEN)
    return fail(SAGE_ERR_UNSUPPORTED, "the score dump covers the INT8 modes 0, 1 and 3 (got %d)", lo);
  if (mode & SAGE_FLAG_FUSED_Q)
    return fail(SAGE_ERR_UNSUPPORTED, "the score dump reads the Q codes that sage_attn_prepare writes without "
                "SAGE_FLAG_FUSED_Q");
  const long long BH = static_cast<long long>(B) * H;
  if (bh < 0 || bh >= BH) return fail(SAGE_ERR_INVALID_ARG, "bh = %d is outside [0, %lld)", bh, BH);
  const int nqt = (N + sage::kWGQ - 1) / sage::kWGQ, nkt = (N + sage::kKTile - 1) / sage::kKTile;
  if (q_tile < 0 || q_tile >= nqt) return fail(SAGE_ERR_INVALID_ARG, "q_tile = %d is outside [0, %d)", q_tile, nqt);
  if (k_tile < 0 || k_tile >= nkt) return fail(SAGE_ERR_INVALID_ARG, "k_tile = %d is outside [0, %d)", k_tile, nkt);
  SAGE_TRY(check_device());
  const sage::Layout L = sage::make_layout(BH, N, d, lo, true);
  sage::AttnArgs a;
  a.BH = static_cast<int>(BH); a.N = N; a.Npad = L.Npad; a.d = d; a.causal = false;
  a.sl2 = static_cast<float>(static_cast<double>(sm_scale) * 1.4426950408889634);
  a.mode = lo; a.out = out;
  (void)hipGetLastError();
  return hip_status(sage::launch_attn_int8_dump(a, at(workspace, L.q_codes), at(workspace, L.k_codes),
                                                v,
                                                reinterpret_cast<const float*>(at(workspace, L.q_scales)),
                                                reinterpret_cast<const float*>(at(workspace, L.k_scales)),
                                                reinterpret_cast<int*>(s_out), bh, q_tile, k_tile,
                                                static_cast<hipStream_t>(stream)),
                    "INT8 attention kernel (score dump)");
}

int sage_quant_qk(const void* q, const void* k, int B, int H, int N, int d, int blk_q, int blk_k, int flags,
                  int8_t* q_codes, float* q_scales, int8_t* k_codes, float* k_scales, float* k_mean,
                  void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  SAGE_TRY(check_dims(B, H, N, d));
  SAGE_TRY(check_ptr(q, "q", 16));
  SAGE_TRY(check_ptr(k, "k", 16));
  SAGE_TRY(check_ptr(q_codes, "q_codes", 16));
  SAGE_TRY(check_ptr(k_codes, "k_codes", 16));
  SAGE_TRY(check_ptr(q_scales, "q_scales", 4));
  SAGE_TRY(check_ptr(k_scales, "k_scales", 4));
  if (k_mean) SAGE_TRY(check_ptr(k_mean, "k_mean", 4));
  auto blk_ok = [](int b) { return b == 1 || b == 16 || b == 32 || b == 64 || b == 128; };
  if (!blk_ok(blk_q) || !blk_ok(blk_k))
    return fail(SAGE_ERR_UNSUPPORTED, "block sizes must be 1, 16, 32, 64 or 128 (got %d, %d)", blk_q, blk_k);
  if (flags & ~SAGE_FLAG_NO_SMOOTH) return fail(SAGE_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
  SAGE_TRY(check_ptr(workspace, "workspace", 256));
  const int BH = B * H;
  const sage::Layout L = sage::make_layout(BH, N, d, 0, false);
  if (workspace_bytes < L.total)
    return fail(SAGE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, L.total);
  SAGE_TRY(check_device());
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool smooth = !(flags & SAGE_FLAG_NO_SMOOTH);
  (void)hipGetLastError();
  float* mu = reinterpret_cast<float*>(at(workspace, L.kmean));
  if (smooth)
    SAGE_TRY(hip_status(sage::launch_kmean(k, reinterpret_cast<long long*>(at(workspace, L.ksum)), mu, k_mean, BH, N,
                                           d, L.chunk, L.nchunk, s), "K mean kernels"));
  const int ntile = (N + sage::kQTile - 1) / sage::kQTile;
  sage::Int8Job jq, jk;
  jq.src = q; jq.codes = q_codes; jq.scales = q_scales; jq.mu = nullptr; jq.blk = blk_q; jq.code_rows = N;
  jq.nscale = (N + blk_q - 1) / blk_q; jq.ntile = ntile;
  jk.src = k; jk.codes = k_codes; jk.scales = k_scales; jk.mu = smooth ? mu : nullptr; jk.blk = blk_k; jk.code_rows = N;
  jk.nscale = (N + blk_k - 1) / blk_k; jk.ntile = ntile;
  return hip_status(sage::launch_int8_quant(jq, jk, BH, N, d, s), "INT8 quantization kernel");
}

int sage_quant_mxfp4(const void* q, const void* k, const void* v, int B, int H, int N, int d, int flags,
                     uint8_t* q_fp4, uint8_t* q_e8m0, uint8_t* k_fp4, uint8_t* k_e8m0, uint8_t* vt_fp4,
                     uint8_t* vt_e8m0, float* k_mean, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  SAGE_TRY(check_dims(B, H, N, d));
  SAGE_TRY(check_ptr(q, "q", 16));
  SAGE_TRY(check_ptr(k, "k", 16));
  SAGE_TRY(check_ptr(v, "v", 16));
  SAGE_TRY(check_ptr(q_fp4, "q_fp4", 16));
  SAGE_TRY(check_ptr(k_fp4, "k_fp4", 16));
  SAGE_TRY(check_ptr(vt_fp4, "vt_fp4", 16));
  SAGE_TRY(check_ptr(q_e8m0, "q_e8m0", 1));
  SAGE_TRY(check_ptr(k_e8m0, "k_e8m0", 1));
  SAGE_TRY(check_ptr(vt_e8m0, "vt_e8m0", 1));
  if (k_mean) SAGE_TRY(check_ptr(k_mean, "k_mean", 4));
  if (flags & ~(SAGE_FLAG_NO_SMOOTH | SAGE_FLAG_FP8_V)) return fail(SAGE_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
  SAGE_TRY(check_ptr(workspace, "workspace", 256));
  const int BH = B * H;
  const sage::Layout L = sage::make_layout(BH, N, d, 0, false);
  if (workspace_bytes < L.total)
    return fail(SAGE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, L.total);
  SAGE_TRY(check_device());
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool smooth = !(flags & SAGE_FLAG_NO_SMOOTH);
  (void)hipGetLastError();
  float* mu = reinterpret_cast<float*>(at(workspace, L.kmean));
  if (smooth)
    SAGE_TRY(hip_status(sage::launch_kmean(k, reinterpret_cast<long long*>(at(workspace, L.ksum)), mu, k_mean, BH, N,
                                           d, L.chunk, L.nchunk, s), "K mean kernels"));
  sage::MxRowJob jq, jk;
  jq.src = q; jq.fp4 = q_fp4; jq.e8 = q_e8m0; jq.mu = nullptr; jq.rows = N;
  jk.src = k; jk.fp4 = k_fp4; jk.e8 = k_e8m0; jk.mu = smooth ? mu : nullptr; jk.rows = N;
  SAGE_TRY(hip_status(sage::launch_mx_rows(jq, jk, BH, N, d, s), "MXFP4 Q/K quantization kernel"));
  const int Nv = sage::round_up(N, 32);
  if (flags & SAGE_FLAG_FP8_V)
    return hip_status(sage::launch_mx_vt8(v, vt_fp4, vt_e8m0, BH, N, Nv, d, s), "MX-FP8 V quantization kernel");
  return hip_status(sage::launch_mx_vt(v, vt_fp4, vt_e8m0, BH, N, Nv, d, s), "MXFP4 V quantization kernel");
}

int sage_quant_v_int8(const void* v, int B, int H, int N, int d, int8_t* vt_codes, float* v_scales,
                      void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  SAGE_TRY(check_dims(B, H, N, d));
  SAGE_TRY(check_ptr(v, "v", 16));
  SAGE_TRY(check_ptr(vt_codes, "vt_codes", 16));
  SAGE_TRY(check_ptr(v_scales, "v_scales", 4));
  SAGE_TRY(check_ptr(workspace, "workspace", 256));
  const int BH = B * H;
  const sage::Layout L = sage::make_layout(BH, N, d, 0, false);
  if (workspace_bytes < L.total)
    return fail(SAGE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, L.total);
  SAGE_TRY(check_device());
  (void)hipGetLastError();
  return hip_status(sage::launch_v_int8(v, reinterpret_cast<unsigned*>(at(workspace, L.vmax)), vt_codes, v_scales,
                                        BH, N, sage::round_up(N, 16), d, L.chunk, L.nchunk,
                                        static_cast<hipStream_t>(stream)),
                    "INT8 V quantization kernels");
}

int sage_clock_probe(long long cycles, long long* out, void* stream) {
  g_err[0] = 0;
  SAGE_TRY(check_ptr(out, "out", 8));
  if (cycles < 1 || cycles > (1LL << 32)) return fail(SAGE_ERR_INVALID_ARG, "cycles = %lld is outside [1, 2^32]", cycles);
  SAGE_TRY(check_device());
  (void)hipGetLastError();
  return hip_status(sage::launch_clock_probe(cycles, out, static_cast<hipStream_t>(stream)), "clock probe kernel");
}

int sage_wall_clock_khz(int* khz) {
  g_err[0] = 0;
  SAGE_TRY(check_ptr(khz, "khz", 4));
  SAGE_TRY(check_device());
  int dev = 0;
  SAGE_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  return hip_status(hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev), "hipDeviceGetAttribute");
}

}  // extern "C"
