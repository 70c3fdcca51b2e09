// C ABI of the tensor-parallel shard library (declarations and contract in tpshard.h).
//
// Host side only: argument validation (everything is checked before any launch),
// the rank's offsets into the full weight matrices, kernel selection, and
// error reporting.  Kernels live in gemm_bf16.hip, gemm_f32.hip, partial_sum.hip
// and attention.hip.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "tp_internal.h"
#include "tpshard.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return TP_OK;
  return fail(TP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Largest leading dimension / feature extent: the bf16 kernels address a 256-row tile
// with 32-bit per-lane byte offsets that must stay below 1 GiB (256 x 2^20 x 2 bytes).
constexpr int64_t kMaxExtent = int64_t(1) << 20;
constexpr int64_t kMaxRows = int64_t(1) << 31;

size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

int check_ptr(const void* p, const char* name) {
  if (!p) return fail(TP_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(TP_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return TP_OK;
}

#define TRY(expr)              \
  do {                         \
    const int _rc = (expr);    \
    if (_rc != TP_OK) return _rc; \
  } while (0)

}  // namespace

extern "C" {

int tp_abi_version(void) { return TPSHARD_ABI_VERSION; }

const char* tp_last_error(void) { return g_err.c_str(); }

int tp_shard_range(int64_t extent, int32_t T_p, int32_t t, int64_t* begin, int64_t* len) {
  if (!begin || !len) return fail(TP_ERR_INVALID_ARG, "tp_shard_range: null output pointer");
  if (T_p < 1) return fail(TP_ERR_INVALID_ARG, "tp_shard_range: T_p=%d < 1", T_p);
  if (t < 0 || t >= T_p) return fail(TP_ERR_INVALID_ARG, "tp_shard_range: rank t=%d outside [0, %d)", t, T_p);
  if (extent < 0) return fail(TP_ERR_INVALID_ARG, "tp_shard_range: negative extent %lld", (long long)extent);
  if (extent % T_p)
    return fail(TP_ERR_NOT_DIVISIBLE, "tp_shard_range: extent %lld not divisible by T_p=%d",
                (long long)extent, T_p);
  const int64_t n = extent / T_p;
  *begin = (int64_t)t * n;
  *len = n;
  return TP_OK;
}

size_t tp_ffn_workspace_bytes(int64_t T, int64_t d_ff, int32_t T_p, int32_t in_dtype) {
  if (T < 0 || d_ff <= 0 || T_p < 1 || d_ff % T_p) return 0;
  if (in_dtype != TP_F32 && in_dtype != TP_BF16) return 0;
  const size_t elt = in_dtype == TP_BF16 ? 2 : 4;
  const size_t h = round256((size_t)T * (size_t)(d_ff / T_p) * elt);
  if (in_dtype != TP_BF16 || d_ff / T_p > kMaxExtent) return h;
  // plus the column product's split-K scratch when it is too small to fill the GPU (its k
  // depth d is not an argument: sized for a deep product, for either activation kind)
  const int32_t n = (int32_t)(d_ff / T_p);
  const size_t plain = tpk::splitk_scratch_bytes(T, 1, &n, int64_t(1) << 30, false);
  const size_t gated = tpk::splitk_scratch_bytes(T, 1, &n, int64_t(1) << 30, true);
  return h + round256(plain > gated ? plain : gated);
}

}  // extern "C"

namespace {

// Shared checks of the FFN entry points.  `need_*` select which pointers are validated.
int check_ffn(const char* fn, const void* x, const void* w1, const void* w3, const void* w2,
              const void* h, const void* y, int64_t T, int64_t d, int64_t d_ff, int32_t T_p,
              int32_t t, int32_t act, int32_t in_dtype, int32_t out_dtype, bool col, bool row) {
  if (T < 0 || T >= kMaxRows) return fail(TP_ERR_INVALID_ARG, "%s: T=%lld out of range", fn, (long long)T);
  if (d <= 0 || d_ff <= 0) return fail(TP_ERR_INVALID_ARG, "%s: d and d_ff must be positive", fn);
  if (d > kMaxExtent || d_ff > kMaxExtent)
    return fail(TP_ERR_UNSUPPORTED, "%s: d or d_ff above %lld", fn, (long long)kMaxExtent);
  if (T_p < 1 || t < 0 || t >= T_p)
    return fail(TP_ERR_INVALID_ARG, "%s: rank t=%d outside [0, T_p=%d)", fn, t, T_p);
  if (d_ff % T_p)
    return fail(TP_ERR_NOT_DIVISIBLE, "%s: d_ff=%lld not divisible by T_p=%d", fn, (long long)d_ff, T_p);
  if (col && (act < TP_ACT_NONE || act > TP_ACT_BILINEAR))
    return fail(TP_ERR_UNSUPPORTED, "%s: unknown activation %d", fn, act);
  if (!((in_dtype == TP_BF16 && (out_dtype == TP_BF16 || out_dtype == TP_F32)) ||
        (in_dtype == TP_F32 && out_dtype == TP_F32)))
    return fail(TP_ERR_UNSUPPORTED, "%s: dtype pair (in=%d, out=%d) not supported", fn, in_dtype, out_dtype);
  if (col) {
    const bool gated = act == TP_ACT_SWIGLU || act == TP_ACT_BILINEAR;
    TRY(check_ptr(x, "x"));
    TRY(check_ptr(w1, "w1"));
    if (gated) TRY(check_ptr(w3, "w3"));
    else if (w3) return fail(TP_ERR_INVALID_ARG, "%s: w3 given for a non-gated activation", fn);
  }
  if (row) {
    TRY(check_ptr(w2, "w2"));
    TRY(check_ptr(y, "y_t"));
  }
  if (h) TRY(check_ptr(h, col && !row ? "h_t" : "workspace"));
  const int64_t n = d_ff / T_p;
  const int vec = in_dtype == TP_BF16 ? 8 : 4;
  if (d % vec || n % vec || d_ff % vec)
    return fail(TP_ERR_UNSUPPORTED, "%s: d=%lld, d_ff=%lld and d_ff/T_p=%lld must be multiples of %d", fn,
                (long long)d, (long long)d_ff, (long long)n, vec);
  return TP_OK;
}

int launch_column(const void* x, const void* w1, const void* w3, void* h, int64_t T, int64_t d,
                  int64_t d_ff, int32_t T_p, int32_t t, int32_t act, bool bf, hipStream_t s,
                  void* part = nullptr, size_t part_bytes = 0) {
  const int64_t n = d_ff / T_p;
  const size_t elt = bf ? 2 : 4;
  const bool gated = act == TP_ACT_SWIGLU || act == TP_ACT_BILINEAR;
  // H(t) = act(X . W1[:, t*n : (t+1)*n] (, X . W3[:, ...]))
  tpk::GemmDesc g{};
  g.A = x;
  g.B0 = (const char*)w1 + (size_t)t * n * elt;
  g.B1 = gated ? (const char*)w3 + (size_t)t * n * elt : nullptr;
  g.C = h;
  g.M = T;
  g.N = (int32_t)n;
  g.K = (int32_t)d;
  g.lda = (int32_t)d;
  g.ldb = (int32_t)d_ff;
  g.ldc = (int32_t)n;
  g.act = act;
  g.out_f32 = !bf;
  if (bf && part_bytes) {
    g.part = (float*)part;
    g.part_bytes = part_bytes;
  }
  return hip_status(bf ? tpk::launch_gemm_bf16(g, s) : tpk::launch_gemm_f32(g, s), "column-parallel GEMM launch");
}

int launch_row(const void* h, const void* w2, void* y, int64_t T, int64_t d, int64_t d_ff, int32_t T_p,
               int32_t t, bool bf, bool out_f32, hipStream_t s) {
  const int64_t n = d_ff / T_p;
  const size_t elt = bf ? 2 : 4;
  // y(t) = H(t) . W2[t*n : (t+1)*n, :]
  tpk::GemmDesc g{};
  g.A = h;
  g.B0 = (const char*)w2 + (size_t)t * n * (size_t)d * elt;
  g.B1 = nullptr;
  g.C = y;
  g.M = T;
  g.N = (int32_t)d;
  g.K = (int32_t)n;
  g.lda = (int32_t)n;
  g.ldb = (int32_t)d;
  g.ldc = (int32_t)d;
  g.act = TP_ACT_NONE;
  g.out_f32 = out_f32;
  return hip_status(bf ? tpk::launch_gemm_bf16(g, s) : tpk::launch_gemm_f32(g, s), "row-parallel GEMM launch");
}

}  // namespace

extern "C" {

int tp_ffn_shard_fwd(const void* x, const void* w1, const void* w3, const void* w2, void* y_t,
                     void* workspace, size_t workspace_bytes, int64_t T, int64_t d, int64_t d_ff,
                     int32_t T_p, int32_t t, int32_t act, int32_t in_dtype, int32_t out_dtype,
                     void* hip_stream) {
  TRY(check_ffn("tp_ffn_shard_fwd", x, w1, w3, w2, nullptr, y_t, T, d, d_ff, T_p, t, act, in_dtype,
                out_dtype, true, true));
  const size_t elt = in_dtype == TP_BF16 ? 2 : 4;
  const size_t hbytes = round256((size_t)T * (size_t)(d_ff / T_p) * elt);   // H(t): required
  if (T > 0) {
    if (!workspace) return fail(TP_ERR_WORKSPACE, "tp_ffn_shard_fwd: workspace is NULL");
    if (!aligned16(workspace)) return fail(TP_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    if (workspace_bytes < hbytes)
      return fail(TP_ERR_WORKSPACE, "tp_ffn_shard_fwd: workspace %zu bytes < %zu needed", workspace_bytes, hbytes);
  }
  if (T == 0) return TP_OK;
  hipStream_t s = (hipStream_t)hip_stream;
  const bool bf = in_dtype == TP_BF16;
  // bytes beyond H(t) serve as the column product's split-K scratch
  TRY(launch_column(x, w1, w3, workspace, T, d, d_ff, T_p, t, act, bf, s, (char*)workspace + hbytes,
                    workspace_bytes - hbytes));
  return launch_row(workspace, w2, y_t, T, d, d_ff, T_p, t, bf, out_dtype == TP_F32, s);
}

}  // extern "C"

// H(t) of tp_ffn_shard_fwd_noalloc.  In host code `scratch` names a host-side stand-in:
// kernels get the device address looked up for the current device, never the name.
static __device__ __align__(256) unsigned char scratch[TP_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on its first use there.
int scratch_address(void** out) {
  int dev = -1;
  TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(TP_ERR_UNSUPPORTED, "device %d outside the %d the library keeps scratch for", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    TRY(hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    if (!p || !aligned16(p)) return fail(TP_ERR_HIP, "scratch address %p is not usable", p);
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return TP_OK;
}

}  // namespace

extern "C" {

int tp_ffn_shard_fwd_noalloc(const void* x, const void* w1, const void* w3, const void* w2,
                             void* y_t, int64_t T, int64_t d, int64_t d_ff, int32_t T_p, int32_t t,
                             int32_t act, int32_t in_dtype, int32_t out_dtype, void* hip_stream) {
  const char* fn = "tp_ffn_shard_fwd_noalloc";
  TRY(check_ffn(fn, x, w1, w3, w2, nullptr, y_t, T, d, d_ff, T_p, t, act, in_dtype, out_dtype, true, true));
  if (T == 0) return TP_OK;
  const size_t elt = in_dtype == TP_BF16 ? 2 : 4;
  const size_t need = round256((size_t)T * (size_t)(d_ff / T_p) * elt);
  if (need > TP_NOALLOC_SCRATCH_BYTES)
    return fail(TP_ERR_WORKSPACE, "%s: H(t) needs %zu bytes, above the %zu bytes of scratch held per GPU",
                fn, need, (size_t)TP_NOALLOC_SCRATCH_BYTES);
  void* h = nullptr;
  TRY(scratch_address(&h));
  hipStream_t s = (hipStream_t)hip_stream;
  const bool bf = in_dtype == TP_BF16;
  // the rest of the scratch serves as the column product's split-K partial sums
  TRY(launch_column(x, w1, w3, h, T, d, d_ff, T_p, t, act, bf, s, (char*)h + need,
                    (size_t)TP_NOALLOC_SCRATCH_BYTES - need));
  return launch_row(h, w2, y_t, T, d, d_ff, T_p, t, bf, out_dtype == TP_F32, s);
}

int tp_ffn_column_fwd(const void* x, const void* w1, const void* w3, void* h_t, int64_t T, int64_t d,
                      int64_t d_ff, int32_t T_p, int32_t t, int32_t act, int32_t in_dtype,
                      void* hip_stream) {
  if (!h_t) return fail(TP_ERR_INVALID_ARG, "tp_ffn_column_fwd: h_t is NULL");
  TRY(check_ffn("tp_ffn_column_fwd", x, w1, w3, nullptr, h_t, nullptr, T, d, d_ff, T_p, t, act,
                in_dtype, in_dtype, true, false));
  if (T == 0) return TP_OK;
  return launch_column(x, w1, w3, h_t, T, d, d_ff, T_p, t, act, in_dtype == TP_BF16,
                       (hipStream_t)hip_stream);
}

int tp_ffn_row_fwd(const void* h_t, const void* w2, void* y_t, int64_t T, int64_t d, int64_t d_ff,
                   int32_t T_p, int32_t t, int32_t in_dtype, int32_t out_dtype, void* hip_stream) {
  if (!h_t) return fail(TP_ERR_INVALID_ARG, "tp_ffn_row_fwd: h_t is NULL");
  TRY(check_ffn("tp_ffn_row_fwd", nullptr, nullptr, nullptr, w2, h_t, y_t, T, d, d_ff, T_p, t,
                TP_ACT_NONE, in_dtype, out_dtype, false, true));
  if (T == 0) return TP_OK;
  return launch_row(h_t, w2, y_t, T, d, d_ff, T_p, t, in_dtype == TP_BF16, out_dtype == TP_F32,
                    (hipStream_t)hip_stream);
}

int tp_ffn_shard_fwd_train(const void* x, const void* w1, const void* w3, const void* w2, void* y_t,
                           void* h_t, void* u_t, void* v_t, int64_t T, int64_t d, int64_t d_ff,
                           int32_t T_p, int32_t t, int32_t act, int32_t out_dtype, void* hip_stream) {
  const char* fn = "tp_ffn_shard_fwd_train";
  if (!h_t) return fail(TP_ERR_INVALID_ARG, "%s: h_t is NULL", fn);
  TRY(check_ffn(fn, x, w1, w3, w2, h_t, y_t, T, d, d_ff, T_p, t, act, TP_BF16, out_dtype, true, true));
  if (act == TP_ACT_NONE)
    return fail(TP_ERR_UNSUPPORTED, "%s: act NONE has no pre-activation to keep (U = H)", fn);
  const bool gated = act == TP_ACT_SWIGLU || act == TP_ACT_BILINEAR;
  TRY(check_ptr(u_t, "u_t"));
  if (gated) TRY(check_ptr(v_t, "v_t"));
  else if (v_t) return fail(TP_ERR_INVALID_ARG, "%s: v_t given for a non-gated activation", fn);
  if (T == 0) return TP_OK;
  hipStream_t s = (hipStream_t)hip_stream;
  const int64_t n = d_ff / T_p;
  // H(t) = act(X W1(t) [, X W3(t)]) with U (and V) stored from the same accumulators
  tpk::GemmDesc g{};
  g.A = x;
  g.B0 = (const __bf16*)w1 + (size_t)t * n;
  g.B1 = gated ? (const __bf16*)w3 + (size_t)t * n : nullptr;
  g.C = h_t;
  g.M = T;
  g.N = (int32_t)n;
  g.K = (int32_t)d;
  g.lda = (int32_t)d;
  g.ldb = (int32_t)d_ff;
  g.ldc = (int32_t)n;
  g.act = act;
  g.out_f32 = false;
  g.U = u_t;
  g.V = gated ? v_t : nullptr;
  g.ldu = (int32_t)n;
  TRY(hip_status(tpk::launch_gemm_bf16(g, s), "column-parallel GEMM launch"));
  return launch_row(h_t, w2, y_t, T, d, d_ff, T_p, t, true, out_dtype == TP_F32, s);
}

size_t tp_ffn_bwd_workspace_bytes(int64_t T, int64_t d_ff, int32_t T_p, int32_t act) {
  if (T < 0 || d_ff <= 0 || T_p < 1 || d_ff % T_p) return 0;
  if (act < TP_ACT_NONE || act > TP_ACT_BILINEAR) return 0;
  const size_t plane = round256((size_t)T * (size_t)(d_ff / T_p) * 2);
  return act == TP_ACT_SWIGLU || act == TP_ACT_BILINEAR ? 2 * plane : plane;
}

int tp_ffn_shard_bwd(const void* x, const void* w1, const void* w3, const void* w2, const void* dy,
                     const void* h_t, const void* u_t, const void* v_t, void* dx_t, void* dw1,
                     void* dw3, void* dw2, void* workspace, size_t workspace_bytes, int64_t T,
                     int64_t d, int64_t d_ff, int32_t T_p, int32_t t, int32_t act, int32_t dx_dtype,
                     int32_t grad_dtype, void* hip_stream) {
  const char* fn = "tp_ffn_shard_bwd";
  if (!dx_t) return fail(TP_ERR_INVALID_ARG, "%s: dx_t is NULL", fn);
  TRY(check_ffn(fn, x, w1, w3, w2, nullptr, dx_t, T, d, d_ff, T_p, t, act, TP_BF16, dx_dtype, true, true));
  if (grad_dtype != TP_BF16 && grad_dtype != TP_F32)
    return fail(TP_ERR_UNSUPPORTED, "%s: grad_dtype %d not supported", fn, grad_dtype);
  const bool gated = act == TP_ACT_SWIGLU || act == TP_ACT_BILINEAR;
  TRY(check_ptr(dy, "dy"));
  TRY(check_ptr(h_t, "h_t"));
  TRY(check_ptr(dw1, "dw1"));
  TRY(check_ptr(dw2, "dw2"));
  if (act != TP_ACT_NONE) TRY(check_ptr(u_t, "u_t"));
  if (gated) {
    TRY(check_ptr(v_t, "v_t"));
    TRY(check_ptr(dw3, "dw3"));
  } else if (v_t || dw3) {
    return fail(TP_ERR_INVALID_ARG, "%s: v_t / dw3 given for a non-gated activation", fn);
  }
  const size_t need = tp_ffn_bwd_workspace_bytes(T, d_ff, T_p, act);
  if (T > 0) {
    if (!workspace) return fail(TP_ERR_WORKSPACE, "%s: workspace is NULL", fn);
    if (!aligned16(workspace)) return fail(TP_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    if (workspace_bytes < need)
      return fail(TP_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, need);
  }
  hipStream_t s = (hipStream_t)hip_stream;
  const int64_t n = d_ff / T_p;
  const size_t b = (size_t)t * n;   // first hidden unit of rank t
  const bool gf32 = grad_dtype == TP_F32;
  const size_t gelt = gf32 ? 4 : 2;
  void* du = workspace;
  void* dv = gated ? (char*)workspace + need / 2 : nullptr;

  if (T > 0) {
    // dU [, dV] = act'(dH) with dH = dY W2(t)^T: W2's row block [n, d] is B^T
    tpk::GemmDesc g{};
    g.A = dy;
    g.B0 = (const __bf16*)w2 + b * (size_t)d;
    g.C = du;
    g.M = T;
    g.N = (int32_t)n;
    g.K = (int32_t)d;
    g.lda = (int32_t)d;
    g.ldb = (int32_t)d;
    g.ldc = (int32_t)n;
    g.act = act;
    g.out_f32 = false;
    g.U = const_cast<void*>(u_t);
    g.V = const_cast<void*>(v_t);
    g.dV = dv;
    g.ldu = (int32_t)n;
    TRY(hip_status(tpk::launch_gemm_bf16_nt(g, s), "dH GEMM launch"));
  }
  {
    // dW2[cols(t), :] = H(t)^T dY: H [T, n] is A^T
    tpk::GemmDesc g{};
    g.A = h_t;
    g.B0 = dy;
    g.C = (char*)dw2 + b * (size_t)d * gelt;
    g.M = n;
    g.N = (int32_t)d;
    g.K = (int32_t)T;
    g.lda = (int32_t)n;
    g.ldb = (int32_t)d;
    g.ldc = (int32_t)d;
    g.act = TP_ACT_NONE;
    g.out_f32 = gf32;
    TRY(hip_status(tpk::launch_gemm_bf16_tn(g, s), "dW2 GEMM launch"));
  }
  if (T > 0) {
    // dX(t) = dU W1(t)^T [+ dV W3(t)^T]: W1's column block is B^T [d, n] at stride d_ff
    tpk::GemmDesc g{};
    g.A = du;
    g.B0 = (const __bf16*)w1 + b;
    g.C = dx_t;
    g.M = T;
    g.N = (int32_t)d;
    g.K = (int32_t)n;
    g.lda = (int32_t)n;
    g.ldb = (int32_t)d_ff;
    g.ldc = (int32_t)d;
    g.act = TP_ACT_NONE;
    g.out_f32 = dx_dtype == TP_F32;
    if (gated) {
      g.A2 = dv;
      g.B2 = (const __bf16*)w3 + b;
      g.K2 = (int32_t)n;
    }
    TRY(hip_status(tpk::launch_gemm_bf16_nt(g, s), "dX GEMM launch"));
  }
  {
    // dW1[:, cols(t)] = X^T dU [, dW3[:, cols(t)] = X^T dV]: X [T, d] is A^T
    tpk::GemmDesc g{};
    g.A = x;
    g.B0 = du;
    g.C = (char*)dw1 + b * gelt;
    g.M = d;
    g.N = (int32_t)n;
    g.K = (int32_t)T;
    g.lda = (int32_t)d;
    g.ldb = (int32_t)n;
    g.ldc = (int32_t)d_ff;
    g.act = TP_ACT_NONE;
    g.out_f32 = gf32;
    if (gated) {
      g.nseg = 2;
      g.Bx[0] = dv;
      g.Cx[0] = (char*)dw3 + b * gelt;
      g.Nx[0] = (int32_t)n;
      g.ldbx[0] = (int32_t)n;
      g.ldcx[0] = (int32_t)d_ff;
    }
    if (T == 0) {   // k = 0: nothing is read (the workspace may be absent), the blocks are zero
      g.B0 = dw1;
      if (gated) g.Bx[0] = dw1;
    }
    TRY(hip_status(tpk::launch_gemm_bf16_tn(g, s), "dW1 GEMM launch"));
  }
  return TP_OK;
}

int tp_attn_outproj_shard_fwd(const void* o_t, const void* wo, void* y_t, int64_t T, int64_t d,
                              int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t T_p,
                              int32_t t, int32_t in_dtype, int32_t out_dtype, void* hip_stream) {
  if (T < 0 || T >= kMaxRows) return fail(TP_ERR_INVALID_ARG, "tp_attn_outproj_shard_fwd: T out of range");
  if (d <= 0 || n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0)
    return fail(TP_ERR_INVALID_ARG, "tp_attn_outproj_shard_fwd: d, head counts and head_dim must be positive");
  if (T_p < 1 || t < 0 || t >= T_p)
    return fail(TP_ERR_INVALID_ARG, "tp_attn_outproj_shard_fwd: rank t=%d outside [0, T_p=%d)", t, T_p);
  if (n_heads % T_p)
    return fail(TP_ERR_NOT_DIVISIBLE, "n_heads=%d is not a multiple of T_p=%d", n_heads, T_p);
  if (n_kv_heads % T_p)
    return fail(TP_ERR_NOT_DIVISIBLE, "n_kv_heads=%d is not a multiple of T_p=%d", n_kv_heads, T_p);
  if (n_heads % n_kv_heads)
    return fail(TP_ERR_INVALID_ARG, "n_heads=%d is not a multiple of n_kv_heads=%d", n_heads, n_kv_heads);
  if (!((in_dtype == TP_BF16 && (out_dtype == TP_BF16 || out_dtype == TP_F32)) ||
        (in_dtype == TP_F32 && out_dtype == TP_F32)))
    return fail(TP_ERR_UNSUPPORTED, "tp_attn_outproj_shard_fwd: dtype pair (in=%d, out=%d) not supported", in_dtype, out_dtype);
  const bool bf = in_dtype == TP_BF16;
  const int64_t kdim = (int64_t)(n_heads / T_p) * head_dim;
  const int vec = bf ? 8 : 4;
  if (d % vec || kdim % vec)
    return fail(TP_ERR_UNSUPPORTED, "tp_attn_outproj_shard_fwd: d and h_t*head_dim must be multiples of %d", vec);
  if (d > kMaxExtent || (int64_t)n_heads * head_dim > kMaxExtent)
    return fail(TP_ERR_UNSUPPORTED, "tp_attn_outproj_shard_fwd: extent too large");
  TRY(check_ptr(o_t, "o_t"));
  TRY(check_ptr(wo, "wo"));
  TRY(check_ptr(y_t, "y_t"));
  if (T == 0) return TP_OK;
  const size_t elt = bf ? 2 : 4;
  tpk::GemmDesc g{};
  g.A = o_t;
  g.B0 = (const char*)wo + (size_t)t * (size_t)kdim * (size_t)d * elt;
  g.B1 = nullptr;
  g.C = y_t;
  g.M = T;
  g.N = (int32_t)d;
  g.K = (int32_t)kdim;
  g.lda = (int32_t)kdim;
  g.ldb = (int32_t)d;
  g.ldc = (int32_t)d;
  g.act = TP_ACT_NONE;
  g.out_f32 = out_dtype == TP_F32;
  hipStream_t s = (hipStream_t)hip_stream;
  return hip_status(bf ? tpk::launch_gemm_bf16(g, s) : tpk::launch_gemm_f32(g, s), "out-projection GEMM launch");
}

}  // extern "C"

namespace {

// Q, K, V of a rank's heads [T, (h_t + 2 kv_t) head_dim] bf16, then the split-K scratch of
// the fused projection when it is too small to fill the GPU (sized for a deep product: d
// is not an argument of the queries).
size_t heads_qkv_bytes(int64_t T, int64_t h_t, int64_t kv_t, int32_t head_dim) {
  return round256((size_t)T * (size_t)((h_t + 2 * kv_t) * head_dim) * 2);
}
size_t heads_split_bytes(int64_t T, int64_t h_t, int64_t kv_t, int32_t head_dim) {
  if ((h_t + 2 * kv_t) * head_dim > kMaxExtent || T >= kMaxRows) return 0;
  const int32_t seg[3] = {(int32_t)(h_t * head_dim), (int32_t)(kv_t * head_dim), (int32_t)(kv_t * head_dim)};
  return round256(tpk::splitk_scratch_bytes(T, 3, seg, int64_t(1) << 30, false));
}

}  // namespace

extern "C" {

size_t tp_attn_heads_workspace_bytes(int64_t n_seq, int64_t seq_len, int32_t n_heads,
                                     int32_t n_kv_heads, int32_t head_dim, int32_t T_p) {
  if (n_seq < 0 || seq_len < 0 || n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 || T_p < 1) return 0;
  if (n_heads % T_p || n_kv_heads % T_p) return 0;
  const int64_t h_t = n_heads / T_p, kv_t = n_kv_heads / T_p, T = n_seq * seq_len;
  return heads_qkv_bytes(T, h_t, kv_t, head_dim) + heads_split_bytes(T, h_t, kv_t, head_dim);
}

size_t tp_attn_heads_kvrep_workspace_bytes(int64_t n_seq, int64_t seq_len, int32_t n_heads,
                                           int32_t n_kv_heads, int32_t head_dim, int32_t T_p) {
  if (n_seq < 0 || seq_len < 0 || n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 || T_p < 1) return 0;
  if (n_kv_heads % T_p == 0)
    return tp_attn_heads_workspace_bytes(n_seq, seq_len, n_heads, n_kv_heads, head_dim, T_p);
  if (n_heads % T_p || T_p % n_kv_heads || n_heads % n_kv_heads) return 0;
  // one (replicated) KV head per rank
  const int64_t h_t = n_heads / T_p, T = n_seq * seq_len;
  return heads_qkv_bytes(T, h_t, 1, head_dim) + heads_split_bytes(T, h_t, 1, head_dim);
}

}  // extern "C"

namespace {

// Shared body of tp_attn_heads_shard_fwd and tp_attn_heads_shard_fwd_kvrep.  With kvrep
// and fewer KV heads than ranks, each KV head serves T_p / n_kv_heads consecutive ranks
// and rank t reads KV head t / (T_p / n_kv_heads) for all of its query heads.
int attn_heads_impl(const char* fn, bool kvrep, const void* x, const void* wq, const void* wk,
                    const void* wv, void* o_t, void* workspace, size_t workspace_bytes,
                    int64_t n_seq, int64_t seq_len, int64_t d, int32_t n_heads, int32_t n_kv_heads,
                    int32_t head_dim, int32_t T_p, int32_t t, int32_t causal, void* hip_stream) {
  if (n_seq < 0 || seq_len < 0 || n_seq > 65535)
    return fail(TP_ERR_INVALID_ARG, "%s: n_seq=%lld / seq_len=%lld out of range", fn, (long long)n_seq,
                (long long)seq_len);
  if (d <= 0 || n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0)
    return fail(TP_ERR_INVALID_ARG, "%s: d, head counts and head_dim must be positive", fn);
  if (T_p < 1 || t < 0 || t >= T_p)
    return fail(TP_ERR_INVALID_ARG, "%s: rank t=%d outside [0, T_p=%d)", fn, t, T_p);
  if (n_heads % T_p)
    return fail(TP_ERR_NOT_DIVISIBLE, "n_heads=%d is not a multiple of T_p=%d", n_heads, T_p);
  const bool replicate = kvrep && n_kv_heads % T_p != 0;
  if (replicate && T_p % n_kv_heads)
    return fail(TP_ERR_NOT_DIVISIBLE, "TP%d cannot replicate %d KV heads evenly (T_p must be a multiple)",
                T_p, n_kv_heads);
  if (!replicate && n_kv_heads % T_p)
    return fail(TP_ERR_NOT_DIVISIBLE, "n_kv_heads=%d is not a multiple of T_p=%d", n_kv_heads, T_p);
  if (n_heads % n_kv_heads)
    return fail(TP_ERR_INVALID_ARG, "n_heads=%d is not a multiple of n_kv_heads=%d", n_heads, n_kv_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(TP_ERR_UNSUPPORTED, "%s: head_dim must be 64 or 128, got %d", fn, head_dim);
  if (causal != 0 && causal != 1) return fail(TP_ERR_INVALID_ARG, "%s: causal must be 0 or 1", fn);
  if (d % 8) return fail(TP_ERR_UNSUPPORTED, "%s: d must be a multiple of 8", fn);
  if (d > kMaxExtent || (int64_t)n_heads * head_dim > kMaxExtent)
    return fail(TP_ERR_UNSUPPORTED, "%s: extent too large", fn);
  const int64_t T = n_seq * seq_len;
  if (T >= kMaxRows) return fail(TP_ERR_INVALID_ARG, "%s: too many tokens", fn);
  const int64_t h_t = n_heads / T_p, kv_t = replicate ? 1 : n_kv_heads / T_p;
  // first KV head of rank t
  const int64_t kv0 = replicate ? t / (T_p / n_kv_heads) : (int64_t)t * kv_t;
  // the attention kernel addresses one sequence of a head with 32-bit byte offsets
  if ((int64_t)seq_len * (h_t + 2 * kv_t) * head_dim * 2 >= (int64_t(1) << 30))
    return fail(TP_ERR_UNSUPPORTED, "%s: seq_len too long for one call", fn);
  TRY(check_ptr(x, "x"));
  TRY(check_ptr(wq, "wq"));
  TRY(check_ptr(wk, "wk"));
  TRY(check_ptr(wv, "wv"));
  TRY(check_ptr(o_t, "o_t"));
  // Q, K, V are required; bytes beyond them serve as the projection's split-K scratch
  const size_t need = heads_qkv_bytes(T, h_t, kv_t, head_dim);
  if (T > 0) {
    if (!workspace) return fail(TP_ERR_WORKSPACE, "%s: workspace is NULL", fn);
    if (!aligned16(workspace)) return fail(TP_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    if (workspace_bytes < need)
      return fail(TP_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, need);
  }
  if (T == 0) return TP_OK;
  hipStream_t s = (hipStream_t)hip_stream;
  __bf16* q = (__bf16*)workspace;
  __bf16* k = q + T * h_t * head_dim;
  __bf16* v = k + T * kv_t * head_dim;
  // Q, K, V column blocks of the rank's heads (column-parallel projections, no activation),
  // as one launch over three column segments that share X.
  tpk::GemmDesc g{};
  g.A = x;
  g.B0 = (const __bf16*)wq + (size_t)t * h_t * head_dim;
  g.B1 = nullptr;
  g.C = q;
  g.M = T;
  g.N = (int32_t)(h_t * head_dim);
  g.K = (int32_t)d;
  g.lda = (int32_t)d;
  g.ldb = (int32_t)(n_heads * head_dim);
  g.ldc = g.N;
  g.act = TP_ACT_NONE;
  g.out_f32 = false;
  g.nseg = 3;
  const void* wkv[2] = {wk, wv};
  __bf16* outs[2] = {k, v};
  for (int i = 0; i < 2; ++i) {
    g.Bx[i] = (const __bf16*)wkv[i] + (size_t)kv0 * head_dim;
    g.Cx[i] = outs[i];
    g.Nx[i] = (int32_t)(kv_t * head_dim);
    g.ldbx[i] = (int32_t)(n_kv_heads * head_dim);
    g.ldcx[i] = g.Nx[i];
  }
  if (workspace_bytes > need) {
    g.part = (float*)((char*)workspace + need);
    g.part_bytes = workspace_bytes - need;
  }
  TRY(hip_status(tpk::launch_gemm_bf16(g, s), "QKV projection GEMM launch"));
  tpk::AttnDesc a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = (__bf16*)o_t;
  a.n_seq = n_seq;
  a.seq_len = (int32_t)seq_len;
  a.head_dim = head_dim;
  a.h_t = (int32_t)h_t;
  a.kv_t = (int32_t)kv_t;
  a.ldq = (int32_t)(h_t * head_dim);
  a.ldkv = (int32_t)(kv_t * head_dim);
  a.ldo = (int32_t)(h_t * head_dim);
  a.causal = causal != 0;
  return hip_status(tpk::launch_attention(a, s), "attention launch");
}

}  // namespace

extern "C" {

int tp_attn_heads_shard_fwd(const void* x, const void* wq, const void* wk, const void* wv,
                            void* o_t, void* workspace, size_t workspace_bytes, int64_t n_seq,
                            int64_t seq_len, int64_t d, int32_t n_heads, int32_t n_kv_heads,
                            int32_t head_dim, int32_t T_p, int32_t t, int32_t causal,
                            void* hip_stream) {
  return attn_heads_impl("tp_attn_heads_shard_fwd", false, x, wq, wk, wv, o_t, workspace,
                         workspace_bytes, n_seq, seq_len, d, n_heads, n_kv_heads, head_dim, T_p, t,
                         causal, hip_stream);
}

int tp_attn_heads_shard_fwd_kvrep(const void* x, const void* wq, const void* wk, const void* wv,
                                  void* o_t, void* workspace, size_t workspace_bytes, int64_t n_seq,
                                  int64_t seq_len, int64_t d, int32_t n_heads, int32_t n_kv_heads,
                                  int32_t head_dim, int32_t T_p, int32_t t, int32_t causal,
                                  void* hip_stream) {
  return attn_heads_impl("tp_attn_heads_shard_fwd_kvrep", true, x, wq, wk, wv, o_t, workspace,
                         workspace_bytes, n_seq, seq_len, d, n_heads, n_kv_heads, head_dim, T_p, t,
                         causal, hip_stream);
}

}  // extern "C"

namespace {
// The argument checks shared by the attention core and the ring step (everything but
// the output / state).
int check_core_args(const char* fn, const void* q, const void* k, const void* v, int64_t n_seq,
                    int64_t seq_len, int32_t h_t, int32_t kv_t, int32_t head_dim, int64_t ldq,
                    int64_t ldkv, int32_t causal) {
  if (n_seq < 0 || seq_len < 0 || n_seq > 65535 || seq_len > 0x7FFFFFFF)
    return fail(TP_ERR_INVALID_ARG, "%s: n_seq / seq_len out of range", fn);
  if (h_t <= 0 || kv_t <= 0 || h_t % kv_t || h_t > 65535)
    return fail(TP_ERR_INVALID_ARG, "%s: h_t=%d must be a positive multiple of kv_t=%d", fn, h_t, kv_t);
  if (head_dim != 64 && head_dim != 128)
    return fail(TP_ERR_UNSUPPORTED, "%s: head_dim must be 64 or 128, got %d", fn, head_dim);
  if (causal != 0 && causal != 1) return fail(TP_ERR_INVALID_ARG, "%s: causal must be 0 or 1", fn);
  if (ldq < (int64_t)h_t * head_dim || ldkv < (int64_t)kv_t * head_dim)
    return fail(TP_ERR_INVALID_ARG, "%s: leading dimension smaller than the heads it holds", fn);
  if (ldq % 8 || ldkv % 8 || ldq > kMaxExtent || ldkv > kMaxExtent)
    return fail(TP_ERR_UNSUPPORTED, "%s: leading dimensions must be multiples of 8 and at most %lld", fn,
                (long long)kMaxExtent);
  if ((int64_t)seq_len * (ldq > ldkv ? ldq : ldkv) * 2 >= (int64_t(1) << 30))
    return fail(TP_ERR_UNSUPPORTED, "%s: seq_len too long for one call", fn);
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(k, "k"));
  TRY(check_ptr(v, "v"));
  return TP_OK;
}

// Checks of a [rows, ld] fp32 ring state holding `cols` columns, and of its [rows, ld_lse]
// log-denominators holding `heads` columns.
int check_ring_state(const char* fn, const void* o_state, const void* lse_state, int32_t cols,
                     int32_t heads, int64_t ld_state, int64_t ld_lse) {
  if (ld_state < cols || ld_state % 4 || ld_state > kMaxExtent)
    return fail(TP_ERR_INVALID_ARG, "%s: ld_state=%lld must be >= %d, a multiple of 4, at most %lld", fn,
                (long long)ld_state, cols, (long long)kMaxExtent);
  if (ld_lse < heads || ld_lse > kMaxExtent)
    return fail(TP_ERR_INVALID_ARG, "%s: ld_lse=%lld must be >= h_t=%d and at most %lld", fn,
                (long long)ld_lse, heads, (long long)kMaxExtent);
  TRY(check_ptr(o_state, "o_state"));
  if (lse_state) TRY(check_ptr(lse_state, "lse_state"));
  return TP_OK;
}

bool overlaps(const void* a, size_t a_bytes, const void* b, size_t b_bytes) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a_bytes && b_bytes && a0 < b0 + b_bytes && b0 < a0 + a_bytes;
}
}  // namespace

extern "C" {

int tp_attn_core_fwd(const void* q, const void* k, const void* v, void* o, int64_t n_seq,
                     int64_t seq_len, int32_t h_t, int32_t kv_t, int32_t head_dim, int64_t ldq,
                     int64_t ldkv, int64_t ldo, int32_t causal, void* hip_stream) {
  const char* fn = "tp_attn_core_fwd";
  TRY(check_core_args(fn, q, k, v, n_seq, seq_len, h_t, kv_t, head_dim, ldq, ldkv, causal));
  if (ldo < (int64_t)h_t * head_dim)
    return fail(TP_ERR_INVALID_ARG, "%s: leading dimension smaller than the heads it holds", fn);
  if (ldo % 8 || ldo > kMaxExtent)
    return fail(TP_ERR_UNSUPPORTED, "%s: leading dimensions must be multiples of 8 and at most %lld", fn,
                (long long)kMaxExtent);
  TRY(check_ptr(o, "o"));
  if (n_seq * seq_len == 0) return TP_OK;
  tpk::AttnDesc a{};
  a.q = (const __bf16*)q;
  a.k = (const __bf16*)k;
  a.v = (const __bf16*)v;
  a.o = (__bf16*)o;
  a.n_seq = n_seq;
  a.seq_len = (int32_t)seq_len;
  a.head_dim = head_dim;
  a.h_t = h_t;
  a.kv_t = kv_t;
  a.ldq = (int32_t)ldq;
  a.ldkv = (int32_t)ldkv;
  a.ldo = (int32_t)ldo;
  a.causal = causal != 0;
  return hip_status(tpk::launch_attention(a, (hipStream_t)hip_stream), "attention launch");
}

int tp_attn_ring_init(void* o_state, void* lse_state, int64_t rows, int32_t h_t, int32_t head_dim,
                      int64_t ld_state, int64_t ld_lse, void* hip_stream) {
  const char* fn = "tp_attn_ring_init";
  if (rows < 0 || rows > kMaxRows) return fail(TP_ERR_INVALID_ARG, "%s: rows out of range", fn);
  if (h_t <= 0 || h_t > 65535) return fail(TP_ERR_INVALID_ARG, "%s: h_t=%d out of range", fn, h_t);
  if (head_dim != 64 && head_dim != 128)
    return fail(TP_ERR_UNSUPPORTED, "%s: head_dim must be 64 or 128, got %d", fn, head_dim);
  const int64_t cols = (int64_t)h_t * head_dim;
  if (cols > kMaxExtent) return fail(TP_ERR_UNSUPPORTED, "%s: h_t*head_dim too large", fn);
  TRY(check_ptr(lse_state, "lse_state"));
  TRY(check_ring_state(fn, o_state, lse_state, (int32_t)cols, h_t, ld_state, ld_lse));
  if (overlaps(o_state, (size_t)(rows ? (rows - 1) * ld_state + cols : 0) * 4, lse_state,
               (size_t)(rows ? (rows - 1) * ld_lse + h_t : 0) * 4))
    return fail(TP_ERR_INVALID_ARG, "%s: o_state and lse_state overlap", fn);
  return hip_status(tpk::launch_ring_init((float*)o_state, (float*)lse_state, rows, (int32_t)cols, h_t,
                                          (int32_t)ld_state, (int32_t)ld_lse, (hipStream_t)hip_stream),
                    "ring-init launch");
}

int tp_attn_ring_step(const void* q, const void* k, const void* v, void* o_state, void* lse_state,
                      int64_t n_seq, int64_t seq_len, int32_t h_t, int32_t kv_t, int32_t head_dim,
                      int64_t ldq, int64_t ldkv, int64_t ld_state, int64_t ld_lse, int64_t q_pos0,
                      int64_t k_pos0, int32_t causal, void* hip_stream) {
  const char* fn = "tp_attn_ring_step";
  TRY(check_core_args(fn, q, k, v, n_seq, seq_len, h_t, kv_t, head_dim, ldq, ldkv, causal));
  TRY(check_ptr(lse_state, "lse_state"));
  TRY(check_ring_state(fn, o_state, lse_state, h_t * head_dim, h_t, ld_state, ld_lse));
  if (q_pos0 < 0 || k_pos0 < 0)
    return fail(TP_ERR_INVALID_ARG, "%s: negative chunk position", fn);
  const int64_t delta = q_pos0 - k_pos0;
  if (delta >= (int64_t(1) << 30) || delta <= -(int64_t(1) << 30))
    return fail(TP_ERR_INVALID_ARG, "%s: |q_pos0 - k_pos0| must be below 2^30", fn);
  const int64_t rows = n_seq * seq_len;
  const size_t st_bytes = (size_t)(rows ? (rows - 1) * ld_state + h_t * head_dim : 0) * 4;
  const size_t lse_bytes = (size_t)(rows ? (rows - 1) * ld_lse + h_t : 0) * 4;
  const size_t q_bytes = (size_t)(rows ? (rows - 1) * ldq + h_t * head_dim : 0) * 2;
  const size_t kv_bytes = (size_t)(rows ? (rows - 1) * ldkv + kv_t * head_dim : 0) * 2;
  if (overlaps(o_state, st_bytes, lse_state, lse_bytes))
    return fail(TP_ERR_INVALID_ARG, "%s: o_state and lse_state overlap", fn);
  const void* ins[3] = {q, k, v};
  const size_t in_bytes[3] = {q_bytes, kv_bytes, kv_bytes};
  for (int i = 0; i < 3; ++i)
    if (overlaps(o_state, st_bytes, ins[i], in_bytes[i]) || overlaps(lse_state, lse_bytes, ins[i], in_bytes[i]))
      return fail(TP_ERR_INVALID_ARG, "%s: the state overlaps q, k or v", fn);
  if (rows == 0) return TP_OK;
  // the whole key chunk comes after the whole query chunk: nothing to fold in
  if (causal && k_pos0 > q_pos0 + seq_len - 1) return TP_OK;
  tpk::AttnDesc a{};
  a.q = (const __bf16*)q;
  a.k = (const __bf16*)k;
  a.v = (const __bf16*)v;
  a.o = nullptr;
  a.n_seq = n_seq;
  a.seq_len = (int32_t)seq_len;
  a.head_dim = head_dim;
  a.h_t = h_t;
  a.kv_t = kv_t;
  a.ldq = (int32_t)ldq;
  a.ldkv = (int32_t)ldkv;
  a.causal = causal != 0;
  a.delta = (int32_t)delta;
  a.o_state = (float*)o_state;
  a.lse_state = (float*)lse_state;
  a.ld_state = (int32_t)ld_state;
  a.ld_lse = (int32_t)ld_lse;
  return hip_status(tpk::launch_attention(a, (hipStream_t)hip_stream), "ring-step launch");
}

int tp_attn_ring_finish(const void* o_state, void* o, int64_t rows, int32_t h_t, int32_t head_dim,
                        int64_t ld_state, int64_t ldo, void* hip_stream) {
  const char* fn = "tp_attn_ring_finish";
  if (rows < 0 || rows > kMaxRows) return fail(TP_ERR_INVALID_ARG, "%s: rows out of range", fn);
  if (h_t <= 0 || h_t > 65535) return fail(TP_ERR_INVALID_ARG, "%s: h_t=%d out of range", fn, h_t);
  if (head_dim != 64 && head_dim != 128)
    return fail(TP_ERR_UNSUPPORTED, "%s: head_dim must be 64 or 128, got %d", fn, head_dim);
  const int64_t cols = (int64_t)h_t * head_dim;
  if (cols > kMaxExtent) return fail(TP_ERR_UNSUPPORTED, "%s: h_t*head_dim too large", fn);
  TRY(check_ring_state(fn, o_state, nullptr, (int32_t)cols, h_t, ld_state, h_t));
  if (ldo < cols || ldo % 4 || ldo > kMaxExtent)
    return fail(TP_ERR_INVALID_ARG, "%s: ldo=%lld must be >= %lld, a multiple of 4, at most %lld", fn,
                (long long)ldo, (long long)cols, (long long)kMaxExtent);
  TRY(check_ptr(o, "o"));
  if (overlaps(o_state, (size_t)(rows ? (rows - 1) * ld_state + cols : 0) * 4, o,
               (size_t)(rows ? (rows - 1) * ldo + cols : 0) * 2))
    return fail(TP_ERR_INVALID_ARG, "%s: o overlaps the state", fn);
  return hip_status(tpk::launch_ring_finish((const float*)o_state, (__bf16*)o, rows, (int32_t)cols,
                                            (int32_t)ld_state, (int32_t)ldo, (hipStream_t)hip_stream),
                    "ring-finish launch");
}

int tp_partial_sum(const void* partials, int64_t partial_stride, int32_t T_p, const void* residual,
                   void* y, int64_t n_elems, int32_t part_dtype, int32_t out_dtype, void* hip_stream) {
  if (T_p < 1) return fail(TP_ERR_INVALID_ARG, "tp_partial_sum: T_p=%d < 1", T_p);
  if (n_elems < 0) return fail(TP_ERR_INVALID_ARG, "tp_partial_sum: negative n_elems");
  if ((part_dtype != TP_F32 && part_dtype != TP_BF16) || (out_dtype != TP_F32 && out_dtype != TP_BF16))
    return fail(TP_ERR_UNSUPPORTED, "tp_partial_sum: dtypes (%d, %d) not supported", part_dtype, out_dtype);
  if (partial_stride < n_elems)
    return fail(TP_ERR_INVALID_ARG, "tp_partial_sum: partial_stride %lld < n_elems %lld",
                (long long)partial_stride, (long long)n_elems);
  if (T_p > 1 && partial_stride % 8)
    return fail(TP_ERR_UNSUPPORTED, "tp_partial_sum: partial_stride must be a multiple of 8 elements");
  TRY(check_ptr(partials, "partials"));
  TRY(check_ptr(y, "y"));
  if (residual) TRY(check_ptr(residual, "residual"));
  const size_t pe = part_dtype == TP_BF16 ? 2 : 4, oe = out_dtype == TP_BF16 ? 2 : 4;
  const uintptr_t p0 = (uintptr_t)partials, p1 = p0 + (uintptr_t)((T_p - 1) * partial_stride + n_elems) * pe;
  const uintptr_t y0 = (uintptr_t)y, y1 = y0 + (uintptr_t)n_elems * oe;
  if (n_elems > 0 && y0 < p1 && p0 < y1)
    return fail(TP_ERR_INVALID_ARG, "tp_partial_sum: y overlaps the partials");
  if (n_elems == 0) return TP_OK;
  return hip_status(tpk::launch_partial_sum(partials, partial_stride, T_p, residual, y, n_elems,
                                            part_dtype == TP_BF16, out_dtype == TP_BF16,
                                            (hipStream_t)hip_stream),
                    "partial-sum launch");
}

int tp_attn_outproj_shard_bwd(const void* o_t, const void* wo, const void* dy, void* do_t, void* dwo,
                              int64_t T, int64_t d, int32_t n_heads, int32_t n_kv_heads,
                              int32_t head_dim, int32_t T_p, int32_t t, int32_t grad_dtype,
                              void* hip_stream) {
  const char* fn = "tp_attn_outproj_shard_bwd";
  if (T < 0 || T >= kMaxRows) return fail(TP_ERR_INVALID_ARG, "%s: T out of range", fn);
  if (d <= 0 || n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0)
    return fail(TP_ERR_INVALID_ARG, "%s: d, head counts and head_dim must be positive", fn);
  if (T_p < 1 || t < 0 || t >= T_p)
    return fail(TP_ERR_INVALID_ARG, "%s: rank t=%d outside [0, T_p=%d)", fn, t, T_p);
  if (n_heads % T_p)
    return fail(TP_ERR_NOT_DIVISIBLE, "n_heads=%d is not a multiple of T_p=%d", n_heads, T_p);
  if (n_kv_heads % T_p)
    return fail(TP_ERR_NOT_DIVISIBLE, "n_kv_heads=%d is not a multiple of T_p=%d", n_kv_heads, T_p);
  if (n_heads % n_kv_heads)
    return fail(TP_ERR_INVALID_ARG, "n_heads=%d is not a multiple of n_kv_heads=%d", n_heads, n_kv_heads);
  if (grad_dtype != TP_BF16 && grad_dtype != TP_F32)
    return fail(TP_ERR_UNSUPPORTED, "%s: grad_dtype %d not supported", fn, grad_dtype);
  const int64_t kdim = (int64_t)(n_heads / T_p) * head_dim;
  if (d % 8 || kdim % 8 || d > kMaxExtent || (int64_t)n_heads * head_dim > kMaxExtent)
    return fail(TP_ERR_UNSUPPORTED, "%s: d and h_t*head_dim must be multiples of 8 (and at most %lld)",
                fn, (long long)kMaxExtent);
  TRY(check_ptr(o_t, "o_t"));
  TRY(check_ptr(wo, "wo"));
  TRY(check_ptr(dy, "dy"));
  TRY(check_ptr(do_t, "do_t"));
  TRY(check_ptr(dwo, "dwo"));
  hipStream_t s = (hipStream_t)hip_stream;
  const size_t r0 = (size_t)t * kdim;   // first row of rank t's block of Wo
  if (T > 0) {
    // dO(t) = dY Wo(t)^T: Wo's row block [kdim, d] is B^T
    tpk::GemmDesc g{};
    g.A = dy;
    g.B0 = (const __bf16*)wo + r0 * (size_t)d;
    g.C = do_t;
    g.M = T;
    g.N = (int32_t)kdim;
    g.K = (int32_t)d;
    g.lda = (int32_t)d;
    g.ldb = (int32_t)d;
    g.ldc = (int32_t)kdim;
    g.act = TP_ACT_NONE;
    g.out_f32 = false;
    TRY(hip_status(tpk::launch_gemm_bf16_nt(g, s), "dO GEMM launch"));
  }
  // dWo[rows(t), :] = O(t)^T dY: O(t) [T, kdim] is A^T (k = 0 when T = 0: the block is zeroed)
  tpk::GemmDesc g{};
  g.A = o_t;
  g.B0 = dy;
  g.C = (char*)dwo + r0 * (size_t)d * (grad_dtype == TP_F32 ? 4 : 2);
  g.M = kdim;
  g.N = (int32_t)d;
  g.K = (int32_t)T;
  g.lda = (int32_t)kdim;
  g.ldb = (int32_t)d;
  g.ldc = (int32_t)d;
  g.act = TP_ACT_NONE;
  g.out_f32 = grad_dtype == TP_F32;
  return hip_status(tpk::launch_gemm_bf16_tn(g, s), "dWo GEMM launch");
}

int tp_reduce_scatter_rows(const void* partials, int64_t partial_stride, int32_t T_p, int32_t t,
                           const void* residual, void* y_rows, int64_t T, int64_t d,
                           int32_t part_dtype, int32_t out_dtype, void* hip_stream) {
  const char* fn = "tp_reduce_scatter_rows";
  if (T_p < 1 || t < 0 || t >= T_p)
    return fail(TP_ERR_INVALID_ARG, "%s: rank t=%d outside [0, T_p=%d)", fn, t, T_p);
  if (T < 0 || T >= kMaxRows || d <= 0)
    return fail(TP_ERR_INVALID_ARG, "%s: T=%lld, d=%lld out of range", fn, (long long)T, (long long)d);
  if (T % T_p)
    return fail(TP_ERR_NOT_DIVISIBLE, "%s: T=%lld tokens not divisible by T_p=%d", fn, (long long)T, T_p);
  if (d % 8) return fail(TP_ERR_UNSUPPORTED, "%s: d=%lld must be a multiple of 8", fn, (long long)d);
  if (partial_stride < T * d)
    return fail(TP_ERR_INVALID_ARG, "%s: partial_stride %lld < T*d", fn, (long long)partial_stride);
  const int64_t rows = T / T_p;
  const size_t pe = part_dtype == TP_BF16 ? 2 : 4;
  TRY(check_ptr(partials, "partials"));
  const void* first = (const char*)partials + (size_t)t * rows * d * pe;
  // rank t's rows of every slice: the same kernel and order as the full sum, on a sub-range
  return tp_partial_sum(first, partial_stride, T_p, residual, y_rows, rows * d, part_dtype, out_dtype,
                        hip_stream);
}

}  // extern "C"
