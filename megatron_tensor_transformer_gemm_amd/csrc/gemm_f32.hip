// fp32 column-/row-parallel GEMM (fp32 inputs, fp32 accumulation, fp32 output).
//
// Used for the float32 workloads, whose results are held to fp32 accuracy.  On
// gfx950 the fp32 matrix-core rate equals the fp32 vector rate (both ~157 TFLOP/s),
// so this path uses plain VALU FMAs over LDS tiles: 64x64 output tile per
// workgroup, each of 256 threads owning a 4x4 block (two blocks for the gated
// activations), k staged 16 at a time.  Bounds are checked on every load and
// store, so any M, N, K is accepted.
#include "tp_internal.h"

namespace tpk {
namespace {

constexpr int kT = 64;
constexpr int kKB = 16;

__device__ __forceinline__ float gelu_erf(float u) {
  return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f));
}

template <bool DUAL, int ACT>
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmDesc g, int tiles_n) {
  constexpr int NSUB = DUAL ? 2 : 1;
  __shared__ float As[kKB][kT + 4];
  __shared__ float Bs[NSUB][kKB][kT];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * kT;
  const int n0 = (blockIdx.x % tiles_n) * kT;
  const float* A = (const float*)g.A;
  const float* B[2] = {(const float*)g.B0, (const float*)(DUAL ? g.B1 : g.B0)};

  float acc[NSUB][4][4];
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[s][i][j] = 0.0f;

  for (int k0 = 0; k0 < g.K; k0 += kKB) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 256 * e;  // 1024 elements of the 64 x 16 A tile
      const int r = idx >> 4, kk = idx & 15;
      const int64_t m = m0 + r;
      const int k = k0 + kk;
      As[kk][r] = (m < g.M && k < g.K) ? A[m * g.lda + k] : 0.0f;
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = tid + 256 * e;  // 1024 elements of the 16 x 64 B tile
        const int kk = idx >> 6, c = idx & 63;
        const int k = k0 + kk, n = n0 + c;
        Bs[s][kk][c] = (k < g.K && n < g.N) ? B[s][(int64_t)k * g.ldb + n] : 0.0f;
      }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kKB; ++kk) {
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        float b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = Bs[s][kk][tx * 4 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[s][i][j] = fmaf(a[i], b[j], acc[s][i][j]);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= g.N) continue;
      const float u = acc[0][i][j];
      const float v = acc[NSUB - 1][i][j];
      float h;
      if constexpr (ACT == kActGelu) h = gelu_erf(u);
      else if constexpr (ACT == kActSwiglu) h = u / (1.0f + expf(-u)) * v;
      else if constexpr (ACT == kActBilinear) h = u * v;
      else h = u;
      ((float*)g.C)[m * g.ldc + n] = h;
    }
  }
}

template <bool DUAL, int ACT>
hipError_t launch(const GemmDesc& g, hipStream_t s) {
  const int64_t tm = (g.M + kT - 1) / kT, tn = (g.N + kT - 1) / kT;
  if (tm * tn > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_f32_kernel<DUAL, ACT>), dim3((unsigned)(tm * tn)), dim3(256), 0, s, g,
                     (int)tn);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_f32(const GemmDesc& g, hipStream_t s) {
  switch (g.act) {
    case kActNone: return launch<false, kActNone>(g, s);
    case kActGelu: return launch<false, kActGelu>(g, s);
    case kActSwiglu: return launch<true, kActSwiglu>(g, s);
    case kActBilinear: return launch<true, kActBilinear>(g, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tpk
