// Local partial sum standing in for the tensor-parallel all-reduce.
//
// y[i] = sum_{t=0}^{T_p-1} P_t[i] (+ residual[i]), fp32 accumulation in ascending t,
// residual last, one rounding to the output type.  The sum over ranks is what the
// all-reduce g computes at the end of each sharded sublayer ("7.9 Tensor and pipeline
// parallelism", section 2.1); a fixed order makes repeated calls bitwise identical.
//
// Pure HBM streaming: each thread owns 8 consecutive elements (one 16-byte bf16 vector
// or two 16-byte fp32 vectors per operand) and issues all T_p loads before adding; the
// grid covers the array (striding over it only beyond 2^28 vectors), and a scalar pass
// handles the n % 8 tail.  Slices whose
// stride is a large power of two put the same element of every slice on the same DRAM
// banks; callers that allocate the partials should pad the stride by a few KiB (a 4 KiB
// pad took an 8-way bf16 reduce from 5.3 to 5.7 TB/s on MI355X).
#include "tp_internal.h"

namespace tpk {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf2f(unsigned short h) {
  return __uint_as_float((unsigned)h << 16);
}
__device__ __forceinline__ unsigned short f2bf(float f) {
  return __builtin_bit_cast(unsigned short, (__bf16)f);
}

template <bool BF>
__device__ __forceinline__ void load8(const void* base, int64_t i, float (&v)[8]) {
  if constexpr (BF) {
    const u16x8 x = __builtin_nontemporal_load((const u16x8*)((const unsigned short*)base + i));
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = bf2f(x[e]);
  } else {
    const f32x4 a = __builtin_nontemporal_load((const f32x4*)((const float*)base + i));
    const f32x4 b = __builtin_nontemporal_load((const f32x4*)((const float*)base + i + 4));
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[e + 4] = b[e]; }
  }
}

template <bool BF>
__device__ __forceinline__ void store8(void* base, int64_t i, const float (&v)[8]) {
  if constexpr (BF) {
    u16x8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = f2bf(v[e]);
    *(u16x8*)((unsigned short*)base + i) = x;
  } else {
    *(f32x4*)((float*)base + i) = f32x4{v[0], v[1], v[2], v[3]};
    *(f32x4*)((float*)base + i + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
}

template <bool BF>
__device__ __forceinline__ float load1(const void* base, int64_t i) {
  if constexpr (BF) return bf2f(((const unsigned short*)base)[i]);
  else return ((const float*)base)[i];
}

// TPC > 0: T_p known at compile time (all loads in flight together); TPC == 0: runtime loop.
template <int TPC, bool PBF, bool OBF, bool RES>
__global__ void __launch_bounds__(256) partial_sum_kernel(const void* __restrict__ parts,
                                                          int64_t stride, int T_p,
                                                          const void* res, void* y, int64_t n) {
  const int tp = TPC > 0 ? TPC : T_p;
  const int64_t nvec = n >> 3;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += step) {
    const int64_t i = v << 3;
    float acc[8];
    if constexpr (TPC > 0) {
      float p[TPC][8];
#pragma unroll
      for (int t = 0; t < TPC; ++t) load8<PBF>(parts, t * stride + i, p[t]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = p[0][e];
#pragma unroll
      for (int t = 1; t < TPC; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += p[t][e];
    } else {
      load8<PBF>(parts, i, acc);
      for (int t = 1; t < tp; ++t) {
        float p[8];
        load8<PBF>(parts, t * stride + i, p);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += p[e];
      }
    }
    if constexpr (RES) {
      float r[8];
      load8<OBF>(res, i, r);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += r[e];
    }
    store8<OBF>(y, i, acc);
  }
  // tail (n % 8 elements): first threads of block 0
  if (blockIdx.x == 0) {
    const int64_t i = (nvec << 3) + threadIdx.x;
    if (i < n) {
      float a = load1<PBF>(parts, i);
      for (int t = 1; t < tp; ++t) a += load1<PBF>(parts, t * stride + i);
      if constexpr (RES) a += load1<OBF>(res, i);
      if constexpr (OBF) ((unsigned short*)y)[i] = f2bf(a);
      else ((float*)y)[i] = a;
    }
  }
}

template <bool PBF, bool OBF, bool RES>
hipError_t launch3(const void* parts, int64_t stride, int T_p, const void* res, void* y, int64_t n,
                   hipStream_t s) {
  const int64_t nvec = n >> 3;
  // One 8-element vector per thread; the grid strides only past 2^28 vectors.  Against a
  // grid-stride loop over 8 workgroups per CU, the 8-way 70B-shaped reduce (2.4 GB) took
  // 430.8 -> 401.4 us (6.0 TB/s), the backward's dX sum 421 -> 394 us (two alternations on
  // one GPU).
  int64_t blocks = (nvec + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  const dim3 grid((unsigned)blocks), block(256);
  switch (T_p) {
    case 1: hipLaunchKernelGGL((partial_sum_kernel<1, PBF, OBF, RES>), grid, block, 0, s, parts, stride, T_p, res, y, n); break;
    case 2: hipLaunchKernelGGL((partial_sum_kernel<2, PBF, OBF, RES>), grid, block, 0, s, parts, stride, T_p, res, y, n); break;
    case 4: hipLaunchKernelGGL((partial_sum_kernel<4, PBF, OBF, RES>), grid, block, 0, s, parts, stride, T_p, res, y, n); break;
    case 8: hipLaunchKernelGGL((partial_sum_kernel<8, PBF, OBF, RES>), grid, block, 0, s, parts, stride, T_p, res, y, n); break;
    default: hipLaunchKernelGGL((partial_sum_kernel<0, PBF, OBF, RES>), grid, block, 0, s, parts, stride, T_p, res, y, n); break;
  }
  return hipGetLastError();
}

template <bool PBF, bool OBF>
hipError_t launch2(const void* parts, int64_t stride, int T_p, const void* res, void* y, int64_t n,
                   hipStream_t s) {
  return res ? launch3<PBF, OBF, true>(parts, stride, T_p, res, y, n, s)
             : launch3<PBF, OBF, false>(parts, stride, T_p, res, y, n, s);
}

}  // namespace

hipError_t launch_partial_sum(const void* parts, int64_t stride, int T_p, const void* res, void* y,
                              int64_t n, int part_bf16, int out_bf16, hipStream_t s) {
  if (part_bf16) {
    return out_bf16 ? launch2<true, true>(parts, stride, T_p, res, y, n, s)
                    : launch2<true, false>(parts, stride, T_p, res, y, n, s);
  }
  return out_bf16 ? launch2<false, true>(parts, stride, T_p, res, y, n, s)
                  : launch2<false, false>(parts, stride, T_p, res, y, n, s);
}

}  // namespace tpk
