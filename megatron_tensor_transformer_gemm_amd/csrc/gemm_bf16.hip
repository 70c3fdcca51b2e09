// Column- and row-parallel bf16 GEMMs for gfx950 (CDNA4) MFMA.
//
// C[M, N] = epilogue(A[M, K] . B[K, N]) with A row-major (K contiguous: the
// token activations X or H(t)) and B row-major (N contiguous: a column block
// of W1/W3, or a row block of W2/Wo).  This is the per-rank matrix product of
// the column-then-row sharded FFN ("7.9 Tensor and pipeline parallelism",
// section 2.1) and of the row-sharded attention output projection (section
// 2.2); the activation runs in the epilogue on the fp32 accumulators, so the
// hidden activation is written once, already activated, and never leaves the
// rank ("Tensor & Pipeline Parallelism", S17 diagram: the activation is
// element-wise, so the sharded hidden state needs no communication).
//
// Design (one workgroup = 4 waves = 256 threads per output tile):
//  * HBM/L2 -> LDS with buffer_load ... lds (16 B per lane): no staging VGPRs,
//    out-of-range rows/columns/k come back as zeros from the buffer
//    descriptor's range check (masked lanes get an out-of-range offset), so
//    ragged M, N and K need no separate edge code.
//  * Two LDS stages (double buffering): tile k+1 streams in while tile k is
//    multiplied.
//  * A fragments: ds_read_b128 of 8 consecutive k of one row.
//  * B fragments: B is N-contiguous in memory and in LDS; ds_read_b64_tr_b16
//    transposes 4 k-rows x 16 columns per 16-lane group on the way to the
//    registers, so no transpose pass and no pre-packed weights are needed.
//  * v_mfma_f32_32x32x16_bf16 with the weight fragment as the first operand:
//    each lane then owns 4 consecutive output columns of one row, which the
//    epilogue stores as one 8-byte (bf16) or 16-byte (fp32) vector.
//  * XOR swizzles on the 16-byte chunk index keep both LDS read patterns
//    free of bank conflicts.
//  * Tile order: workgroups are dealt round-robin over the 8 XCDs; each XCD
//    is given a contiguous range of tiles in a grouped raster (4 tile rows),
//    so concurrently running tiles of one XCD share A and B panels in its L2.
#include "tp_internal.h"

namespace tpk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_raw __attribute__((__vector_size__(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kBK = 64;          // k per LDS stage
constexpr int kThreads = 256;    // 4 waves
constexpr uint32_t kOOB = 0x40000000u;       // voffset of a masked lane: >= num_records
constexpr int kNumRecords = 0x40000000;      // every valid per-lane offset is below 1 GiB
constexpr int kRsrcWord3 = 0x00020000;       // raw buffer, 32-bit data format (gfx9 family)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, kNumRecords,
                                           kRsrcWord3);
}

// Physical 16-byte chunk (of 8 per 128-byte A row) holding logical chunk c of row r is
// c ^ swz_a(r): 16 consecutive rows read at the same logical chunk land on 16 distinct
// 4-bank groups (and 8 consecutive rows on 8 distinct groups).
__device__ __forceinline__ int swz_a(int r) { return (r ^ ((r >> 3) & 3)) & 7; }

// Physical chunk of logical chunk c in B k-row r is c ^ swz_b(r): the four k-rows a
// transposing read touches at once get disjoint chunk sets both in 32-byte pairs and in
// 64-byte quads.  Pattern by r mod 4: 0, 6, 10, 12.
__device__ __forceinline__ int swz_b(int r) { return (0xCA60 >> (4 * (r & 3))) & 15; }

__device__ __forceinline__ void map_tile(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int q = total >> 3, r = total & 7;
  const int x = bid & 7, i = bid >> 3;
  const int logical = x * q + (x < r ? x : r) + i;
  constexpr int G = 4;
  const int per_group = G * tiles_n;
  const int grp = logical / per_group;
  const int first_m = grp * G;
  const int gm = (tiles_m - first_m) < G ? (tiles_m - first_m) : G;
  const int in = logical - grp * per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

__device__ __forceinline__ float gelu_erf(float u) {
  return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f));
}
__device__ __forceinline__ float silu(float u) { return u / (1.0f + expf(-u)); }

template <int ACT>
__device__ __forceinline__ float epilogue(float u, float v) {
  if constexpr (ACT == kActGelu) return gelu_erf(u);
  else if constexpr (ACT == kActSwiglu) return silu(u) * v;
  else if constexpr (ACT == kActBilinear) return u * v;
  else return u;
}

template <int BM, int BN, bool DUAL, int ACT, bool OUT_F32>
__global__ void __launch_bounds__(kThreads) gemm_bf16_kernel(GemmDesc g, int tiles_m, int tiles_n) {
  constexpr int NSUB = DUAL ? 2 : 1;          // B sub-tiles: W1 block | W3 block
  constexpr int BNS = BN / NSUB;              // B columns per sub-tile = output tile width
  constexpr int WTM = BM / 2;                 // rows per wave (2 x 2 waves)
  constexpr int MB = WTM / 32;                // 32-row MFMA blocks per wave
  constexpr int WCOLS = BNS / 2;              // sub-tile columns per wave
  constexpr int NBS = WCOLS / 32;             // 32-column MFMA blocks per wave per sub-tile
  constexpr int NB = NBS * NSUB;
  constexpr int A_BYTES = BM * kBK * 2;
  constexpr int SUB_BYTES = kBK * BNS * 2;
  constexpr int STAGE = A_BYTES + NSUB * SUB_BYTES;
  constexpr int A_LD = A_BYTES / 1024 / 4;    // 1 KiB buffer->LDS loads per wave per stage
  constexpr int B_LD = NSUB * SUB_BYTES / 1024 / 4;
  constexpr int QSUB = SUB_BYTES / 1024;      // loads per sub-tile
  constexpr int CPR = BNS / 8;                // 16-byte chunks per B row
  constexpr int PITCH = BNS * 2;              // bytes per B row
  static_assert(MB >= 1 && NBS >= 1 && A_LD >= 1 && B_LD >= 1, "tile too small");
  static_assert(CPR >= 8, "B sub-tile narrower than 64 columns");

  // One array per stage: the buffer->LDS copies into one stage and the fragment reads
  // of the other are then provably disjoint, so no wait on the copies is inserted
  // before the reads (the copies of stage k+1 overlap the products of stage k).
  __shared__ __attribute__((aligned(1024))) unsigned char smem0[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char smem1[STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  map_tile(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BNS;
  const int64_t rows_left64 = g.M - m0;
  const int rows_left = rows_left64 < BM ? (int)rows_left64 : BM;

  const __bf16* A = (const __bf16*)g.A + m0 * g.lda;
  const __bf16* B0 = (const __bf16*)g.B0 + n0;
  const __bf16* B1 = DUAL ? (const __bf16*)g.B1 + n0 : B0;

  // ---- per-lane global->LDS descriptors (fixed over the k loop).  Lanes whose row (A)
  // or column (B) lies outside the matrix get an out-of-range offset once and for all;
  // the k-tail is masked only in the last, partial k-tile.
  uint32_t a_voff[A_LD];
  int a_kc[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int q = wave * A_LD + i;
    const int row = q * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz_a(row);
    a_voff[i] = row < rows_left ? (uint32_t)(row * g.lda + 8 * c) * 2u : kOOB;
    a_kc[i] = 8 * c;
  }
  uint32_t b_voff[B_LD];
  int b_kr[B_LD];
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int q = wave * B_LD + i;
    const int pos = (q % QSUB) * 64 + lane;
    const int row = pos / CPR;
    const int c = (pos % CPR) ^ (swz_b(row) & (CPR - 1));
    b_voff[i] = (n0 + 8 * c < g.N) ? (uint32_t)(row * g.ldb + 8 * c) * 2u : kOOB;
    b_kr[i] = row;
  }
  // B sub-tile a wave's copies land in is the same for all of its copies.
  const bool b_second = (wave * B_LD) / QSUB != 0;

  // (Each offset goes through a local before the builtin call: handing the builtin an
  // element of a captured array directly makes the host compilation pass drop the
  // kernel's launch stub.)
  auto issue = [&](int kt, LDS_AS unsigned char* base) {
    const int k0 = kt * kBK;
    const bool full = k0 + kBK <= g.K;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + k0);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc((b_second ? B1 : B0) + (int64_t)k0 * g.ldb);
    if (full) {
#pragma unroll
      for (int i = 0; i < A_LD; ++i) {
        const uint32_t v = a_voff[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (LDS_AS void*)(base + (wave * A_LD + i) * 1024), 16, v, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < B_LD; ++i) {
        const uint32_t v = b_voff[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (LDS_AS void*)(base + A_BYTES + (wave * B_LD + i) * 1024), 16, v, 0, 0, 0);
      }
    } else {  // last, partial k-tile
#pragma unroll
      for (int i = 0; i < A_LD; ++i) {
        const uint32_t v = (k0 + a_kc[i] < g.K) ? a_voff[i] : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (LDS_AS void*)(base + (wave * A_LD + i) * 1024), 16, v, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < B_LD; ++i) {
        const uint32_t v = (k0 + b_kr[i] < g.K) ? b_voff[i] : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (LDS_AS void*)(base + A_BYTES + (wave * B_LD + i) * 1024), 16, v, 0, 0, 0);
      }
    }
  };


  // ---- per-lane LDS read offsets
  const int arow = wm * WTM + (lane & 31);
  uint32_t a_rd[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int c = 2 * s + (lane >> 5);
    a_rd[s] = (uint32_t)(arow * 128 + ((c ^ swz_a(arow)) << 4));
  }
  const int g4 = lane >> 4, i16 = lane & 15;
  const int krow_l = 8 * (g4 >> 1) + (i16 >> 2);
  const int sw = swz_b(krow_l) & (CPR - 1);
  uint32_t b_rd[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int sub = nb / NBS;
    const int colbase = wn * WCOLS + (nb % NBS) * 32;
    const int n = colbase + 16 * (g4 & 1) + 4 * (i16 & 3);
    b_rd[nb] = (uint32_t)(sub * SUB_BYTES + krow_l * PITCH + (((n >> 3) ^ sw) << 4) +
                          ((n >> 2) & 1) * 8);
  }

  f32x16 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x16{};

  // Fragments of k-substep s (16 k) of the stage at `As`.
  auto load_frags = [&](const LDS_AS unsigned char* As, int s, bf16x8 (&af)[MB],
                        bf16x8 (&bfr)[NB]) {
    const LDS_AS unsigned char* Bs = As + A_BYTES;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      af[mb] = *(const LDS_AS bf16x8*)(As + a_rd[s] + mb * 32 * 128);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const LDS_AS unsigned char* p = Bs + b_rd[nb] + 16 * s * PITCH;
      bf16x4_raw lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)(p));
      bf16x4_raw hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)(p + 4 * PITCH));
      bfr[nb] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  // All products of one stage.  The fragments of substep s+1 are read while substep s
  // multiplies: the scheduler is told to alternate one MFMA with one LDS read.
  constexpr int NREAD = MB + 2 * NB;  // LDS reads per substep
  constexpr int NMFMA = MB * NB;      // MFMAs per substep
  constexpr int NPAIR = NMFMA < NREAD ? NMFMA : NREAD;
  auto compute = [&](const LDS_AS unsigned char* As) {
    bf16x8 af[2][MB];
    bf16x8 bfr[2][NB];
    load_frags(As, 0, af[0], bfr[0]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) load_frags(As, s + 1, af[(s + 1) & 1], bfr[(s + 1) & 1]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[s & 1][nb], af[s & 1][mb],
                                                                 acc[mb][nb], 0, 0, 0);
    }
    // schedule: reads of substep 0, then per substep one MFMA / one read pairs
    __builtin_amdgcn_sched_group_barrier(0x100, NREAD, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) {
#pragma unroll
        for (int i = 0; i < NPAIR; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if (NMFMA > NPAIR) __builtin_amdgcn_sched_group_barrier(0x008, NMFMA - NPAIR, 0);
        if (NREAD > NPAIR) __builtin_amdgcn_sched_group_barrier(0x100, NREAD - NPAIR, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, NMFMA, 0);
      }
    }
  };

  LDS_AS unsigned char* S0 = (LDS_AS unsigned char*)smem0;
  LDS_AS unsigned char* S1 = (LDS_AS unsigned char*)smem1;
  const int nk = (g.K + kBK - 1) / kBK;
  issue(0, S0);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    issue(kt + 1, S1);                        // stays ahead of the products below
    __builtin_amdgcn_sched_barrier(0);
    compute(S0);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 2 < nk) issue(kt + 2, S0);
    __builtin_amdgcn_sched_barrier(0);
    compute(S1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (kt < nk) {  // odd number of k-tiles: the last one sits in stage 0
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    compute(S0);
  }

  // ---- epilogue: activation on the fp32 accumulators, one rounding, vector stores
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = wm * WTM + mb * 32 + (lane & 31);
    if (r >= rows_left) continue;
    const int64_t m = m0 + r;
#pragma unroll
    for (int nb = 0; nb < NBS; ++nb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * WCOLS + nb * 32 + 8 * q + 4 * (lane >> 5);
        if (n >= g.N) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float u = acc[mb][nb][4 * q + e];
          const float w = DUAL ? acc[mb][nb + NBS][4 * q + e] : 0.0f;
          v[e] = epilogue<ACT>(u, w);
        }
        if constexpr (OUT_F32) {
          float* c = (float*)g.C + m * g.ldc + n;
          *(f32x4*)c = f32x4{v[0], v[1], v[2], v[3]};
        } else {
          __bf16* c = (__bf16*)g.C + m * g.ldc + n;
          *(bf16x4*)c = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        }
      }
    }
  }
}

template <int BM, int BN, bool DUAL, int ACT, bool OUT_F32>
hipError_t launch_cfg(const GemmDesc& g, hipStream_t s) {
  constexpr int OUT_BN = DUAL ? BN / 2 : BN;
  const int64_t tm = (g.M + BM - 1) / BM;
  const int64_t tn = (g.N + OUT_BN - 1) / OUT_BN;
  if (tm * tn > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, DUAL, ACT, OUT_F32>), dim3((unsigned)(tm * tn)),
                     dim3(kThreads), 0, s, g, (int)tm, (int)tn);
  return hipGetLastError();
}

// Large tiles once they give at least one full wave of workgroups over the 256 CUs.
template <bool DUAL, int ACT, bool OUT_F32>
hipError_t launch_sized(const GemmDesc& g, hipStream_t s) {
  constexpr int OUT_BN = DUAL ? 128 : 256;
  const int64_t big = ((g.M + 255) / 256) * ((g.N + OUT_BN - 1) / OUT_BN);
  if (big >= 256) return launch_cfg<256, 256, DUAL, ACT, OUT_F32>(g, s);
  return launch_cfg<128, DUAL ? 256 : 128, DUAL, ACT, OUT_F32>(g, s);
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmDesc& g, hipStream_t s) {
  if (g.out_f32) {
    if (g.act != kActNone) return hipErrorInvalidValue;
    return launch_sized<false, kActNone, true>(g, s);
  }
  switch (g.act) {
    case kActNone: return launch_sized<false, kActNone, false>(g, s);
    case kActGelu: return launch_sized<false, kActGelu, false>(g, s);
    case kActSwiglu: return launch_sized<true, kActSwiglu, false>(g, s);
    case kActBilinear: return launch_sized<true, kActBilinear, false>(g, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tpk
