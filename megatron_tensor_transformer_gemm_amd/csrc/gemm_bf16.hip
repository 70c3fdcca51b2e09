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
// Design (one workgroup per output tile: 8 waves, two per SIMD, so that one wave of a
// SIMD multiplies while the other issues copies; small-tile fallbacks keep 4 waves.
// Forward products of more tiles than CUs run a persistent form: one workgroup per CU
// walks its tiles with the copy pipeline running on across tile boundaries):
//  * HBM/L2 -> LDS with buffer_load ... lds (16 B per lane): no staging VGPRs,
//    out-of-range rows/columns/k come back as zeros from the buffer
//    descriptor's range check (masked lanes get an out-of-range offset), so
//    ragged M, N and K need no separate edge code.
//  * Two to four LDS stages in flight: later k-tiles stream in while the current
//    one is multiplied.  In the forward layout the next stage's copies are issued one
//    at a time between the MFMAs of a stage's last substep.
//  * Products too small to fill the GPU split k over several workgroups per tile
//    (fp32 partials in the caller's workspace, summed in split order by a second
//    kernel that applies the activation).
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
#include "lds_copy.h"
#include <atomic>

namespace tpk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_raw __attribute__((__vector_size__(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))


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

// Activation arithmetic on the hardware's exp2 and reciprocal (each within about 1 ulp),
// far below the bf16 rounding of the outputs.
constexpr float kLog2e = 1.4426950408889634f;
// logistic s(u) = 1 / (1 + e^-u)
__device__ __forceinline__ float logistic(float u) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * u));
}
__device__ __forceinline__ float silu(float u) { return u * logistic(u); }
// erfc(x) by the Chebyshev-fitted form of Press et al., "Numerical Recipes" (erfcc):
// t = 1 / (1 + |x|/2), erfc(|x|) = t exp(-x^2 + P(t)) with a degree-9 polynomial P,
// fractional error below 1.2e-7 for every x; erfc(-|x|) = 2 - erfc(|x|).  Evaluating
// Phi(u) = erfc(-u / sqrt 2) / 2 this way keeps the relative accuracy of GELU's
// negative tail, which 1 + erf(u / sqrt 2) loses to cancellation.
__device__ __forceinline__ float erfc_cheb(float x) {
  const float z = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.5f * z);
  float p = 0.17087277f;
  p = __builtin_fmaf(p, t, -0.82215223f);
  p = __builtin_fmaf(p, t, 1.48851587f);
  p = __builtin_fmaf(p, t, -1.13520398f);
  p = __builtin_fmaf(p, t, 0.27886807f);
  p = __builtin_fmaf(p, t, -0.18628806f);
  p = __builtin_fmaf(p, t, 0.09678418f);
  p = __builtin_fmaf(p, t, 0.37409196f);
  p = __builtin_fmaf(p, t, 1.00002368f);
  p = __builtin_fmaf(p, t, -1.26551223f);
  const float r = t * __builtin_amdgcn_exp2f((p - z * z) * kLog2e);
  return x >= 0.0f ? r : 2.0f - r;
}
// standard normal distribution function Phi(u)
__device__ __forceinline__ float norm_cdf(float u) {
  return 0.5f * erfc_cheb(-0.70710678118654752f * u);
}
__device__ __forceinline__ float gelu(float u) { return u * norm_cdf(u); }

template <int ACT>
__device__ __forceinline__ float epilogue(float u, float v) {
  if constexpr (ACT == kActGelu) return gelu(u);
  else if constexpr (ACT == kActSwiglu) return silu(u) * v;
  else if constexpr (ACT == kActBilinear) return u * v;
  else return u;
}

// dU (and dV) from dH and the pre-activations u, v: the chain rule through the activation.
// gelu'(u) = Phi(u) + u phi(u), phi the standard normal density
__device__ __forceinline__ float gelu_grad(float u) {
  return norm_cdf(u) + u * 0.39894228040143268f * __builtin_amdgcn_exp2f(-0.5f * kLog2e * u * u);
}
template <int ACT>
__device__ __forceinline__ void act_backward(float dh, float u, float v, float& du, float& dv) {
  if constexpr (ACT == kActGelu) {
    du = dh * gelu_grad(u);
    dv = 0.0f;
  } else if constexpr (ACT == kActSwiglu) {
    const float sg = logistic(u);
    du = dh * v * sg * (1.0f + u * (1.0f - sg));
    dv = dh * u * sg;
  } else if constexpr (ACT == kActBilinear) {
    du = dh * v;
    dv = dh * u;
  } else {
    du = dh;
    dv = 0.0f;
  }
}

// Operand layouts.  kNN: A [M, K] and B [K, N] (the forward products).  kNT: B given as
// B^T [N, K], both operands k-contiguous (dH = dY W2^T, dX = dU W1^T).  kTN: A given as
// A^T [K, M], both operands m/n-contiguous (dW = X^T dU, H^T dY).  A k-contiguous operand
// is staged as [rows][BK] and read with ds_read_b128; an m/n-contiguous one as [BK][cols]
// and read with ds_read_b64_tr_b16, which transposes on the way to the registers.
enum Layout : int { kNN = 0, kNT = 1, kTN = 2 };

// Physical chunk of logical chunk c in A row r (ACPR 16-byte chunks per row) is
// c ^ swz_a<ACPR>(r): 16 consecutive rows read at one logical chunk land on 16 distinct
// 4-bank groups, and 8 consecutive rows on 8 distinct groups.
template <int ACPR>
__device__ __forceinline__ int swz_a(int r) {
  if constexpr (ACPR == 8) return (r ^ ((r >> 3) & 3)) & 7;
  else return ((r >> 2) ^ (r >> 1)) & 3;
}

// BK k per LDS stage, NST stages in flight.  The stage boundary is moved one 16-k substep
// early: the wait and barrier for stage k+1 happen before the last substep of stage k, so
// the next stage's first fragments are read, and the copies of stage k+NST are issued into
// stage k's (now free) buffer, while that last substep multiplies.
template <int BM, int BN, int BK, int NST, bool DUAL, int ACT, bool OUT_F32, int LAYOUT, bool SAVE, int NW>
__global__ void __launch_bounds__(NW * 64) gemm_bf16_kernel(GemmDesc g, int tiles_m, int tiles_n) {
  constexpr bool A_KC = LAYOUT != kTN;        // A tile [BM][BK] (else [BK][BM])
  constexpr bool B_KC = LAYOUT == kNT;        // B tile [BN][BK] (else [BK][BN])
  static_assert(!DUAL || LAYOUT == kNN, "gated pair only in the forward layout");
  static_assert(!SAVE || (LAYOUT == kNN && !OUT_F32), "pre-activations are kept by the forward");
  constexpr int NSUB = DUAL ? 2 : 1;          // B sub-tiles: W1 block | W3 block
  constexpr int BNS = BN / NSUB;              // B columns per sub-tile = output tile width
  // NW waves: 2 x 2, or with 8 waves 2 x 4 (4 x 2 when the tile's columns do not split in 4)
  constexpr int WNG = BNS % (32 * (NW / 2)) == 0 ? NW / 2 : 2;   // waves along N
  constexpr int WMG = NW / WNG;                                  // waves along M
  constexpr int WTM = BM / WMG;               // rows per wave
  constexpr int MB = WTM / 32;                // 32-row MFMA blocks per wave
  constexpr int WCOLS = BNS / WNG;            // sub-tile columns per wave
  constexpr int NBS = WCOLS / 32;             // 32-column MFMA blocks per wave per sub-tile
  constexpr int NB = NBS * NSUB;
  constexpr int KSUB = BK / 16;               // 16-k substeps per stage
  constexpr int ACPR = BK / 8;                // 16-byte chunks per A row
  constexpr int AROWB = BK * 2;               // bytes per A row
  constexpr int ARPI = 1024 / AROWB;          // A rows per 1 KiB copy
  constexpr int A_BYTES = BM * AROWB;
  constexpr int SUB_BYTES = BK * BNS * 2;
  constexpr int STAGE = A_BYTES + NSUB * SUB_BYTES;
  // Waves that issue the copies: with 8 waves only waves 0-3, one per SIMD (waves go to
  // the SIMDs round-robin), so that a wave held at copy issue, which also slows the other
  // wave of its SIMD, has a partner with no copies of its own to be held on (70B backward
  // 39.7 -> 39.4 ms per step, training forward 2,327 -> 2,297 us per rank, GPT block 9.18
  // -> 9.01 ms; three alternations on one GPU).
  constexpr int CW = NW == 8 ? NW / 2 : NW;
  constexpr int A_LD = A_BYTES / 1024 / CW;   // 1 KiB buffer->LDS copies per copying wave per stage
  constexpr int B_LD = NSUB * SUB_BYTES / 1024 / CW;
  constexpr int LPS = A_LD + B_LD;            // copies per copying wave per stage
  constexpr int QSUB = SUB_BYTES / 1024;      // copies per sub-tile
  constexpr int CPR = BNS / 8;                // 16-byte chunks per B row ([BK][BN] tile)
  constexpr int PITCH = BNS * 2;              // bytes per B row ([BK][BN] tile)
  constexpr int MCPR = BM / 8;                // 16-byte chunks per A row ([BK][BM] tile)
  constexpr int MPITCH = BM * 2;              // bytes per A row ([BK][BM] tile)
  static_assert(MB >= 1 && NBS >= 1 && A_LD >= 1 && B_LD >= 1, "tile too small");
  static_assert(CPR >= 8 && MCPR >= 8, "tile narrower than 64 columns");
  // the XOR swizzles of m/n-contiguous tiles mask the chunk index: those widths are powers
  // of two (k-contiguous A tiles may have any multiple of 64 rows, e.g. 192)
  static_assert(A_KC || (BM & (BM - 1)) == 0, "m-contiguous A tile width");
  // Swizzle of n-contiguous B rows.  Power-of-two chunk counts take swz_b.  Rows of 24
  // chunks (192 columns, 384 bytes) put k-rows r and r+2 on the same banks; XOR by
  // 2 (r mod 4) gives the four k-rows of a transposing read disjoint 32-byte pairs and
  // 64-byte quads, and touches only the low 3 bits, so every chunk stays inside its
  // aligned group of 8 (a permutation of the row's chunks).
  static_assert(B_KC || (CPR & (CPR - 1)) == 0 || CPR == 24, "n-contiguous B tile width");
  auto swz_n = [](int r) -> int {
    if constexpr ((CPR & (CPR - 1)) == 0) return swz_b(r) & (CPR - 1);
    else return (r & 3) << 1;
  };
  static_assert(A_BYTES % (1024 * CW) == 0 && (NSUB * SUB_BYTES) % (1024 * CW) == 0,
                "copies split evenly over the copying waves");
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(BM % (32 * WMG) == 0, "whole 32-row blocks per wave");
  static_assert(KSUB % 2 == 0 && (ACPR == 4 || ACPR == 8), "BK must be 32 or 64");
  static_assert(NST >= 2 && NST <= 5 && (NST - 1) * LPS <= 63, "stages");

  // One array per stage: copies into one stage and fragment reads of another are then
  // provably disjoint, so the compiler inserts no wait on the copies before the reads.
  __shared__ __attribute__((aligned(1024))) unsigned char st0[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[NST > 2 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char st3[NST > 3 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char st4[NST > 4 ? STAGE : 16];
  auto buf = [&](int i) -> LDS_AS unsigned char* {
    switch (i) {
      case 0: return (LDS_AS unsigned char*)st0;
      case 1: return (LDS_AS unsigned char*)st1;
      case 2: return (LDS_AS unsigned char*)st2;
      case 3: return (LDS_AS unsigned char*)st3;
      default: return (LDS_AS unsigned char*)st4;
    }
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WNG, wn = wave % WNG;
  const bool copier = CW == NW || wave < CW;
  const int cwave = CW == NW ? wave : wave % CW;   // the copies a copying wave issues
  int tm, tn;
  // split-K: workgroups [s * tiles, (s + 1) * tiles) take k range s (forward layout only)
  int split = 0, bid = blockIdx.x;
  // (only the plain forward with bf16 outputs splits: other kernels compile without it)
  constexpr bool CAN_SPLIT = LAYOUT == kNN && !SAVE && !OUT_F32;
  const bool splitk = CAN_SPLIT && g.ksplit > 1;
  if (splitk) {
    split = bid / (tiles_m * tiles_n);
    bid -= split * tiles_m * tiles_n;
  }
  map_tile(bid, tiles_m, tiles_n, tm, tn);
  // column segment of this tile (all values wave-uniform); pcol0: its first column in
  // the split-K partial rows
  const void* Bseg = g.B0;
  void* Cseg = g.C;
  int N_ = g.N, ldb_ = g.ldb, ldc_ = g.ldc;
  int pcol0 = 0;
  if (!DUAL && g.nseg > 1) {
    const int t0 = (g.N + BNS - 1) / BNS;
    if (tn >= t0) {
      tn -= t0;
      const int t1 = (g.Nx[0] + BNS - 1) / BNS;
      const int sg = (g.nseg > 2 && tn >= t1) ? 1 : 0;
      if (sg) tn -= t1;
      Bseg = g.Bx[sg];
      Cseg = g.Cx[sg];
      N_ = g.Nx[sg];
      ldb_ = g.ldbx[sg];
      ldc_ = g.ldcx[sg];
      pcol0 = g.N + (sg ? g.Nx[0] : 0);
    }
  }
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BNS;
  const int64_t rows_left64 = g.M - m0;
  const int rows_left = rows_left64 < BM ? (int)rows_left64 : BM;
  // k range of this workgroup
  const int kbeg = splitk ? split * g.kchunk : 0;
  const int Kv = splitk ? (g.K - kbeg < g.kchunk ? g.K - kbeg : g.kchunk) : g.K;

  // Tile origins; a k-tile then advances by k0 (k-contiguous) or k0 rows (m/n-contiguous).
  const int64_t a_org = A_KC ? m0 * g.lda + kbeg : m0;
  const int64_t b_org = B_KC ? (int64_t)n0 * ldb_ : n0 + (int64_t)kbeg * ldb_;
  const __bf16* A = (const __bf16*)g.A + a_org;
  const __bf16* B0 = (const __bf16*)Bseg + b_org;
  const __bf16* B1 = DUAL ? (const __bf16*)g.B1 + n0 + (int64_t)kbeg * ldb_ : B0;
  // second k segment (kNT): same origins in A2/B2
  const __bf16* A2 = LAYOUT == kNT && g.A2 ? (const __bf16*)g.A2 + a_org : A;
  const __bf16* B2 = LAYOUT == kNT && g.B2 ? (const __bf16*)g.B2 + b_org : B0;
  const int nk0 = LAYOUT == kNT ? (Kv + BK - 1) / BK : 0x7FFFFFFF;

  // ---- per-lane global->LDS descriptors (fixed over the k loop).  Lanes whose row (A)
  // or column (B) lies outside the matrix get an out-of-range offset once and for all;
  // the k-tail is masked only in the last, partial k-tile.
  // a_kc / b_kr: the k of the copied chunk (k-contiguous) or of the copied row.
  uint32_t a_voff[A_LD];
  int a_kc[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int q = cwave * A_LD + i;
    if constexpr (A_KC) {
      const int row = q * ARPI + lane / ACPR;
      const int c = (lane % ACPR) ^ swz_a<ACPR>(row);
      a_voff[i] = row < rows_left ? (uint32_t)(row * g.lda + 8 * c) * 2u : kOOB;
      a_kc[i] = 8 * c;
    } else {
      const int pos = q * 64 + lane;
      const int row = pos / MCPR;
      const int c = (pos % MCPR) ^ (swz_b(row) & (MCPR - 1));
      a_voff[i] = 8 * c < rows_left ? (uint32_t)(row * g.lda + 8 * c) * 2u : kOOB;
      a_kc[i] = row;
    }
  }
  uint32_t b_voff[B_LD];
  int b_kr[B_LD];
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int q = cwave * B_LD + i;
    const int pos = (q % QSUB) * 64 + lane;
    if constexpr (B_KC) {
      const int row = pos / ACPR;
      const int c = (pos % ACPR) ^ swz_a<ACPR>(row);
      b_voff[i] = n0 + row < N_ ? (uint32_t)(row * ldb_ + 8 * c) * 2u : kOOB;
      b_kr[i] = 8 * c;
    } else {
      const int row = pos / CPR;
      const int c = (pos % CPR) ^ swz_n(row);
      b_voff[i] = (n0 + 8 * c < N_) ? (uint32_t)(row * ldb_ + 8 * c) * 2u : kOOB;
      b_kr[i] = row;
    }
  }
  // B sub-tile a wave's copies land in is the same for all of its copies.
  static_assert(QSUB % B_LD == 0, "a copying wave's B copies stay within one sub-tile");
  const bool b_second = (cwave * B_LD) / QSUB != 0;

  // Copies [first, first + count) of stage kt's LPS per copying wave (A copies first, then B).
  auto issue_range = [&](int kt, LDS_AS unsigned char* base, int first, int count) {
    int k0 = kt * BK;
    int Kc = Kv;
    const __bf16* Ab = A;
    const __bf16* Bb = b_second ? B1 : B0;
    if constexpr (LAYOUT == kNT) {
      if (kt >= nk0) {   // second k segment (past its end every copy is masked)
        k0 -= nk0 * BK;
        Kc = g.K2;
        Ab = A2;
        Bb = B2;
      }
    }
    const bool full = k0 + BK <= Kc;
    i32x4 da = make_desc(Ab + (A_KC ? (int64_t)k0 : (int64_t)k0 * g.lda));
    i32x4 db = make_desc(Bb + (B_KC ? (int64_t)k0 : (int64_t)k0 * ldb_));
    if constexpr (LAYOUT != kNN) {
      // uniform, but with the copies spread between MFMAs the compiler keeps these
      // layouts' descriptors in vector registers, which the copy's assembly cannot take
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        da[w] = __builtin_amdgcn_readfirstlane(da[w]);
        db[w] = __builtin_amdgcn_readfirstlane(db[w]);
      }
    }
    const uint32_t lds = (uint32_t)(uintptr_t)base;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      if (i < first || i >= first + count) continue;
      const uint32_t v = (full || k0 + a_kc[i] < Kc) ? a_voff[i] : kOOB;
      copy16_to_lds(da, v, __builtin_amdgcn_readfirstlane(lds + (cwave * A_LD + i) * 1024));
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      if (A_LD + i < first || A_LD + i >= first + count) continue;
      const uint32_t v = (full || k0 + b_kr[i] < Kc) ? b_voff[i] : kOOB;
      copy16_to_lds(db, v,
                    __builtin_amdgcn_readfirstlane(lds + A_BYTES + (cwave * B_LD + i) * 1024));
    }
  };
  auto issue = [&](int kt, LDS_AS unsigned char* base) { issue_range(kt, base, 0, LPS); };

  // ---- per-lane LDS read offsets
  // k-contiguous tiles: row r of the fragment at lane r % 32, chunk 2*s + lane / 32.
  // m/n-contiguous tiles: 16-lane group g4 reads 4 k-rows x 16 columns per transposing read.
  const int arow = wm * WTM + (lane & 31);
  uint32_t a_rd[A_KC ? KSUB : MB];
  const int g4 = lane >> 4, i16 = lane & 15;
  const int krow_l = 8 * (g4 >> 1) + (i16 >> 2);
  if constexpr (A_KC) {
#pragma unroll
    for (int s = 0; s < KSUB; ++s) {
      const int c = 2 * s + (lane >> 5);
      a_rd[s] = (uint32_t)(arow * AROWB + ((c ^ swz_a<ACPR>(arow)) << 4));
    }
  } else {
    const int swm = swz_b(krow_l) & (MCPR - 1);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int n = wm * WTM + mb * 32 + 16 * (g4 & 1) + 4 * (i16 & 3);
      a_rd[mb] = (uint32_t)(krow_l * MPITCH + (((n >> 3) ^ swm) << 4) + ((n >> 2) & 1) * 8);
    }
  }
  const int sw = swz_n(krow_l);
  const int bcol = wn * WCOLS + (lane & 31);
  uint32_t b_rd[B_KC ? KSUB : NB];
  if constexpr (B_KC) {
#pragma unroll
    for (int s = 0; s < KSUB; ++s) {
      const int c = 2 * s + (lane >> 5);
      b_rd[s] = (uint32_t)(bcol * AROWB + ((c ^ swz_a<ACPR>(bcol)) << 4));
    }
  } else {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int sub = nb / NBS;
      const int colbase = wn * WCOLS + (nb % NBS) * 32;
      const int n = colbase + 16 * (g4 & 1) + 4 * (i16 & 3);
      b_rd[nb] = (uint32_t)(sub * SUB_BYTES + krow_l * PITCH + (((n >> 3) ^ sw) << 4) +
                            ((n >> 2) & 1) * 8);
    }
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
    for (int mb = 0; mb < MB; ++mb) {
      if constexpr (A_KC) {
        af[mb] = *(const LDS_AS bf16x8*)(As + a_rd[s] + mb * 32 * AROWB);
      } else {
        const LDS_AS unsigned char* p = As + a_rd[mb] + 16 * s * MPITCH;
        bf16x4_raw lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)(p));
        bf16x4_raw hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)(p + 4 * MPITCH));
        af[mb] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if constexpr (B_KC) {
        bfr[nb] = *(const LDS_AS bf16x8*)(Bs + b_rd[s] + nb * 32 * AROWB);
      } else {
        const LDS_AS unsigned char* p = Bs + b_rd[nb] + 16 * s * PITCH;
        bf16x4_raw lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)(p));
        bf16x4_raw hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)(p + 4 * PITCH));
        bfr[nb] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    }
  };
  // Fragment read group j of substep s, as load_frags reads it: j < MB an A fragment, else
  // a B fragment (one b128 read of a k-contiguous tile, two transposing reads otherwise);
  // the last substep of a stage interleaves them with its MFMAs one group at a time.
  auto read_group = [&](const LDS_AS unsigned char* As, int s, bf16x8 (&af)[MB], bf16x8 (&bfr)[NB],
                        int j) {
    const LDS_AS unsigned char* Bs = As + A_BYTES;
    if (j < MB) {
      if constexpr (A_KC) {
        af[j] = *(const LDS_AS bf16x8*)(As + a_rd[s] + j * 32 * AROWB);
      } else {
        const LDS_AS unsigned char* p = As + a_rd[j] + 16 * s * MPITCH;
        bf16x4_raw lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)(p));
        bf16x4_raw hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)(p + 4 * MPITCH));
        af[j] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    } else {
      const int nb = j - MB;
      if constexpr (B_KC) {
        bfr[nb] = *(const LDS_AS bf16x8*)(Bs + b_rd[s] + nb * 32 * AROWB);
      } else {
        const LDS_AS unsigned char* p = Bs + b_rd[nb] + 16 * s * PITCH;
        bf16x4_raw lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)(p));
        bf16x4_raw hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)(p + 4 * PITCH));
        bfr[nb] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    }
  };
  auto mfmas = [&](const bf16x8 (&af)[MB], const bf16x8 (&bfr)[NB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nb], af[mb], acc[mb][nb], 0, 0, 0);
  };
  // Scheduling hint for one substep with the next substep's reads: alternate one MFMA and
  // one LDS read, then the rest.
  constexpr int NREAD = (A_KC ? MB : 2 * MB) + (B_KC ? NB : 2 * NB);  // LDS reads per substep
  constexpr int NMFMA = MB * NB;      // MFMAs per substep
  constexpr int NPAIR = NMFMA < NREAD ? NMFMA : NREAD;
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < NPAIR; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if (NMFMA > NPAIR) __builtin_amdgcn_sched_group_barrier(0x008, NMFMA - NPAIR, 0);
    if (NREAD > NPAIR) __builtin_amdgcn_sched_group_barrier(0x100, NREAD - NPAIR, 0);
  };

  bf16x8 af[2][MB];
  bf16x8 bfr[2][NB];
  // k-tiles, padded to a multiple of NST: tiles past K load as zeros (every copy
  // out of range), so every stage runs the same branch-free product code.
  const int nk_all = LAYOUT == kNT ? nk0 + (g.K2 + BK - 1) / BK : (Kv + BK - 1) / BK;
  const int nk = (nk_all + NST - 1) / NST * NST;

  // The backward's dH product (kNT with the activation's derivative): U (and V) come in and
  // dU (and dV) go out through LDS as whole row segments, as the bf16 outputs do, instead
  // of 8-byte accesses spread over 32 rows per instruction (its direct form cost ~430 us of
  // a 70B rank's 5.0 ms backward).  Each wave stages its own WTM x WCOLS block of U in one
  // region and of V in a second, where the whole set fits in the stage buffers.  With
  // 64-row wave blocks the U (and V) row segments are loaded into registers before the
  // k-loop (64 VGPRs at most), so that they arrive while the tile is multiplied instead of
  // in a burst at every tile's end.
  constexpr int DSREG = WTM * WCOLS * 2;
  constexpr int DOPS = ACT == kActGelu ? 1 : 2;
  constexpr bool DSTAGED = LAYOUT == kNT && ACT != kActNone && !OUT_F32 &&
                           (WCOLS == 64 || WCOLS == 128) && STAGE % DSREG == 0 &&
                           DOPS * NW * DSREG <= NST * STAGE;
  constexpr int DSCH = WCOLS / 8, DSRPI = 64 / DSCH;   // chunks per row, rows per instruction
  constexpr bool DPRE = DSTAGED && WTM == 64 && WCOLS == 64;
  constexpr int NPRE = DPRE ? WTM / DSRPI : 1;
  const bool dstaged = DSTAGED && (N_ & 7) == 0 && (g.ldu & 7) == 0;
  bf16x8 pre_u[NPRE], pre_v[NPRE];
  if constexpr (DPRE) {
    if (dstaged) {
#pragma unroll
      for (int it = 0; it < NPRE; ++it) {
        const int row = DSRPI * it + lane / DSCH, ch = lane % DSCH;
        const int r = wm * WTM + row;
        const int n = n0 + wn * WCOLS + ch * 8;
        const bool in = r < rows_left && n < N_;
        const int64_t off = (m0 + r) * g.ldu + n;
        pre_u[it] = in ? *(const bf16x8*)((const __bf16*)g.U + off) : bf16x8{};
        if constexpr (DOPS == 2) pre_v[it] = in ? *(const bf16x8*)((const __bf16*)g.V + off) : bf16x8{};
      }
    }
  }

  // prologue: NST stages in flight, then stage 0's first fragments
#pragma unroll
  for (int p = 0; p < NST; ++p)
    if (copier) issue(p, buf(p));
  sync_copies<(NST - 1) * LPS>();
  load_frags(buf(0), 0, af[0], bfr[0]);

  // One stage; `u` is the stage's buffer (kt mod NST), a constant after unrolling.
  // Copies deferred by one substep (the backward's dX and weight-gradient products on 8
  // waves): the buffer a stage's barrier frees is not read again before the next stage's
  // barrier, so each copying wave issues the last DEFC of its copies for it in the next
  // stage's first substep, and the copy path works over twice the window.  70B rank,
  // kernel traces, two runs each: dW1|dW3 and dW2 (TN) 1,276 -> 1,233 us on average, dX
  // (NT) 1,535 -> 1,520 us.  Not used for the dH product with the activation's derivative
  // (128 x 256 tiles, three stages: 936 -> 1,013 us), nor for tiles with fewer than 8 MFMAs
  // per substep to spread the extra items over (as those), nor in the forward layout (its
  // later copies landed too late: GPT block +2.8 %, training forward +1.3 %).
  constexpr int NFR = MB + NB;
  constexpr int DEFC = (NW == 8 && LAYOUT != kNN && ACT == kActNone && MB * NB >= 8) ? LPS / 2 : 0;
  auto stage = [&](int kt, int u) {
    LDS_AS unsigned char* cur = buf(u);
    LDS_AS unsigned char* nxt = buf(u + 1 == NST ? 0 : u + 1);
    if constexpr (DEFC > 0) {
      // substep 0 with the deferred copies of k-tile kt - 1 + NST, into the buffer the
      // previous stage's barrier freed (none at kt = 0: the prologue copies whole stages)
      LDS_AS unsigned char* prv = buf(u == 0 ? NST - 1 : u - 1);
      constexpr int NIT = NFR + DEFC;
#pragma unroll
      for (int i = 0; i < NMFMA; ++i) {
        const int mb = i / NB, nb = i % NB;
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[0][nb], af[0][mb], acc[mb][nb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NIT; ++j) {
          if (j * NMFMA / NIT != i) continue;
          if (j < NFR) {
            read_group(cur, 1, af[1], bfr[1], j);
          } else {
            if (copier && kt != 0) issue_range(kt - 1 + NST, prv, LPS - DEFC + (j - NFR), 1);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int s = 1; s + 1 < KSUB; ++s) {
        load_frags(cur, s + 1, af[(s + 1) & 1], bfr[(s + 1) & 1]);
        mfmas(af[s & 1], bfr[s & 1]);
        interleave();
      }
    } else {
#pragma unroll
      for (int s = 0; s + 1 < KSUB; ++s) {
        load_frags(cur, s + 1, af[(s + 1) & 1], bfr[(s + 1) & 1]);
        mfmas(af[s & 1], bfr[s & 1]);
        interleave();
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // Stage kt+1 is complete for every wave; stage kt's buffer is free for stage kt+NST.
    // Past the end the copies are all out of range (zero fill, no memory traffic), so
    // every stage issues the same number of copies and the loop has no data-dependent
    // branches (only the wave-uniform one that skips copies on the non-copying waves).
    sync_copies<(NST - 2) * LPS>();
    // The last substep: its MFMAs with stage kt+NST's copies and then the next stage's
    // first fragment reads spread between them, items j = 0 .. LPS+NFR-1 (copies first)
    // after MFMA j*NMFMA/(LPS+NFR).  A copy holds its wave at issue for tens of cycles:
    // issued as one block after the barrier they idled the matrix pipe for about a quarter
    // of the forward's loop (cycle counters around the block); one at a time they overlap
    // the MFMA in flight, and with no fragment reads in flight yet they stall less.  (70B
    // forward 9 % fewer loop cycles; backward's NT and TN products, 8 ranks: 41.3 -> 40.3
    // ms per step.)  After the last stage the reads see a stale buffer; those fragments
    // are not used.
    constexpr int NITEM = LPS - DEFC + NFR;
#pragma unroll
    for (int i = 0; i < NMFMA; ++i) {
      const int mb = i / NB, nb = i % NB;
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[1][nb], af[1][mb], acc[mb][nb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NITEM; ++j) {
        if (j * NMFMA / NITEM != i) continue;
        if (j < LPS - DEFC) {
          if (copier) issue_range(kt + NST, cur, j, 1);
        } else {
          read_group(nxt, 0, af[0], bfr[0], j - (LPS - DEFC));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (int kt0 = 0; kt0 < nk; kt0 += NST) {
#pragma unroll
    for (int u = 0; u < NST; ++u) stage(kt0 + u, u);
  }
  // the trailing zero-fill copies must land before this workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- split-K: this workgroup's fp32 partial product (U columns, then V columns of the
  // gated pair), summed and finished by splitk_reduce_kernel
  // The partials go through LDS as the bf16 outputs do: each wave stages half of its rows
  // at a time (its whole fp32 block does not fit in the stage buffers) and stores whole row
  // segments, 16 B per lane, instead of 32 B per row over 32 rows per instruction (GPT
  // block, same GPU: 9.28 -> 9.21 ms per step).  Their bytes, not their pattern, are the
  // cost: a timing-only variant that skips these stores ran the block 11 % faster.
  if (splitk) {
    float* P = g.part + (int64_t)split * g.pslice;
    constexpr int PCOLS = NB * 32;              // fp32 columns per wave block (U, then V)
    constexpr int PCH = PCOLS / 4;              // 16-byte chunks per staged row
    constexpr int PPITCH = PCOLS * 4;           // bytes per staged row
    constexpr int PMB = (MB + 1) / 2;           // accumulator row blocks per pass
    constexpr int PREG = PMB * 32 * PPITCH;     // one wave's region
    constexpr int RPB = STAGE / PREG;           // regions per stage buffer
    constexpr bool PSTAGED = CAN_SPLIT && RPB >= 1 && NW <= NST * RPB && PCH % 8 == 0;
    if constexpr (PSTAGED) {
      // physical chunk of chunk c in staged row r: an XOR by the row inside aligned groups
      // of 8 chunks (a permutation of each row's chunks for 16 and 24 chunks alike)
      auto ppos = [](int r, int c) -> int { return (c & ~7) | ((c ^ r) & 7); };
      __syncthreads();   // every wave's copies have landed and its fragment reads are done
      LDS_AS unsigned char* R = buf(wave / RPB) + (wave % RPB) * PREG;
      static_assert((PMB * 32 * PCH) % 64 == 0, "whole store instructions");
#pragma unroll
      for (int pass = 0; pass * PMB < MB; ++pass) {
#pragma unroll
        for (int mb = pass * PMB; mb < MB && mb < (pass + 1) * PMB; ++mb) {
          const int r = (mb - pass * PMB) * 32 + (lane & 31);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int c = nb * 8 + 2 * q + (lane >> 5);
              const f32x16& a = acc[mb][nb];
              *(LDS_AS f32x4*)(R + r * PPITCH + (ppos(r, c) << 4)) =
                  f32x4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
            }
        }
#pragma unroll 4
        for (int it = 0; it < PMB * 32 * PCH / 64; ++it) {
          const int idx = it * 64 + lane;
          const int row = idx / PCH, ch = idx % PCH;
          const f32x4 v = *(const LDS_AS f32x4*)(R + row * PPITCH + (ppos(row, ch) << 4));
          const int rr = wm * WTM + pass * PMB * 32 + row;
          const int nb = ch / 8;                  // 32-column block (U blocks, then V)
          const int n = n0 + wn * WCOLS + (nb % NBS) * 32 + (ch % 8) * 4;
          if (rr < rows_left && n < N_)
            *(f32x4*)(P + (m0 + rr) * g.pld + pcol0 + (DUAL && nb >= NBS ? g.N : 0) + n) = v;
        }
      }
      return;
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int r = wm * WTM + mb * 32 + (lane & 31);
        if (r >= rows_left) continue;
        float* prow = P + (m0 + r) * g.pld + pcol0;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = n0 + wn * WCOLS + (nb % NBS) * 32 + 8 * q + 4 * (lane >> 5);
            if (n >= N_) continue;
            const f32x16& a = acc[mb][nb];
            *(f32x4*)(prow + (DUAL && nb >= NBS ? g.N : 0) + n) =
                f32x4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
          }
      }
      return;
    }
  }

  // ---- bf16 outputs through LDS.  Each lane holds 4 consecutive columns of 16 rows per
  // accumulator block, so direct stores write 8 bytes into each of 32 rows per
  // instruction.  Instead every wave rounds its WTM x WCOLS block (the forward activation
  // applied first) into a free stage buffer, rows of WCOLS*2 bytes with 16-byte chunk c of
  // row r at c ^ (r mod chunks-per-row), and stores it back as whole row segments: 256 or
  // 128 bytes per row, 4 or 8 rows per instruction (row GEMM 1,003 -> 966 us,
  // out-projection 377 -> 334 us).  The training forward's extra U/V outputs, the
  // derivative epilogues and fp32 outputs keep the direct stores below.
  // 96-column wave blocks (192-column tiles) stage too: each wave's region lies inside one
  // stage buffer, and the stores walk the block's chunks in order, 64 per instruction,
  // across row boundaries.  Their 192-byte rows repeat the bank pattern every 4 rows, so
  // chunks are permuted within aligned groups of 4 by r / 4: the 32 rows an 8-byte staging
  // write touches fall 2 to a bank group (the floor for half a wave of 8-byte writes),
  // against 8 with r mod 4; the 16-byte row-segment reads stay conflict-free.
  constexpr int SREG = WTM * WCOLS * 2;   // one wave's block, bf16
  // (32-column blocks: the gated pair's 128 output columns over 4 waves)
  constexpr bool POW2W = WCOLS == 32 || WCOLS == 64 || WCOLS == 128;
  constexpr int SPB = STAGE / SREG;       // wave regions per stage buffer (96-column blocks)
  // The training forward (SAVE) stages H, then U, then V through the same wave region
  // (8-wave tiles; the 4-wave ones have no registers to spare for it).
  constexpr bool STAGED = !OUT_F32 && (!SAVE || (LAYOUT == kNN && POW2W && NW == 8)) &&
                          (ACT == kActNone || LAYOUT == kNN) &&
                          (POW2W ? STAGE % SREG == 0 && NW * SREG <= NST * STAGE
                                 : WCOLS == 96 && SPB >= 1 && NW <= NST * SPB);
  if constexpr (DSTAGED) {
    if (dstaged) {
      constexpr int SCH = WCOLS / 8;        // 16-byte chunks per staged row
      constexpr int SPITCH = WCOLS * 2;     // bytes per staged row
      constexpr int SRPI = 64 / SCH;        // rows per load / store instruction
      auto spos = [](int r, int c) -> int { return (c ^ r) & (SCH - 1); };
      auto region = [&](int i) -> LDS_AS unsigned char* {
        const int off = i * SREG;
        return buf(off / STAGE) + off % STAGE;
      };
      LDS_AS unsigned char* RU = region(wave);
      LDS_AS unsigned char* RV = region(DOPS == 2 ? NW + wave : wave);
      __syncthreads();   // every wave's copies have landed and its fragment reads are done
      // U [, V] of this wave's block -> LDS (zeros outside the matrix; never stored back)
      if constexpr (DPRE) {
#pragma unroll
        for (int it = 0; it < NPRE; ++it) {
          const int row = SRPI * it + lane / SCH, ch = lane % SCH;
          *(LDS_AS bf16x8*)(RU + row * SPITCH + (spos(row, ch) << 4)) = pre_u[it];
          if constexpr (DOPS == 2) *(LDS_AS bf16x8*)(RV + row * SPITCH + (spos(row, ch) << 4)) = pre_v[it];
        }
      } else {
#pragma unroll 4
        for (int it = 0; it < WTM / SRPI; ++it) {
          const int row = SRPI * it + lane / SCH, ch = lane % SCH;
          const int r = wm * WTM + row;
          const int n = n0 + wn * WCOLS + ch * 8;
          const bool in = r < rows_left && n < N_;
          const int64_t off = (m0 + r) * g.ldu + n;
          const bf16x8 u = in ? *(const bf16x8*)((const __bf16*)g.U + off) : bf16x8{};
          *(LDS_AS bf16x8*)(RU + row * SPITCH + (spos(row, ch) << 4)) = u;
          if constexpr (DOPS == 2) {
            const bf16x8 v = in ? *(const bf16x8*)((const __bf16*)g.V + off) : bf16x8{};
            *(LDS_AS bf16x8*)(RV + row * SPITCH + (spos(row, ch) << 4)) = v;
          }
        }
      }
      __syncthreads();
      // dU [, dV] from dH (the accumulators) at the same places, written back in place
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int r = mb * 32 + (lane & 31);
#pragma unroll
        for (int nb = 0; nb < NBS; ++nb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = nb * 32 + 8 * q + 4 * (lane >> 5);
            const int pos = r * SPITCH + (spos(r, c >> 3) << 4) + (c & 7) * 2;
            const bf16x4 uu = *(const LDS_AS bf16x4*)(RU + pos);
            bf16x4 vv = bf16x4{};
            if constexpr (DOPS == 2) vv = *(const LDS_AS bf16x4*)(RV + pos);
            float du[4], dv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              act_backward<ACT>(acc[mb][nb][4 * q + e], (float)uu[e], (float)vv[e], du[e], dv[e]);
            *(LDS_AS bf16x4*)(RU + pos) = bf16x4{(__bf16)du[0], (__bf16)du[1], (__bf16)du[2], (__bf16)du[3]};
            if constexpr (DOPS == 2)
              *(LDS_AS bf16x4*)(RV + pos) = bf16x4{(__bf16)dv[0], (__bf16)dv[1], (__bf16)dv[2], (__bf16)dv[3]};
          }
      }
      __syncthreads();
#pragma unroll 4
      for (int it = 0; it < WTM / SRPI; ++it) {
        const int row = SRPI * it + lane / SCH, ch = lane % SCH;
        const int r = wm * WTM + row;
        const int n = n0 + wn * WCOLS + ch * 8;
        if (r < rows_left && n < N_) {
          const int64_t off = (m0 + r) * ldc_ + n;
          // non-temporal: dX and dW read dU, dV later, after other tiles' traffic (70B
          // backward 39.89 -> 39.78 ms)
          __builtin_nontemporal_store(*(const LDS_AS bf16x8*)(RU + row * SPITCH + (spos(row, ch) << 4)),
                                      (bf16x8*)((__bf16*)Cseg + off));
          if constexpr (DOPS == 2)
            __builtin_nontemporal_store(*(const LDS_AS bf16x8*)(RV + row * SPITCH + (spos(row, ch) << 4)),
                                        (bf16x8*)((__bf16*)g.dV + off));
        }
      }
      return;
    }
  }
  if constexpr (STAGED) {
    if ((N_ & 7) == 0 && (!SAVE || (g.ldu & 7) == 0)) {
      constexpr int SCH = WCOLS / 8;        // 16-byte chunks per staged row
      constexpr int SPITCH = WCOLS * 2;     // bytes per staged row
      // physical chunk of chunk c in staged row r
      // 64-byte rows (4 chunks) repeat the bank pattern every 4 rows, as the 192-byte ones
      // do: permute by r / 4 there too (70B column GEMM + SwiGLU: 1,462 -> 1,456 us against
      // its earlier direct stores)
      auto spos = [](int r, int c) -> int {
        if constexpr (SCH == 4) return (c ^ (r >> 2)) & 3;
        else if constexpr (POW2W) return (c ^ r) & (SCH - 1);
        else return (c & ~3) | ((c ^ (r >> 2)) & 3);
      };
      // Products without an activation (row GEMM, out-projection, dX: partial sums that the
      // partial-sum kernel reads later, from HBM) are stored non-temporally (70B step, same
      // GPU: out-projection 271 -> 266 us, the partial sum after the row GEMMs 439 -> 433
      // us).  H, which the row GEMM reads next, keeps ordinary stores (non-temporal ones
      // there measured level).
      auto store_out = [](const bf16x8& v, bf16x8* dst) {
        if constexpr (ACT == kActNone) __builtin_nontemporal_store(v, dst);
        else *dst = v;
      };
      __syncthreads();   // every wave's copies have landed and its fragment reads are done
      LDS_AS unsigned char* R;
      if constexpr (POW2W) {
        const int off = wave * SREG;
        R = buf(off / STAGE) + off % STAGE;
      } else {
        R = buf(wave / SPB) + (wave % SPB) * SREG;
      }
      // one pass per output: H (activated); with SAVE also U and V (pre-activations)
      constexpr int NPASS = SAVE ? (DUAL ? 3 : 2) : 1;
#pragma unroll
      for (int pass = 0; pass < NPASS; ++pass) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int r = mb * 32 + (lane & 31);
#pragma unroll
          for (int nb = 0; nb < NBS; ++nb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int c = nb * 32 + 8 * q + 4 * (lane >> 5);
              float v[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float u = acc[mb][nb][4 * q + e];
                if (pass == 1) v[e] = u;
                else if (pass == 2) v[e] = acc[mb][nb + NBS][4 * q + e];
                else if constexpr (LAYOUT == kNN) v[e] = epilogue<ACT>(u, DUAL ? acc[mb][nb + NBS][4 * q + e] : 0.0f);
                else v[e] = u;
              }
              *(LDS_AS bf16x4*)(R + r * SPITCH + (spos(r, c >> 3) << 4) + (c & 7) * 2) =
                  bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
            }
        }
        if (pass == 0) __syncthreads();
        if constexpr (POW2W) {
          constexpr int SRPI = 64 / SCH;      // rows per store instruction
          __bf16* dst = pass == 0 ? (__bf16*)Cseg : (__bf16*)(pass == 1 ? g.U : g.V);
          const int64_t ld = pass == 0 ? ldc_ : g.ldu;
#pragma unroll 4
          for (int it = 0; it < WTM / SRPI; ++it) {
            const int row = SRPI * it + lane / SCH, ch = lane % SCH;
            const int r = wm * WTM + row;
            const int n = n0 + wn * WCOLS + ch * 8;
            const bf16x8 v = *(const LDS_AS bf16x8*)(R + row * SPITCH + (spos(row, ch) << 4));
            if (r < rows_left && n < N_) store_out(v, (bf16x8*)(dst + (m0 + r) * ld + n));
          }
        } else {
          static_assert((WTM * SCH) % 64 == 0, "whole store instructions");
#pragma unroll 4
          for (int it = 0; it < WTM * SCH / 64; ++it) {
            const int idx = it * 64 + lane;
            const int row = idx / SCH, ch = idx % SCH;
            const int r = wm * WTM + row;
            const int n = n0 + wn * WCOLS + ch * 8;
            const bf16x8 v = *(const LDS_AS bf16x8*)(R + row * SPITCH + (spos(row, ch) << 4));
            if (r < rows_left && n < N_) store_out(v, (bf16x8*)((__bf16*)Cseg + (m0 + r) * ldc_ + n));
          }
        }
      }
      return;
    }
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
        if (n >= N_) continue;
        float v[4];
        if constexpr (LAYOUT == kNT && ACT != kActNone) {
          // accumulator = dH; U [, V] saved by the forward -> dU (C) [, dV]
          const bf16x4 uu = *(const bf16x4*)((const __bf16*)g.U + m * g.ldu + n);
          bf16x4 vv = bf16x4{};
          if constexpr (ACT != kActGelu) vv = *(const bf16x4*)((const __bf16*)g.V + m * g.ldu + n);
          float dv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            act_backward<ACT>(acc[mb][nb][4 * q + e], (float)uu[e], (float)vv[e], v[e], dv[e]);
          if constexpr (ACT != kActGelu)
            *(bf16x4*)((__bf16*)g.dV + m * ldc_ + n) =
                bf16x4{(__bf16)dv[0], (__bf16)dv[1], (__bf16)dv[2], (__bf16)dv[3]};
        } else if constexpr (LAYOUT == kNN) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float u = acc[mb][nb][4 * q + e];
            const float w = DUAL ? acc[mb][nb + NBS][4 * q + e] : 0.0f;
            v[e] = epilogue<ACT>(u, w);
          }
          if constexpr (SAVE) {   // keep the pre-activations for the backward pass
            const f32x16& au = acc[mb][nb];
            *(bf16x4*)((__bf16*)g.U + m * g.ldu + n) =
                bf16x4{(__bf16)au[4 * q], (__bf16)au[4 * q + 1], (__bf16)au[4 * q + 2], (__bf16)au[4 * q + 3]};
            if constexpr (DUAL) {
              const f32x16& av = acc[mb][nb + NBS];
              *(bf16x4*)((__bf16*)g.V + m * g.ldu + n) =
                  bf16x4{(__bf16)av[4 * q], (__bf16)av[4 * q + 1], (__bf16)av[4 * q + 2], (__bf16)av[4 * q + 3]};
            }
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[mb][nb][4 * q + e];
        }
        if constexpr (OUT_F32) {
          float* c = (float*)Cseg + m * ldc_ + n;
          *(f32x4*)c = f32x4{v[0], v[1], v[2], v[3]};
        } else {
          __bf16* c = (__bf16*)Cseg + m * ldc_ + n;
          *(bf16x4*)c = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        }
      }
    }
  }
}

// ---- Forward products of more than one wave of 256 x 256 tiles: one workgroup per CU
// takes tiles gridDim.x apart, and the copy pipeline runs on across tile boundaries.  The
// second-to-last stage of a tile copies k-tile 0 of the workgroup's next tile (instead of
// the zero fill that pads a lone tile's loop); the last stage copies nothing (beyond the
// deferred part of that k-tile, in the plain products), so that k-tile 0 arrives while
// the last stages multiply; k-tile 1 is issued between the last stage's final MFMAs,
// and k-tile 0 waited for before the epilogue's first store.  The epilogue therefore may not use the stage
// buffers: each wave rounds its 128-row block 32 rows at a time into a 4 KiB region of
// its own (32 KiB beside the two 64 KiB stages: the whole 160 KiB of LDS) and stores
// whole row segments from there, with no workgroup barrier.
// A workgroup launched per tile cost 4-5 us per tile that this hides (probe timestamps in
// the 70B products: dispatch gap 0.8-1.3 us, prologue 1.9-2.5 us, store drain 0.4-0.8 us).
// Fragment reads and MFMA order are those of gemm_bf16_kernel in the forward layout with
// 256 x 256 x 64 tiles, two stages and 8 waves, so the results are bit-identical.  The
// copies differ: waves 0-3 issue all of them (16 per stage each), waves 4-7 none.  Waves go
// to the SIMDs round-robin, so each SIMD pairs a copying wave with one free of copies; a
// wave held at copy issue (the L2 -> LDS path takes 16-18 cycles per 1 KiB copy per CU,
// a stage's 64 copies half the stage's MFMA time) slows the other wave of its SIMD, which
// then has no copies of its own to be held on.  Measured on the 70B products over nine
// alternations: forward step 0.5-0.6 % faster, row GEMM 0.5 %, out-projection 1.2 %.
template <bool DUAL, int ACT>
__global__ void __launch_bounds__(512) gemm_fwd_persistent_kernel(GemmDesc g, int tiles_m, int tiles_n) {
  constexpr int BM = 256, BN = 256, BK = 64, NST = 2, NW = 8;
  constexpr int NSUB = DUAL ? 2 : 1;          // B sub-tiles: W1 block | W3 block
  constexpr int BNS = BN / NSUB;              // output columns per tile
  constexpr int WNG = 4;                      // waves along N (2 x 4)
  constexpr int WTM = BM / (NW / WNG);        // 128 rows per wave
  constexpr int MB = WTM / 32;
  constexpr int WCOLS = BNS / WNG;            // 32 (gated pair) or 64 columns per wave
  constexpr int NBS = WCOLS / 32;
  constexpr int NB = NBS * NSUB;
  constexpr int KSUB = BK / 16;
  constexpr int ACPR = BK / 8;
  constexpr int AROWB = BK * 2;
  constexpr int ARPI = 1024 / AROWB;
  constexpr int A_BYTES = BM * AROWB;
  constexpr int SUB_BYTES = BK * BNS * 2;
  constexpr int STAGE = A_BYTES + NSUB * SUB_BYTES;
  constexpr int CW = NW / 2;                  // copying waves: 0 .. CW-1
  constexpr int A_LD = A_BYTES / 1024 / CW;   // 1 KiB copies per copying wave per stage
  constexpr int B_LD = NSUB * SUB_BYTES / 1024 / CW;
  constexpr int LPS = A_LD + B_LD;
  constexpr int QSUB = SUB_BYTES / 1024;
  constexpr int CPR = BNS / 8;
  constexpr int PITCH = BNS * 2;
  constexpr int ECH = WCOLS / 8;              // 16-byte chunks per staged row
  constexpr int EPITCH = WCOLS * 2;           // bytes per staged row
  constexpr int ERPI = 64 / ECH;              // staged rows per store instruction
  constexpr int EREG = 4096;                  // one wave's staging region
  static_assert(STAGE == 65536 && LPS == 16 && 32 * EPITCH <= EREG, "tile shape");
  static_assert(2 * STAGE + NW * EREG <= 160 * 1024, "LDS");

  __shared__ __attribute__((aligned(1024))) unsigned char st0[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char ep[NW * EREG];
  auto buf = [&](int i) -> LDS_AS unsigned char* {
    return i == 0 ? (LDS_AS unsigned char*)st0 : (LDS_AS unsigned char*)st1;
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WNG, wn = wave % WNG;
  const bool copier = wave < CW;
  const int cwave = wave % CW;                // the copies a copying wave issues
  const int64_t ntile = (int64_t)tiles_m * tiles_n;
  const int nk = ((g.K + BK - 1) / BK + NST - 1) / NST * NST;   // k-tiles, padded

  // ---- the tile whose stages are being copied.  The k of a lane's A chunk and its B
  // k-row do not depend on the tile; the offsets do (masks, segment strides).
  int a_kc[A_LD], b_kr[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int row = (cwave * A_LD + i) * ARPI + lane / ACPR;
    a_kc[i] = 8 * ((lane % ACPR) ^ swz_a<ACPR>(row));
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) b_kr[i] = (((cwave * B_LD + i) % QSUB) * 64 + lane) / CPR;
  static_assert(QSUB % B_LD == 0, "a copying wave's B copies stay within one sub-tile");
  const bool b_second = (cwave * B_LD) / QSUB != 0;
  uint32_t a_voff[A_LD], b_voff[B_LD];
  const __bf16* A = nullptr;
  const __bf16* Bc = nullptr;                 // this wave's B sub-tile
  __bf16* Cseg = nullptr;
  int64_t m0 = 0;
  int n0 = 0, rows_left = 0, N_ = 0, ldb_ = 0, ldc_ = 0;
  // has_tile false: every copy out of range (zero fill, no memory traffic)
  auto set_tile = [&](int64_t tile, bool has_tile) {
    int tm = 0, tn = 0;
    if (has_tile) map_tile((int)tile, tiles_m, tiles_n, tm, tn);
    const void* Bseg = g.B0;
    void* Cs = g.C;
    int Nn = g.N, ldb = g.ldb, ldc = g.ldc;
    if (!DUAL && g.nseg > 1) {
      const int t0 = (g.N + BNS - 1) / BNS;
      if (tn >= t0) {
        tn -= t0;
        const int t1 = (g.Nx[0] + BNS - 1) / BNS;
        const int sg = (g.nseg > 2 && tn >= t1) ? 1 : 0;
        if (sg) tn -= t1;
        Bseg = g.Bx[sg];
        Cs = g.Cx[sg];
        Nn = g.Nx[sg];
        ldb = g.ldbx[sg];
        ldc = g.ldcx[sg];
      }
    }
    m0 = (int64_t)tm * BM;
    n0 = tn * BNS;
    const int64_t rl = g.M - m0;
    rows_left = has_tile ? (rl < BM ? (int)rl : BM) : 0;
    N_ = Nn;
    ldb_ = ldb;
    ldc_ = ldc;
    Cseg = (__bf16*)Cs;
    A = (const __bf16*)g.A + m0 * g.lda;
    Bc = (const __bf16*)(DUAL && b_second ? g.B1 : Bseg) + n0;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int row = (cwave * A_LD + i) * ARPI + lane / ACPR;
      a_voff[i] = row < rows_left ? (uint32_t)(row * g.lda + a_kc[i]) * 2u : kOOB;
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int pos = ((cwave * B_LD + i) % QSUB) * 64 + lane;
      const int c = (pos % CPR) ^ (swz_b(b_kr[i]) & (CPR - 1));
      b_voff[i] = (has_tile && n0 + 8 * c < N_) ? (uint32_t)(b_kr[i] * ldb_ + 8 * c) * 2u : kOOB;
    }
  };

  // Copies [first, first + count) of k-tile kt of the tile set_tile chose (copying waves).
  auto issue_range = [&](int kt, LDS_AS unsigned char* base, int first, int count) {
    const int k0 = kt * BK;
    const bool full = k0 + BK <= g.K;
    const i32x4 da = make_desc(A + k0);
    const i32x4 db = make_desc(Bc + (int64_t)k0 * ldb_);
    const uint32_t lds = (uint32_t)(uintptr_t)base;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      if (i < first || i >= first + count) continue;
      const uint32_t v = (full || k0 + a_kc[i] < g.K) ? a_voff[i] : kOOB;
      copy16_to_lds(da, v, __builtin_amdgcn_readfirstlane(lds + (cwave * A_LD + i) * 1024));
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      if (A_LD + i < first || A_LD + i >= first + count) continue;
      const uint32_t v = (full || k0 + b_kr[i] < g.K) ? b_voff[i] : kOOB;
      copy16_to_lds(db, v, __builtin_amdgcn_readfirstlane(lds + A_BYTES + (cwave * B_LD + i) * 1024));
    }
  };

  // ---- per-lane LDS read offsets (as gemm_bf16_kernel)
  const int arow = wm * WTM + (lane & 31);
  uint32_t a_rd[KSUB];
#pragma unroll
  for (int s = 0; s < KSUB; ++s) {
    const int c = 2 * s + (lane >> 5);
    a_rd[s] = (uint32_t)(arow * AROWB + ((c ^ swz_a<ACPR>(arow)) << 4));
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
    b_rd[nb] = (uint32_t)(sub * SUB_BYTES + krow_l * PITCH + (((n >> 3) ^ sw) << 4) + ((n >> 2) & 1) * 8);
  }

  f32x16 acc[MB][NB];
  bf16x8 af[2][MB];
  bf16x8 bfr[2][NB];
  auto load_frags = [&](const LDS_AS unsigned char* As, int s, bf16x8 (&a)[MB], bf16x8 (&b)[NB]) {
    const LDS_AS unsigned char* Bs = As + A_BYTES;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) a[mb] = *(const LDS_AS bf16x8*)(As + a_rd[s] + mb * 32 * AROWB);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const LDS_AS unsigned char* p = Bs + b_rd[nb] + 16 * s * PITCH;
      bf16x4_raw lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)(p));
      bf16x4_raw hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)(p + 4 * PITCH));
      b[nb] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  auto read_group = [&](const LDS_AS unsigned char* As, int j) {
    if (j < MB) {
      af[0][j] = *(const LDS_AS bf16x8*)(As + a_rd[0] + j * 32 * AROWB);
    } else {
      const int nb = j - MB;
      const LDS_AS unsigned char* p = As + A_BYTES + b_rd[nb];
      bf16x4_raw lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)(p));
      bf16x4_raw hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)(p + 4 * PITCH));
      bfr[0][nb] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  // fragment group j (A groups, then B groups) of substep s into register set st
  auto read_grp = [&](const LDS_AS unsigned char* As, int s, int st, int j) {
    if (j < MB) {
      af[st][j] = *(const LDS_AS bf16x8*)(As + a_rd[s] + j * 32 * AROWB);
    } else {
      const int nb = j - MB;
      const LDS_AS unsigned char* p = As + A_BYTES + b_rd[nb] + 16 * s * PITCH;
      bf16x4_raw lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)(p));
      bf16x4_raw hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_raw*)(p + 4 * PITCH));
      bfr[st][nb] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  auto mfmas = [&](const bf16x8 (&a)[MB], const bf16x8 (&b)[NB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[nb], a[mb], acc[mb][nb], 0, 0, 0);
  };
  constexpr int NREAD = MB + 2 * NB;
  constexpr int NMFMA = MB * NB;
  constexpr int NPAIR = NMFMA < NREAD ? NMFMA : NREAD;
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < NPAIR; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if (NMFMA > NPAIR) __builtin_amdgcn_sched_group_barrier(0x008, NMFMA - NPAIR, 0);
    if (NREAD > NPAIR) __builtin_amdgcn_sched_group_barrier(0x100, NREAD - NPAIR, 0);
  };

  // Epilogue target of the tile being multiplied (set_tile moves on to the next tile
  // before the last stages' copies)
  __bf16* e_c = nullptr;
  int64_t e_m0 = 0;
  int e_n0 = 0, e_rows = 0, e_N = 0, e_ldc = 0;
  int64_t tile = blockIdx.x;
  bool next_ok = false;

  // One stage of the tile (all but the last); at stage nk - NST the copies move on to
  // the next tile.
  // Copies deferred by one substep.  The buffer a stage's barrier frees is not read again
  // until after the next stage's barrier, so the plain products (row GEMM, out-projection)
  // issue the last DEFC of each copying wave's copies for it in the next stage's first
  // substep instead of the stage tail: the copy path (16-18 cycles per 1 KiB copy per CU)
  // then works over twice the window.  70B row GEMM 750 -> 735 us, out-projection 245 ->
  // 241.5 us (three alternations, one GPU).  The gated column GEMM, whose A panels come
  // from beyond L2 more often, keeps every copy in the tail: the later copies have less
  // time to land before the next barrier, and deferring 2 or 4 of 8 there was slower.
  constexpr int NFR = MB + NB;
  constexpr int DEFC = DUAL ? 0 : LPS / 2;
  // Substep 0 of a stage: its MFMAs, the fragment reads of substep 1 and the deferred
  // copies of k-tile kd into nb_buf (`copies`: false where the previous stage left none).
  auto sub0 = [&](const LDS_AS unsigned char* cur, LDS_AS unsigned char* nb_buf, int kd, bool copies) {
    constexpr int NIT = NFR + DEFC;
#pragma unroll
    for (int i = 0; i < NMFMA; ++i) {
      const int mb = i / NB, nb = i % NB;
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[0][nb], af[0][mb], acc[mb][nb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NIT; ++j) {
        if (j * NMFMA / NIT != i) continue;
        if (j < NFR) {
          read_grp(cur, 1, 1, j);
        } else {
          if (copier && copies) issue_range(kd, nb_buf, LPS - DEFC + (j - NFR), 1);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the substeps from `first` on whose reads are of the same stage
  auto substeps = [&](const LDS_AS unsigned char* cur, int first) {
#pragma unroll
    for (int s = first; s + 1 < KSUB; ++s) {
      load_frags(cur, s + 1, af[(s + 1) & 1], bfr[(s + 1) & 1]);
      mfmas(af[s & 1], bfr[s & 1]);
      interleave();
    }
  };
  auto stage = [&](int kt, int u) {
    LDS_AS unsigned char* cur = buf(u);
    LDS_AS unsigned char* nxt = buf(u + 1 == NST ? 0 : u + 1);
    if constexpr (DEFC > 0) {
      // k-tile kt+1's deferred copies (none at a tile's first stage: the transition
      // copies k-tile 1 whole)
      sub0(cur, nxt, kt + 1, kt != 0);
      substeps(cur, 1);
    } else {
      substeps(cur, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // k-tile kt+1 (of this tile or the next) is complete for every wave; this stage's
    // buffer is free for k-tile kt+NST
    sync_copies<(NST - 2) * LPS>();
    if (kt == nk - NST) {
      e_c = Cseg;
      e_m0 = m0;
      e_n0 = n0;
      e_rows = rows_left;
      e_N = N_;
      e_ldc = ldc_;
      next_ok = tile + gridDim.x < ntile;
      set_tile(tile + gridDim.x, next_ok);
    }
    const int kc = kt + NST < nk ? kt + NST : kt + NST - nk;
    __builtin_amdgcn_sched_barrier(0);
    constexpr int NITEM = LPS - DEFC + NFR;
#pragma unroll
    for (int i = 0; i < NMFMA; ++i) {
      const int mb = i / NB, nb = i % NB;
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[1][nb], af[1][mb], acc[mb][nb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NITEM; ++j) {
        if (j * NMFMA / NITEM != i) continue;
        if (j < LPS - DEFC) {
          if (copier) issue_range(kc, cur, j, 1);
        } else {
          read_group(nxt, j - (LPS - DEFC));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Products without an activation (partial sums read later by the partial-sum kernel)
  // are stored non-temporally, as in gemm_bf16_kernel.  (Every output segment is a
  // multiple of 8 columns wide with 16-byte aligned rows: the launcher checks.)
  auto store_out = [](const bf16x8& v, bf16x8* dst) {
    if constexpr (ACT == kActNone) __builtin_nontemporal_store(v, dst);
    else *dst = v;
  };
  // physical chunk of chunk c in staged row r (as gemm_bf16_kernel's staging)
  auto spos = [](int r, int c) -> int {
    if constexpr (ECH == 4) return (c ^ (r >> 2)) & 3;
    else return (c ^ r) & (ECH - 1);
  };
  LDS_AS unsigned char* E = (LDS_AS unsigned char*)ep + wave * EREG;

  // ---- first tile: prologue
  set_tile(tile, true);
#pragma unroll
  for (int p = 0; p < NST; ++p)
    if (copier) issue_range(p, buf(p), 0, LPS);
  sync_copies<(NST - 1) * LPS>();
  load_frags(buf(0), 0, af[0], bfr[0]);

  static_assert(NST == 2, "the tile transition below assumes two stages");
  for (;;) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x16{};
    for (int kt0 = 0; kt0 + NST < nk; kt0 += NST) {
#pragma unroll
      for (int u = 0; u < NST; ++u) stage(kt0 + u, u);
    }
    stage(nk - 2, 0);   // copies k-tile 0 of the next tile
    // The last stage: no reads of the next stage and no wait for copies, so that the next
    // tile's k-tile 0 (copied since stage nk - 2, and in the plain products partly in this
    // stage's first substep) is waited for only in the epilogue; its last MFMAs carry the
    // next tile's k-tile 1 copies.
    {
      const LDS_AS unsigned char* cur = buf(1);
      if constexpr (DEFC > 0) {
        sub0(cur, buf(0), 0, true);   // the next tile's k-tile 0, deferred part
        substeps(cur, 1);
      } else {
        substeps(cur, 0);
      }
      // Every wave has read buffer 1 once its last fragment reads are done: the next
      // tile's k-tile 1 goes in during the last MFMAs, ahead of this tile's stores in the
      // copy path.  (Against issuing it after the epilogue, which made the transition wait
      // for the stores: out-projection 238.7 -> 234.4 us, row GEMM 732 -> 729 us; issuing
      // it between the last MFMAs rather than after them: row GEMM 724.9 -> 720.5 us.
      // Three alternations on one GPU each.)
      __builtin_amdgcn_sched_barrier(0);
      if (next_ok) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int i = 0; i < NMFMA; ++i) {
        const int mb = i / NB, nb = i % NB;
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[1][nb], af[1][mb], acc[mb][nb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < LPS; ++j) {
          if (j * NMFMA / LPS != i) continue;
          if (copier && next_ok) issue_range(1, buf(1), j, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // ---- epilogue: 32 rows at a time through this wave's own region; the next tile's
    // first stages are in flight meanwhile.  (The lane index goes through an empty asm so
    // that the epilogue's per-lane offsets are formed here rather than hoisted out of the
    // tile loop, where they would hold registers through every k-loop.)
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = ln & 31;
#pragma unroll
      for (int nb = 0; nb < NBS; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = nb * 32 + 8 * q + 4 * (ln >> 5);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = epilogue<ACT>(acc[mb][nb][4 * q + e], DUAL ? acc[mb][nb + NBS][4 * q + e] : 0.0f);
          *(LDS_AS bf16x4*)(E + r * EPITCH + (spos(r, c >> 3) << 4) + (c & 7) * 2) =
              bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        }
      // Before the first store: the next tile's k-tile 0 complete for this wave.  Its copies
      // are older than k-tile 1's LPS and no store is in flight yet, so the count is exact
      // (the stores themselves, some skipped on ragged tiles, are left to drain during the
      // next tile's first stage, whose wait covers them).
      if (mb == 0 && next_ok) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPS) : "memory");
#pragma unroll
      for (int it = 0; it < 32 / ERPI; ++it) {
        const int row = ERPI * it + ln / ECH, ch = ln % ECH;
        const bf16x8 v = *(const LDS_AS bf16x8*)(E + row * EPITCH + (spos(row, ch) << 4));
        const int rr = wm * WTM + mb * 32 + row;
        const int n = e_n0 + wn * WCOLS + ch * 8;
        if (rr < e_rows && n < e_N) store_out(v, (bf16x8*)(e_c + (e_m0 + rr) * e_ldc + n));
      }
    }
    if (!next_ok) break;
    tile += gridDim.x;
    // k-tile 0 complete for every wave (each copying wave waited for its own copies)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    load_frags(buf(0), 0, af[0], bfr[0]);
  }
  // the trailing zero-fill copies must land before the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Compute units of the current device (cached per device; 0 if the query fails).
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// A bf16 forward product with more tiles of 256 x 256 than the GPU has CUs runs on the
// persistent kernel, one workgroup per CU; false when it does not apply.
template <bool DUAL, int ACT>
bool launch_persistent(const GemmDesc& g, hipStream_t s, hipError_t& e) {
  constexpr int OUT_BN = DUAL ? 128 : 256;
  const int64_t tm = (g.M + 255) / 256;
  int64_t tn = (g.N + OUT_BN - 1) / OUT_BN;
  for (int i = 0; i + 1 < g.nseg && !DUAL; ++i) tn += (g.Nx[i] + OUT_BN - 1) / OUT_BN;
  const int cus = device_cus();
  if (g.ksplit > 1 || cus <= 0 || tm * tn <= cus || tm * tn > 0x7FFFFFFF) return false;
  // the epilogue stores 16-byte row segments
  bool rows16 = g.N % 8 == 0 && g.ldc % 8 == 0;
  for (int i = 0; i + 1 < g.nseg && !DUAL; ++i) rows16 = rows16 && g.Nx[i] % 8 == 0 && g.ldcx[i] % 8 == 0;
  if (!rows16) return false;
  hipLaunchKernelGGL((gemm_fwd_persistent_kernel<DUAL, ACT>), dim3((unsigned)cus), dim3(512), 0, s, g,
                     (int)tm, (int)tn);
  e = hipGetLastError();
  return true;
}

template <int BM, int BN, int BK, int NST, bool DUAL, int ACT, bool OUT_F32, int LAYOUT, bool SAVE, int NW = 4>
hipError_t launch_cfg(const GemmDesc& g, hipStream_t s) {
  constexpr int OUT_BN = DUAL ? BN / 2 : BN;
  const int64_t tm = (g.M + BM - 1) / BM;
  int64_t tn = (g.N + OUT_BN - 1) / OUT_BN;
  for (int i = 0; i + 1 < g.nseg && !DUAL; ++i) tn += (g.Nx[i] + OUT_BN - 1) / OUT_BN;
  const int64_t ks = LAYOUT == kNN && g.ksplit > 1 ? g.ksplit : 1;
  if (tm * tn * ks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, NST, DUAL, ACT, OUT_F32, LAYOUT, SAVE, NW>),
                     dim3((unsigned)(tm * tn * ks)), dim3(NW * 64), 0, s, g, (int)tm, (int)tn);
  return hipGetLastError();
}

// ---- split-K for products too small to fill the GPU (a few thousand tokens): the k range
// is split over S workgroups per output tile, each writing an fp32 partial product, and
// splitk_reduce_kernel adds the S partials in split order (one rounding per sum, the same
// order every call) and applies the epilogue.  Output columns live in up to three
// segments (the fused Q, K, V projections).
struct SplitOut {
  void* C[3];
  int32_t ldc[3];
  int32_t ncol[3];
  int32_t nseg;
};

template <int ACT, bool GATED>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* part, int S, int64_t pslice, int pld,
                                                            int64_t M, int N, SplitOut o) {
  const int cpr = N / 8;   // 8-column chunks per output row
  const int64_t total = M * cpr;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int64_t m = idx / cpr;
    const int c = (int)(idx - m * cpr) * 8;
    const float* p = part + m * pld + c;
    f32x4 u0 = *(const f32x4*)p, u1 = *(const f32x4*)(p + 4);
    f32x4 v0 = f32x4{}, v1 = f32x4{};
    if constexpr (GATED) {
      v0 = *(const f32x4*)(p + N);
      v1 = *(const f32x4*)(p + N + 4);
    }
    for (int sp = 1; sp < S; ++sp) {
      const float* q = p + sp * pslice;
      u0 += *(const f32x4*)q;
      u1 += *(const f32x4*)(q + 4);
      if constexpr (GATED) {
        v0 += *(const f32x4*)(q + N);
        v1 += *(const f32x4*)(q + N + 4);
      }
    }
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[e] = (__bf16)epilogue<ACT>(u0[e], v0[e]);
      out[4 + e] = (__bf16)epilogue<ACT>(u1[e], v1[e]);
    }
    int seg = 0, cc = c;
    if (o.nseg > 1 && cc >= o.ncol[0]) {
      cc -= o.ncol[0];
      seg = 1;
      if (o.nseg > 2 && cc >= o.ncol[1]) {
        cc -= o.ncol[1];
        seg = 2;
      }
    }
    *(bf16x8*)((__bf16*)o.C[seg] + m * o.ldc[seg] + cc) = out;
  }
}

// Split plan: output tile width (256, or 192 when every segment is a multiple of 192; the
// gated pair only 128 outputs of 256 accumulator columns) and S, chosen to fill the most
// CUs with at most one workgroup each: tiles * S <= 256, each split at least 1,024 deep,
// S <= 4.  Products with at least 192 tiles of 256 x 256 do not split.
struct SplitPlan {
  int bn;        // output columns per tile (0: no split)
  int S;
  int64_t tiles;
  int64_t pld;   // partial row length
};

SplitPlan plan_split(int64_t M, int nseg, const int32_t* segN, int64_t K, bool gated) {
  SplitPlan best{0, 1, 0, 0};
  if (M < 1024 || K < 2048) return best;
  int64_t ncols = 0;
  bool div192 = !gated;
  for (int i = 0; i < nseg; ++i) {
    ncols += segN[i];
    if (segN[i] % 192) div192 = false;
  }
  const int64_t tmr = (M + 255) / 256;
  auto tiles_for = [&](int bn) {
    int64_t t = 0;
    for (int i = 0; i < nseg; ++i) t += (segN[i] + bn - 1) / bn;
    return tmr * t;
  };
  const int64_t t_full = tiles_for(gated ? 128 : 256);
  if (t_full >= 192) return best;
  int64_t best_occ = 0;
  for (int opt = 0; opt < 2; ++opt) {
    const int bn = opt == 0 ? (gated ? 128 : 256) : 192;
    if (opt == 1 && !div192) continue;
    const int64_t t = tiles_for(bn);
    int64_t S = 256 / t;
    if (S > 4) S = 4;
    while (S > 1 && K / S < 1024) --S;
    if (S < 2) continue;
    if (t * S > best_occ) {
      best_occ = t * S;
      best = SplitPlan{bn, (int)S, t, gated ? 2 * ncols : ncols};
    }
  }
  return best;
}

template <bool DUAL, int ACT>
hipError_t launch_split(const GemmDesc& g0, const SplitPlan& pl, hipStream_t s) {
  GemmDesc g = g0;
  g.ksplit = pl.S;
  // k per split: a multiple of 64 so that every split starts on a whole k-tile
  g.kchunk = (int32_t)(((int64_t)g.K + pl.S * 64 - 1) / (pl.S * 64) * 64);
  g.pld = (int32_t)pl.pld;
  g.pslice = g.M * pl.pld;
  // 8 waves with two 64-deep stages, as the unsplit forward tiles
  hipError_t e = hipErrorInvalidValue;
  if (!DUAL && pl.bn == 192) {
    if constexpr (!DUAL) e = launch_cfg<256, 192, 64, 2, DUAL, ACT, false, kNN, false, 8>(g, s);
  } else {
    e = launch_cfg<256, 256, 64, 2, DUAL, ACT, false, kNN, false, 8>(g, s);
  }
  if (e != hipSuccess) return e;
  SplitOut o{};
  o.nseg = DUAL ? 1 : g.nseg;
  o.C[0] = g.C;
  o.ldc[0] = g.ldc;
  o.ncol[0] = g.N;
  for (int i = 0; i + 1 < o.nseg; ++i) {
    o.C[i + 1] = g.Cx[i];
    o.ldc[i + 1] = g.ldcx[i];
    o.ncol[i + 1] = g.Nx[i];
  }
  const int64_t ntot = DUAL ? g.N : pl.pld;
  const int64_t chunks = g.M * (ntot / 8);
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL((splitk_reduce_kernel<ACT, DUAL>), dim3((unsigned)blocks), dim3(256), 0, s,
                     (const float*)g.part, pl.S, g.pslice, g.pld, g.M, (int)ntot, o);
  return hipGetLastError();
}

// Tile choice.  A forward product (bf16 output, no kept pre-activations) given split-K
// scratch takes the split path when plan_split finds one.  Otherwise 256x256 tiles once they
// give at least one full wave of workgroups over the 256 CUs, on 8 waves (two 64-k stages;
// the weight-gradient (kTN) products four 32-k stages for long k-loops), with smaller tiles
// below that (the forward rules further down), else 128x128 (or 128x256 for the gated
// pair) on 4 waves.  With both operands k-contiguous (kNT) every tile row is a
// k-run in memory, and 64-k stages fetch whole 128-byte lines: measured 2-5% faster than
// 32-k stages at every depth; there a last wave of 256x256 tiles at most 3/4 full switches
// to 128x256 tiles.
template <bool DUAL, int ACT, bool OUT_F32, int LAYOUT = kNN, bool SAVE = false>
hipError_t launch_sized(const GemmDesc& g, hipStream_t s) {
  constexpr int OUT_BN = DUAL ? 128 : 256;
  if constexpr (LAYOUT == kNN && !OUT_F32 && !SAVE) {
    if (g.part) {
      int32_t segN[3] = {g.N, g.Nx[0], g.Nx[1]};
      const int nseg = DUAL ? 1 : g.nseg;
      const SplitPlan pl = plan_split(g.M, nseg, segN, g.K, DUAL);
      bool ok = pl.bn > 0;
      for (int i = 0; i < nseg && ok; ++i) ok = segN[i] % 8 == 0;
      if (ok && (size_t)pl.S * (size_t)g.M * (size_t)pl.pld * 4 <= g.part_bytes)
        return launch_split<DUAL, ACT>(g, pl, s);
    }
  }
  int64_t ncols = g.N;
  for (int i = 0; i + 1 < g.nseg && !DUAL; ++i) ncols += g.Nx[i];
  const int64_t big = ((g.M + 255) / 256) * ((ncols + OUT_BN - 1) / OUT_BN);
  const int64_t kdepth = (int64_t)g.K + (LAYOUT == kNT ? g.K2 : 0);
  if constexpr (LAYOUT == kNT) {
    if (big >= 256) {
      const int64_t last = big % 256;
      // 128x256 tiles leave LDS for a third 64-deep stage (3 x 48 KiB); measured on the 70B
      // dH product (1,792 tiles): 1,171 -> 1,089 us against two stages
      // 8 waves, as the forward tiles (70B backward, same GPU: 43.3-44.0 -> 42.2 ms per step
      // together with the TN products below; either layout alone gained less)
      if (last != 0 && last <= 192) return launch_cfg<128, 256, 64, 3, DUAL, ACT, OUT_F32, LAYOUT, SAVE, 8>(g, s);
      return launch_cfg<256, 256, 64, 2, DUAL, ACT, OUT_F32, LAYOUT, SAVE, 8>(g, s);
    }
  }
  if constexpr (LAYOUT == kNN && !DUAL) {
    // Below one full wave of 256x256 tiles, 192-column tiles can fill the CUs where 256- and
    // 128-column ones leave a quarter idle.  The GPT block's 2048 x 6144 products take 256
    // tiles of 256x192 instead of 192 of 256x256 (row GEMM 81.9 -> 76.5 us, out-projection
    // 30.9 -> 28.7 us); its 2048 x 3072 column GEMM + GELU 256 tiles of 128x192 instead of
    // 192 of 256x128 (115 -> 102 us).
    if (g.nseg == 1 && big < 256 && g.N % 192 == 0) {
      const int64_t c192 = g.N / 192;
      const int64_t t256 = ((g.M + 255) / 256) * c192, t128 = ((g.M + 127) / 128) * c192;
      if (t256 >= 224 && t256 <= 256) {
        if constexpr (!SAVE) return launch_cfg<256, 192, 64, 2, DUAL, ACT, OUT_F32, LAYOUT, SAVE, 8>(g, s);
        else if (kdepth > 2048) return launch_cfg<256, 192, 32, 4, DUAL, ACT, OUT_F32, LAYOUT, SAVE>(g, s);
        else return launch_cfg<256, 192, 64, 2, DUAL, ACT, OUT_F32, LAYOUT, SAVE>(g, s);
      }
      if (t128 >= 224 && t128 <= 256) {
        if (kdepth > 2048) return launch_cfg<128, 192, 32, 4, DUAL, ACT, OUT_F32, LAYOUT, SAVE>(g, s);
        return launch_cfg<128, 192, 64, 2, DUAL, ACT, OUT_F32, LAYOUT, SAVE>(g, s);
      }
    }
    // Forward products of a few thousand tokens (measured at 2048 x 2304..6144 x 768..6144):
    // 256x256 tiles already pay off when they occupy 3/4 of the CUs, else 256x128 tiles
    // when those occupy half of them; 128x128 only below that.
    if (big >= 192) {
      if constexpr (!SAVE) {
        if constexpr (!OUT_F32) {
          hipError_t e;
          if (launch_persistent<DUAL, ACT>(g, s, e)) return e;
        }
        return launch_cfg<256, 256, 64, 2, DUAL, ACT, OUT_F32, LAYOUT, SAVE, 8>(g, s);
      } else {
        if (kdepth > 2048) return launch_cfg<256, 256, 32, 4, DUAL, ACT, OUT_F32, LAYOUT, SAVE>(g, s);
        return launch_cfg<256, 256, 64, 2, DUAL, ACT, OUT_F32, LAYOUT, SAVE>(g, s);
      }
    }
    int64_t half = (g.N + 127) / 128;
    for (int i = 0; i + 1 < g.nseg; ++i) half += (g.Nx[i] + 127) / 128;
    const int64_t t256 = ((g.M + 255) / 256) * half;
    if (t256 >= 128) {
      // The smallest tile that still fits in one wave: the wave is the same and each tile
      // does less work.  128x128 (GPT-2-medium's 4096 x 1024 products: 128 -> 256 tiles,
      // 27 -> 22 us with GELU), else 192x128 (the GPT block's fused QKV, 2048 x 3x768:
      // 144 -> 198 tiles, 86 -> 72 us).
      if (t256 <= 256 && ((g.M + 127) / 128) * half <= 256)
        return launch_cfg<128, 128, 64, 2, DUAL, ACT, OUT_F32, LAYOUT, SAVE>(g, s);
      if (t256 <= 256 && ((g.M + 191) / 192) * half <= 256) {
        if (kdepth > 2048) return launch_cfg<192, 128, 32, 4, DUAL, ACT, OUT_F32, LAYOUT, SAVE>(g, s);
        return launch_cfg<192, 128, 64, 2, DUAL, ACT, OUT_F32, LAYOUT, SAVE>(g, s);
      }
      if (kdepth > 2048) return launch_cfg<256, 128, 32, 4, DUAL, ACT, OUT_F32, LAYOUT, SAVE>(g, s);
      return launch_cfg<256, 128, 64, 2, DUAL, ACT, OUT_F32, LAYOUT, SAVE>(g, s);
    }
  }
  if (big >= 256) {
    // Forward 256 x 256 tiles: 8 waves (two per SIMD, 128 x 64 each) with two 64-deep
    // stages.  While one wave of a SIMD is held issuing a copy the other keeps the matrix
    // pipe fed; measured alone (same operands repeated, same GPU) against 4 waves with four
    // 32-deep stages: 70B column GEMM + SwiGLU 1,440 against 1,470 us, row GEMM 735-748
    // against 754 us, out-projection 257-261 against 273 us (two 64-deep stages).
    if constexpr (LAYOUT == kNN && !SAVE) {
      if constexpr (!OUT_F32) {
        hipError_t e;
        if (launch_persistent<DUAL, ACT>(g, s, e)) return e;
      }
      return launch_cfg<256, 256, 64, 2, DUAL, ACT, OUT_F32, LAYOUT, SAVE, 8>(g, s);
    } else if constexpr (LAYOUT == kTN) {
      // the weight gradients: 8 waves with four 32-deep stages (two 64-deep ones measured
      // 2.5 % slower over the backward step)
      if (kdepth > 2048) return launch_cfg<256, 256, 32, 4, DUAL, ACT, OUT_F32, LAYOUT, SAVE, 8>(g, s);
      return launch_cfg<256, 256, 64, 2, DUAL, ACT, OUT_F32, LAYOUT, SAVE, 8>(g, s);
    } else {
      // the training forward, which also stores U (and V): 8 waves, two 64-deep stages
      // (70B column GEMM + row GEMM of one rank: 2,383-2,397 -> 2,324-2,327 us)
      return launch_cfg<256, 256, 64, 2, DUAL, ACT, OUT_F32, LAYOUT, SAVE, 8>(g, s);
    }
  }
  return launch_cfg<128, DUAL ? 256 : 128, 64, 2, DUAL, ACT, OUT_F32, LAYOUT, SAVE>(g, s);
}

}  // namespace

size_t splitk_scratch_bytes(int64_t M, int nseg, const int32_t* segN, int64_t K, bool gated) {
  const SplitPlan pl = plan_split(M, nseg, segN, K, gated);
  if (pl.bn == 0) return 0;
  return (size_t)pl.S * (size_t)M * (size_t)pl.pld * 4;
}

hipError_t launch_gemm_bf16(const GemmDesc& g, hipStream_t s) {
  if (g.out_f32) {
    if (g.act != kActNone || g.U) return hipErrorInvalidValue;
    return launch_sized<false, kActNone, true>(g, s);
  }
  if (g.U) {   // forward that also keeps U (and V) for the backward
    switch (g.act) {
      case kActGelu: return launch_sized<false, kActGelu, false, kNN, true>(g, s);
      case kActSwiglu: return launch_sized<true, kActSwiglu, false, kNN, true>(g, s);
      case kActBilinear: return launch_sized<true, kActBilinear, false, kNN, true>(g, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (g.act) {
    case kActNone: return launch_sized<false, kActNone, false>(g, s);
    case kActGelu: return launch_sized<false, kActGelu, false>(g, s);
    case kActSwiglu: return launch_sized<true, kActSwiglu, false>(g, s);
    case kActBilinear: return launch_sized<true, kActBilinear, false>(g, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_bf16_nt(const GemmDesc& g, hipStream_t s) {
  if (g.out_f32) {
    if (g.act != kActNone) return hipErrorInvalidValue;
    return launch_sized<false, kActNone, true, kNT>(g, s);
  }
  switch (g.act) {
    case kActNone: return launch_sized<false, kActNone, false, kNT>(g, s);
    case kActGelu: return launch_sized<false, kActGelu, false, kNT>(g, s);
    case kActSwiglu: return launch_sized<false, kActSwiglu, false, kNT>(g, s);
    case kActBilinear: return launch_sized<false, kActBilinear, false, kNT>(g, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_bf16_tn(const GemmDesc& g, hipStream_t s) {
  if (g.act != kActNone) return hipErrorInvalidValue;
  return g.out_f32 ? launch_sized<false, kActNone, true, kTN>(g, s)
                   : launch_sized<false, kActNone, false, kTN>(g, s);
}

}  // namespace tpk
