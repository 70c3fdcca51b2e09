// Internal interface between the C ABI (capi.hip) and the kernel files.
// Launchers enqueue on the given stream and return hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpk {

enum Act : int { kActNone = 0, kActGelu = 1, kActSwiglu = 2, kActBilinear = 3 };

// C[M, N] = epilogue(A[M, K] . B0[K, N] (, A . B1[K, N])), all row-major.
// B0/B1 point at the first element of the rank's block (offsets already applied).
// Up to two more column segments (nseg > 1, ungated activations only) extend the output
// columns: segment i multiplies the same A by Bx[i] [K, Nx[i]] into Cx[i] -- one launch
// for several products that share A (the Q, K and V projections).
struct GemmDesc {
  const void* A;
  const void* B0;
  const void* B1;  // only for the gated activations (SwiGLU, bilinear)
  void* C;
  int64_t M;
  int32_t N, K;
  int32_t lda, ldb, ldc;
  int act;
  bool out_f32;
  int32_t nseg = 1;
  const void* Bx[2] = {nullptr, nullptr};
  void* Cx[2] = {nullptr, nullptr};
  int32_t Nx[2] = {0, 0}, ldbx[2] = {0, 0}, ldcx[2] = {0, 0};
  // Second k segment (launch_gemm_bf16_nt): C = A.B0 + A2.B2, A2/B2 K2 deep with the
  // same leading dimensions (dX = dU W1^T + dV W3^T in one accumulation).
  const void* A2 = nullptr;
  const void* B2 = nullptr;
  int32_t K2 = 0;
  // Pre-activations U, V [M, N] with leading dimension ldu: the forward stores them when
  // non-null; the backward reads them and writes dU to C and dV (gated kinds) to dV.
  void* U = nullptr;
  void* V = nullptr;
  void* dV = nullptr;
  int32_t ldu = 0;
  // Split-K (forward layout, bf16 outputs, no saved pre-activations): when `part` is
  // non-null the launcher may split the k range over `ksplit` workgroups per tile; each
  // writes its fp32 partial product into part + split * pslice ([M, pld] with pld the
  // total output width, doubled for the gated pair: U columns then V columns), and a
  // second kernel sums the partials in split order and applies the epilogue.
  // part_bytes bounds what the launcher may use.
  float* part = nullptr;
  size_t part_bytes = 0;
  int32_t ksplit = 1;   // set by the launcher
  int32_t kchunk = 0;   // k per split (a multiple of the stage depth), set by the launcher
  int64_t pslice = 0;   // elements per split, set by the launcher
  int32_t pld = 0;      // partial row length, set by the launcher
};

// Split-K scratch (bytes) the forward launcher uses for a bf16 product of M rows, k depth
// K and nseg column segments of segN[i] outputs (gated: one segment, 2N accumulator
// columns): 0 when the product fills the GPU without splitting.  With K unknown, pass a
// large K: the launcher never needs more than that bound.
size_t splitk_scratch_bytes(int64_t M, int nseg, const int32_t* segN, int64_t K, bool gated);

// bf16 inputs, fp32 accumulation on MFMA; output bf16 (or fp32 if out_f32).
// A [M, K] and B [K, N], both row-major; the activation `act` in the epilogue.
hipError_t launch_gemm_bf16(const GemmDesc& g, hipStream_t s);
// A [M, K] and B given as B^T [N, K] (rows of B^T at stride ldb); with act != none the
// accumulator is dH and the epilogue applies the activation's derivative:
// C = dU (bf16), dV for the gated kinds.
hipError_t launch_gemm_bf16_nt(const GemmDesc& g, hipStream_t s);
// A given as A^T [K, M] (stride lda) and B [K, N]: C = A.B, no activation (weight
// gradients X^T dU, H^T dY).
hipError_t launch_gemm_bf16_tn(const GemmDesc& g, hipStream_t s);
// fp32 inputs and output.
hipError_t launch_gemm_f32(const GemmDesc& g, hipStream_t s);

// y = sum_t parts[t*stride + i] (+ res[i]); dtypes: 0 = f32, 1 = bf16.
hipError_t launch_partial_sum(const void* parts, int64_t stride, int T_p, const void* res,
                              void* y, int64_t n, int part_bf16, int out_bf16, hipStream_t s);

// Scaled dot-product attention of a rank's heads (see attention.hip).  Q, K, V and O
// are token-row-major; head j occupies columns [j*head_dim, (j+1)*head_dim).
struct AttnDesc {
  const __bf16* q;   // [n_seq*seq_len, ldq]
  const __bf16* k;   // [n_seq*seq_len, ldkv]
  const __bf16* v;   // [n_seq*seq_len, ldkv]
  __bf16* o;         // [n_seq*seq_len, ldo]
  int64_t n_seq;
  int32_t seq_len, head_dim, h_t, kv_t;
  int32_t ldq, ldkv, ldo;
  bool causal;
  // Causal masking by position: query row i sees key row k when k <= i + delta (delta =
  // position of the first query minus that of the first key; 0 within one sequence).
  int32_t delta;
  // Ring step (o == nullptr): fold this K/V chunk into the running state instead of
  // writing O.  o_state [n_seq*seq_len, ld_state] fp32 holds the normalised output so far,
  // lse_state [n_seq*seq_len, ld_lse] fp32 the natural log of each row's softmax
  // denominator (-inf: no key seen yet).
  float* o_state;
  float* lse_state;
  int32_t ld_state, ld_lse;
};
hipError_t launch_attention(const AttnDesc& a, hipStream_t s);
// o_state[:, :h_t*head_dim] = 0 and lse_state[:, :h_t] = -inf for `rows` rows
hipError_t launch_ring_init(float* o_state, float* lse_state, int64_t rows, int32_t cols,
                            int32_t heads, int32_t ld_state, int32_t ld_lse, hipStream_t s);
// o[:, :cols] = bf16(o_state[:, :cols]) for `rows` rows (cols a multiple of 4)
hipError_t launch_ring_finish(const float* o_state, __bf16* o, int64_t rows, int32_t cols,
                              int32_t ld_state, int32_t ldo, hipStream_t s);

}  // namespace tpk
