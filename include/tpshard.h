/*
 * tpshard.h -- C ABI of one tensor-parallel rank's share of a Megatron-style
 * transformer sublayer, on AMD Instinct MI355X (gfx950).
 *
 * What is computed (row-vector convention, everything row-major):
 *
 *   FFN sublayer, rank t of T_p ("7.9 Tensor and pipeline parallelism",
 *   section 2.1, the column-shard of W1 and row-shard of W2; the ShardedFFN
 *   listing of "Tensor & Pipeline Parallelism" (llminference S17),
 *   section "Core idea"):
 *       n      = d_ff / T_p,  cols(t) = [t*n, (t+1)*n)
 *       H(t)   = act(X . W1[:, cols(t)])                      (GELU, erf form)
 *              | silu(X . W1[:, cols(t)]) * (X . W3[:, cols(t)])   (SwiGLU)
 *       y(t)   = H(t) . W2[cols(t), :]        -- the rank's partial sum
 *   Attention output projection, rank t (same page, section 2.2;
 *   S17 "Implementation", the row shard of wo by the rank's heads):
 *       a(t)   = O(t) . Wo[rows(t), :],  rows(t) = [t*h_t*d_h, (t+1)*h_t*d_h)
 *   Head-sharded attention core (section 2.2: projections, softmax and value
 *   mixing of the rank's heads are local):
 *       O(t)   = [softmax(Q_j K_j^T / sqrt(d_h) + causal mask) V_j]_j
 *   All-reduce "g" (section 2.1: y = sum over ranks of y(t)), here the local
 *   stand-in that adds all T_p partials held on one GPU:
 *       y      = sum_{t=0}^{T_p-1} y(t)  [+ residual]
 *
 * Conventions shared by every entry point:
 *  - Weights are passed UNSHARDED (the full W1/W3 [d, d_ff], W2 [d_ff, d],
 *    Wq [d, n_heads*d_h], Wk/Wv [d, n_kv_heads*d_h], Wo [n_heads*d_h, d]);
 *    the library applies the rank's offsets.  A caller holding only its own
 *    shard passes the shard's extent with T_p = 1, t = 0.
 *  - All pointers are DEVICE pointers owned by the caller, 16-byte aligned.
 *    The library never allocates, frees or synchronises: it enqueues kernels
 *    on `hip_stream` (a hipStream_t; NULL = the default stream) and returns.
 *  - Every argument check runs on the host before any launch.  A non-zero
 *    status leaves all outputs untouched; tp_last_error() then describes it.
 *    Faults inside a kernel surface at the caller's next synchronisation.
 *  - Shapes that T_p does not divide are errors (TP_ERR_NOT_DIVISIBLE), as
 *    the pages only ever divide evenly.
 *  - Row (token) counts may be anything >= 0 (0 is a no-op).  Feature
 *    extents (d, n, h_t*d_h) must be multiples of 8 (bf16) or 4 (fp32) so
 *    every row is made of whole 16-byte vectors (TP_ERR_UNSUPPORTED).
 *  - Arithmetic: bf16 inputs are multiplied on MFMA with fp32 accumulation;
 *    the activation runs on the fp32 accumulator and H(t) is rounded once to
 *    bf16 (round-to-nearest-even).  fp32 inputs stay fp32 throughout.
 *  - Thread safety: calls may be issued from several host threads; the
 *    error message is thread-local.
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TPSHARD_ABI_VERSION 3

/* Status codes. */
#define TP_OK                 0
#define TP_ERR_INVALID_ARG   -1  /* null/misaligned pointer, negative or out-of-range size, rank >= T_p */
#define TP_ERR_NOT_DIVISIBLE -2  /* d_ff, n_heads or n_kv_heads not divisible by T_p */
#define TP_ERR_WORKSPACE     -3  /* workspace missing or smaller than the query says */
#define TP_ERR_UNSUPPORTED   -4  /* dtype / activation combination or extent not supported */
#define TP_ERR_HIP           -5  /* a HIP runtime call or kernel launch failed */

/* Activation of the column-parallel GEMM's epilogue. */
#define TP_ACT_NONE      0  /* H = U (no activation)                                */
#define TP_ACT_GELU      1  /* H = U * Phi(U) = U/2 (1 + erf(U / sqrt 2))           */
#define TP_ACT_SWIGLU    2  /* H = silu(U) * V,  U = X.W1(t), V = X.W3(t)           */
#define TP_ACT_BILINEAR  3  /* H = U * V (gate with no non-linearity)               */

/* Element types. */
#define TP_F32   0
#define TP_BF16  1

/* ABI version of the loaded library (TPSHARD_ABI_VERSION). */
int tp_abi_version(void);

/* Message of the calling thread's last non-zero status ("" if none). The
 * pointer stays valid until the thread's next call into the library. */
const char* tp_last_error(void);

/*
 * Block of `extent` owned by rank t of T_p: *begin = t*(extent/T_p),
 * *len = extent/T_p ("7.9 Tensor and pipeline parallelism", section 2.1:
 * the d_ff hidden units are divided into T_p groups, device t holds group
 * t).  Host-only integer arithmetic.  Errors: TP_ERR_INVALID_ARG (T_p < 1,
 * t outside [0, T_p), extent < 0, null outputs), TP_ERR_NOT_DIVISIBLE.
 */
int tp_shard_range(int64_t extent, int32_t T_p, int32_t t, int64_t* begin, int64_t* len);

/*
 * Bytes of device workspace for tp_ffn_shard_fwd: H(t), T * (d_ff/T_p) *
 * sizeof(element of in_dtype) rounded up to 256 bytes, followed, for bf16 products
 * too small to fill the GPU (a few thousand tokens), by scratch for the column
 * product's split-K: S fp32 partial products [S][T][d_ff/T_p] (twice as wide for
 * SWIGLU/BILINEAR), S <= 4, rounded up to 256 bytes; d is not an argument, so the
 * scratch is sized for the largest S any depth allows.  Shapes that never split
 * (e.g. 16384 tokens, or fp32) get H(t) alone.  Returns 0 for invalid arguments
 * (and for T == 0).
 */
size_t tp_ffn_workspace_bytes(int64_t T, int64_t d_ff, int32_t T_p, int32_t in_dtype);

/*
 * FFN share of rank t: y_t = act(x . W1(t) [, x . W3(t)]) . W2(t).
 *
 *   x         [T, d]      in_dtype
 *   w1, w3    [d, d_ff]   in_dtype, full matrices (w3 only for SWIGLU/BILINEAR,
 *                         must be NULL otherwise)
 *   w2        [d_ff, d]   in_dtype, full matrix
 *   y_t       [T, d]      out_dtype: the rank's partial sum (written, not accumulated)
 *   workspace             >= tp_ffn_workspace_bytes(T, d_ff, T_p, in_dtype); receives
 *                         H(t) [T, d_ff/T_p] in in_dtype (readable by the caller after
 *                         the stream reaches this point)
 *   in_dtype / out_dtype  (BF16, BF16), (BF16, F32) or (F32, F32)
 *
 * Two kernels are enqueued: the column-parallel GEMM with the activation
 * fused into its epilogue, then the row-parallel GEMM.  No communication.
 * Errors: TP_ERR_INVALID_ARG, TP_ERR_NOT_DIVISIBLE (d_ff % T_p),
 * TP_ERR_WORKSPACE, TP_ERR_UNSUPPORTED, TP_ERR_HIP.
 *
 * Workspace: at least H(t)'s bytes (TP_ERR_WORKSPACE below that).  With the
 * whole query size, a bf16 column product that cannot fill the GPU runs split
 * over k: each split writes fp32 partials into the scratch after H(t) and a
 * second kernel adds them in split order (the same order on every call, so
 * results repeat bit for bit) and applies the activation; three kernels are
 * enqueued then.  With only H(t)'s bytes the unsplit product runs.  The two
 * differ only in fp32 summation order.
 */
int tp_ffn_shard_fwd(const void* x, const void* w1, const void* w3, const void* w2,
                     void* y_t, void* workspace, size_t workspace_bytes,
                     int64_t T, int64_t d, int64_t d_ff, int32_t T_p, int32_t t,
                     int32_t act, int32_t in_dtype, int32_t out_dtype, void* hip_stream);

/*
 * tp_ffn_shard_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments without the workspace, the same two kernels, bit-identical results.
 * H(t) lives in a buffer the library itself holds on each GPU it runs on: a
 * file-scope device array of TP_NOALLOC_SCRATCH_BYTES (128 MiB), kept until the
 * process ends; its address is looked up once per device, on the first call with
 * that device current.  The call itself allocates and frees nothing.
 * The array's bytes past H(t) serve as the column product's split-K scratch
 * when they hold it (else that product runs unsplit).
 *
 *   T * (d_ff/T_p) * sizeof(element of in_dtype), rounded up to 256 bytes, must
 *   not exceed TP_NOALLOC_SCRATCH_BYTES (TP_ERR_WORKSPACE otherwise; y_t untouched).
 *
 * All calls on one GPU share that buffer, which keeps the last call's H(t): calls
 * that overlap on one GPU (other streams, other host threads) race and must be
 * ordered by the caller.  hip_stream must belong to the current device.
 * Errors: as tp_ffn_shard_fwd.
 */
#define TP_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int tp_ffn_shard_fwd_noalloc(const void* x, const void* w1, const void* w3, const void* w2,
                             void* y_t, int64_t T, int64_t d, int64_t d_ff, int32_t T_p,
                             int32_t t, int32_t act, int32_t in_dtype, int32_t out_dtype,
                             void* hip_stream);

/*
 * The two halves of tp_ffn_shard_fwd, for callers that schedule them
 * separately (e.g. to overlap the previous sublayer's exchange with the
 * column-parallel product, or to time each kernel).
 *
 * tp_ffn_column_fwd: h_t [T, d_ff/T_p] (in_dtype) = act(x . W1(t) [, x . W3(t)])
 *   -- the column-parallel GEMM with the activation fused into its epilogue
 *   ("7.9 Tensor and pipeline parallelism", section 2.1, h^(t)).
 * tp_ffn_row_fwd: y_t [T, d] (out_dtype) = h_t . W2[cols(t), :]
 *   -- the row-parallel GEMM producing the rank's partial sum (section 2.1, y^(t)).
 * Arguments mean what they mean for tp_ffn_shard_fwd; h_t is caller-owned,
 * 16-byte aligned, T*(d_ff/T_p) elements.
 */
int tp_ffn_column_fwd(const void* x, const void* w1, const void* w3, void* h_t,
                      int64_t T, int64_t d, int64_t d_ff, int32_t T_p, int32_t t,
                      int32_t act, int32_t in_dtype, void* hip_stream);
int tp_ffn_row_fwd(const void* h_t, const void* w2, void* y_t,
                   int64_t T, int64_t d, int64_t d_ff, int32_t T_p, int32_t t,
                   int32_t in_dtype, int32_t out_dtype, void* hip_stream);

/*
 * Training forward of rank t's FFN share: tp_ffn_shard_fwd in bf16 that also
 * keeps what the backward needs, in caller-owned buffers.
 *
 *   h_t       [T, n] bf16, n = d_ff/T_p: H(t), the activation output (input of W2(t))
 *   u_t       [T, n] bf16: U = x . W1(t), the pre-activation
 *   v_t       [T, n] bf16: V = x . W3(t) for SWIGLU/BILINEAR, must be NULL otherwise
 *   y_t       [T, d] out_dtype (BF16 or F32): the rank's partial sum
 * U and V are rounded once from the same fp32 accumulators the activation reads.
 * act must be GELU, SWIGLU or BILINEAR (with NONE, U is H).  Other arguments as
 * for tp_ffn_shard_fwd; inputs are bf16.
 * Errors: as tp_ffn_shard_fwd; TP_ERR_UNSUPPORTED for act NONE.
 */
int tp_ffn_shard_fwd_train(const void* x, const void* w1, const void* w3, const void* w2,
                           void* y_t, void* h_t, void* u_t, void* v_t,
                           int64_t T, int64_t d, int64_t d_ff, int32_t T_p, int32_t t,
                           int32_t act, int32_t out_dtype, void* hip_stream);

/*
 * Backward of rank t's out-projection a(t) = O(t) . Wo[rows(t), :]
 * ("7.9 Tensor and pipeline parallelism", section 2.2, with the f-g pattern of
 * section 2.1: the sum over ranks passes dY unchanged to every rank).
 *
 *   o_t   [T, h_t*head_dim] bf16: rank t's head outputs (the forward's input)
 *   wo    [n_heads*head_dim, d] bf16, full matrix
 *   dy    [T, d] bf16: dL/da for the summed output
 *   do_t  [T, h_t*head_dim] bf16: dO(t) = dY Wo(t)^T, the gradient of rank t's heads
 *         (no sum over ranks: each rank's heads are its own)
 *   dwo   [n_heads*head_dim, d] grad_dtype (BF16/F32): rows of rank t's heads
 *         := O(t)^T dY (overwritten; other rows untouched; zero when T = 0)
 * Divisibility and shape rules as tp_attn_outproj_shard_fwd.  Two kernels.
 * Errors: TP_ERR_INVALID_ARG, TP_ERR_NOT_DIVISIBLE, TP_ERR_UNSUPPORTED, TP_ERR_HIP.
 */
int tp_attn_outproj_shard_bwd(const void* o_t, const void* wo, const void* dy, void* do_t,
                              void* dwo, int64_t T, int64_t d, int32_t n_heads,
                              int32_t n_kv_heads, int32_t head_dim, int32_t T_p, int32_t t,
                              int32_t grad_dtype, void* hip_stream);

/* Workspace of tp_ffn_shard_bwd: dU (and dV for the gated kinds), bf16 [T, n]
 * each, every plane rounded up to 256 bytes.  0 for invalid arguments. */
size_t tp_ffn_bwd_workspace_bytes(int64_t T, int64_t d_ff, int32_t T_p, int32_t act);

/*
 * Backward of rank t's FFN share ("7.9 Tensor and pipeline parallelism",
 * section 2.1, the f-g pattern: g, the all-reduce after the row shard, is the
 * identity backward, so every rank receives the whole dY; f, the identity
 * before the column shard, all-reduces the ranks' input gradients).
 *
 *   dy        [T, d] bf16: dL/dy for the full sublayer output
 *   x, w1, w3, w2        as for the forward (full matrices, bf16)
 *   h_t, u_t, v_t        what tp_ffn_shard_fwd_train kept (u_t unused and may be
 *                        NULL for act NONE; v_t only for SWIGLU/BILINEAR)
 *   dx_t      [T, d] dx_dtype (BF16/F32): this rank's partial input gradient
 *             dX(t) = dU W1(t)^T [+ dV W3(t)^T]; tp_partial_sum over the ranks
 *             gives dX (the f all-reduce)
 *   dw2       [d_ff, d] grad_dtype (BF16/F32): rows cols(t) := H(t)^T dY
 *   dw1, dw3  [d, d_ff] grad_dtype: columns cols(t) := X^T dU, X^T dV (dw3 only
 *             for SWIGLU/BILINEAR, NULL otherwise)
 *   workspace >= tp_ffn_bwd_workspace_bytes(T, d_ff, T_p, act); receives dU [, dV]
 * with dH = dY W2(t)^T and (dU, dV) its image through the activation's
 * derivative: GELU dU = dH gelu'(U); SWIGLU dU = dH V silu'(U), dV = dH silu(U);
 * BILINEAR dU = dH V, dV = dH U; NONE dU = dH.
 * The weight-gradient blocks are overwritten (not accumulated); entries outside
 * rank t's blocks are not touched.  With T = 0 the blocks are set to zero.
 * Four kernels are enqueued (dU, dW2, dX, dW1 [+ dW3 in the same launch]).
 * Errors: TP_ERR_INVALID_ARG, TP_ERR_NOT_DIVISIBLE, TP_ERR_WORKSPACE,
 * TP_ERR_UNSUPPORTED (dtype, shapes not multiples of 8), TP_ERR_HIP.
 */
int tp_ffn_shard_bwd(const void* x, const void* w1, const void* w3, const void* w2,
                     const void* dy, const void* h_t, const void* u_t, const void* v_t,
                     void* dx_t, void* dw1, void* dw3, void* dw2,
                     void* workspace, size_t workspace_bytes,
                     int64_t T, int64_t d, int64_t d_ff, int32_t T_p, int32_t t, int32_t act,
                     int32_t dx_dtype, int32_t grad_dtype, void* hip_stream);

/*
 * Row-sharded attention output projection of rank t: y_t = o_t . Wo[rows(t), :].
 *
 *   o_t   [T, h_t*head_dim]         in_dtype, the rank's heads' outputs, contiguous
 *   wo    [n_heads*head_dim, d]     in_dtype, full matrix
 *   y_t   [T, d]                    out_dtype, the rank's partial sum
 * h_t = n_heads / T_p.  Both n_heads and n_kv_heads must be divisible by T_p
 * (the GQA constraint of S17, "Attention shards by head, and GQA caps the
 * degree"): otherwise TP_ERR_NOT_DIVISIBLE and nothing is launched.
 */
int tp_attn_outproj_shard_fwd(const void* o_t, const void* wo, void* y_t,
                              int64_t T, int64_t d, int32_t n_heads, int32_t n_kv_heads,
                              int32_t head_dim, int32_t T_p, int32_t t,
                              int32_t in_dtype, int32_t out_dtype, void* hip_stream);

/*
 * Bytes of device workspace for tp_attn_heads_shard_fwd: the rank's Q, K and V,
 * n_seq*seq_len * (h_t + 2*kv_t) * head_dim * 2 rounded up to 256, followed, when
 * the fused Q/K/V product is too small to fill the GPU, by split-K scratch: S fp32
 * partials [S][n_seq*seq_len][(h_t + 2*kv_t)*head_dim], S <= 4, rounded up to 256.
 * tp_attn_heads_shard_fwd accepts any workspace of at least the Q, K, V bytes and
 * splits only when the scratch fits (as tp_ffn_shard_fwd).  Returns 0 for invalid
 * arguments.
 */
size_t tp_attn_heads_workspace_bytes(int64_t n_seq, int64_t seq_len, int32_t n_heads,
                                     int32_t n_kv_heads, int32_t head_dim, int32_t T_p);

/*
 * Head-sharded attention of rank t (bf16 only): for each of the rank's h_t
 * query heads j (global head t*h_t + j) and its KV head (grouped-query: local
 * KV head j / (h_t/kv_t)):
 *     Q_j = x . Wq[:, head cols],  K_j = x . Wk[:, kv cols],  V_j = x . Wv[:, kv cols]
 *     O_j = softmax(Q_j K_j^T / sqrt(head_dim) [+ causal mask: key <= query]) V_j
 * independently for each of the n_seq sequences of seq_len tokens in x.
 *
 *   x          [n_seq*seq_len, d]            bf16
 *   wq         [d, n_heads*head_dim]         bf16, full
 *   wk, wv     [d, n_kv_heads*head_dim]      bf16, full
 *   o_t        [n_seq*seq_len, h_t*head_dim] bf16, head j in columns [j*head_dim, (j+1)*head_dim)
 *   workspace  >= tp_attn_heads_workspace_bytes(...)
 * head_dim must be 64 or 128.  causal: 1 = causal mask, 0 = none.
 */
int tp_attn_heads_shard_fwd(const void* x, const void* wq, const void* wk, const void* wv,
                            void* o_t, void* workspace, size_t workspace_bytes,
                            int64_t n_seq, int64_t seq_len, int64_t d,
                            int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                            int32_t T_p, int32_t t, int32_t causal, void* hip_stream);

/*
 * tp_attn_heads_shard_fwd for tensor-parallel degrees above the KV head count
 * (grouped-query attention): "Tensor & Pipeline Parallelism" (S17), "Attention
 * shards by head, and GQA caps the degree" -- TP16 with 8 KV heads needs KV heads
 * replicated across ranks.  When T_p is a multiple of n_kv_heads, each KV head
 * serves T_p / n_kv_heads consecutive ranks: rank t projects and uses KV head
 * t / (T_p / n_kv_heads) for all of its h_t = n_heads / T_p query heads.  When T_p
 * divides n_kv_heads this is exactly tp_attn_heads_shard_fwd.  Same arguments;
 * workspace >= tp_attn_heads_kvrep_workspace_bytes(...).
 * Errors: as tp_attn_heads_shard_fwd; TP_ERR_NOT_DIVISIBLE when neither T_p divides
 * n_kv_heads nor n_kv_heads divides T_p.
 */
int tp_attn_heads_shard_fwd_kvrep(const void* x, const void* wq, const void* wk, const void* wv,
                                  void* o_t, void* workspace, size_t workspace_bytes,
                                  int64_t n_seq, int64_t seq_len, int64_t d,
                                  int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                  int32_t T_p, int32_t t, int32_t causal, void* hip_stream);

/* Workspace of tp_attn_heads_shard_fwd_kvrep: Q of the h_t query heads, K and V of the
 * rank's KV heads (one when replicated), n_seq*seq_len rows, bf16, rounded up to 256,
 * then split-K scratch as for tp_attn_heads_workspace_bytes when the product splits.
 * 0 for invalid arguments. */
size_t tp_attn_heads_kvrep_workspace_bytes(int64_t n_seq, int64_t seq_len, int32_t n_heads,
                                           int32_t n_kv_heads, int32_t head_dim, int32_t T_p);

/*
 * The attention core alone (the second half of tp_attn_heads_shard_fwd), on the rank's
 * already-projected heads: for each local query head j and sequence s,
 *     O_j = softmax(Q_j K_kv(j)^T / sqrt(head_dim) [+ causal mask]) V_kv(j),
 * kv(j) = j / (h_t / kv_t).  bf16 in and out, fp32 softmax statistics.
 *
 *   q      [n_seq*seq_len, ldq]   head j in columns [j*head_dim, (j+1)*head_dim), ldq >= h_t*head_dim
 *   k, v   [n_seq*seq_len, ldkv]  KV head i in columns [i*head_dim, ...), ldkv >= kv_t*head_dim
 *   o      [n_seq*seq_len, ldo]   written like q
 * h_t % kv_t must be 0; head_dim 64 or 128; leading dimensions multiples of 8.
 */
int tp_attn_core_fwd(const void* q, const void* k, const void* v, void* o,
                     int64_t n_seq, int64_t seq_len, int32_t h_t, int32_t kv_t,
                     int32_t head_dim, int64_t ldq, int64_t ldkv, int64_t ldo,
                     int32_t causal, void* hip_stream);

/*
 * Context parallelism (ring attention): "7.9 Tensor and pipeline parallelism",
 * section 6; "Parallelism II: model", "Sequence and context parallelism"; and
 * "Tensor & Pipeline Parallelism" (S17), which names passing the FlashAttention
 * running state round a ring.  The sequence is split into chunks over the ranks of
 * a context-parallel group; each rank keeps its query chunk and folds in the K/V
 * chunks one at a time as they come round.  These three calls are one rank's
 * share: set up the running state, fold one K/V chunk into it, and turn it into O.
 *
 * The running state of each query row r and local head j:
 *   o_state[r, j*head_dim + c]  fp32, the softmax-weighted mean of the values of
 *                               the keys folded in so far (0 before the first);
 *   lse_state[r, j]             fp32, ln of the row's softmax denominator over
 *                               those keys, sum_k exp(q.k / sqrt(head_dim))
 *                               (-inf before the first).
 * Folding chunk c into (O, lse) with the chunk's own (O_c, lse_c):
 *   lse' = ln(e^lse + e^lse_c),  O' = e^(lse - lse') O + e^(lse_c - lse') O_c.
 * Any order of chunks gives the same result up to rounding; after all of them O is
 * softmax(Q K^T / sqrt(head_dim) [+ causal mask]) V over the whole sequence.
 *
 * tp_attn_ring_init: o_state[:, :h_t*head_dim] = 0, lse_state[:, :h_t] = -inf for
 *   `rows` rows.  o_state 16-byte aligned, ld_state >= h_t*head_dim and a multiple
 *   of 4; ld_lse >= h_t.
 */
int tp_attn_ring_init(void* o_state, void* lse_state, int64_t rows, int32_t h_t,
                      int32_t head_dim, int64_t ld_state, int64_t ld_lse, void* hip_stream);

/*
 * tp_attn_ring_step: fold one K/V chunk into the running state of this rank's query
 * chunk.  q, k, v as for tp_attn_core_fwd (n_seq sequences of seq_len rows each;
 * every sequence is split the same way, so the query and key chunks have the same
 * length).  q_pos0 / k_pos0: the position in the sequence of the chunks' first rows.
 * Causal: query row i (position q_pos0 + i) sees key row k (position k_pos0 + k)
 * when k_pos0 + k <= q_pos0 + i.  A query row that sees no key of this chunk keeps
 * its state bit for bit, and a chunk that lies wholly after the query chunk is a
 * no-op (nothing is launched).  The state is read and written in place (rows
 * [0, n_seq*seq_len)); it must not overlap q, k or v.
 * Errors: as tp_attn_core_fwd; TP_ERR_INVALID_ARG for negative positions or
 * |q_pos0 - k_pos0| >= 2^30, or a misaligned / too narrow state.
 */
int tp_attn_ring_step(const void* q, const void* k, const void* v, void* o_state,
                      void* lse_state, int64_t n_seq, int64_t seq_len, int32_t h_t,
                      int32_t kv_t, int32_t head_dim, int64_t ldq, int64_t ldkv,
                      int64_t ld_state, int64_t ld_lse, int64_t q_pos0, int64_t k_pos0,
                      int32_t causal, void* hip_stream);

/*
 * tp_attn_ring_finish: o[:, :h_t*head_dim] = bf16(o_state[:, :h_t*head_dim]), round
 * to nearest even, for `rows` rows.  ldo >= h_t*head_dim, a multiple of 4; o 16-byte
 * aligned and not overlapping the state.  After every chunk has been folded in, o
 * equals what tp_attn_core_fwd writes for the whole sequence (up to rounding; with a
 * single chunk, bit for bit).
 */
int tp_attn_ring_finish(const void* o_state, void* o, int64_t rows, int32_t h_t,
                        int32_t head_dim, int64_t ld_state, int64_t ldo, void* hip_stream);

/*
 * Local partial sum standing in for the all-reduce ("7.9 Tensor and
 * pipeline parallelism", section 2.1: y is the sum over ranks of y(t)):
 *     y[i] = sum_{t=0}^{T_p-1} partials[t*partial_stride + i]  (+ residual[i])
 * accumulated in fp32 in ascending t, residual added last, rounded once to
 * out_dtype.  The order is fixed, so repeated calls are bitwise identical.
 *
 *   partials        T_p slices of n_elems elements, part_dtype, slice t at
 *                   offset t*partial_stride elements (partial_stride >= n_elems,
 *                   a multiple of 8 when T_p > 1).  A stride that is a large power
 *                   of two maps the same element of every slice onto the same DRAM
 *                   banks; padding it by a few KiB streams measurably faster.
 *   residual        NULL or [n_elems] out_dtype; may equal y (in place)
 *   y               [n_elems] out_dtype; must not overlap the partials
 * Supported: part_dtype and out_dtype each BF16 or F32.  n_elems == 0 is a no-op.
 */
int tp_partial_sum(const void* partials, int64_t partial_stride, int32_t T_p,
                   const void* residual, void* y, int64_t n_elems,
                   int32_t part_dtype, int32_t out_dtype, void* hip_stream);

/*
 * Sequence-parallel form of the sum ("7.9 Tensor and pipeline parallelism",
 * section 2.5; "Parallelism II: model", "Sequence and context parallelism"):
 * the all-reduce after the row shard becomes a reduce-scatter in which rank t
 * keeps token rows [t*T/T_p, (t+1)*T/T_p) of y = sum_s y(s) (+ residual).
 *
 *   partials       T_p slices [T, d] at partial_stride elements (>= T*d), part_dtype
 *   t              the rank whose rows are produced
 *   residual       [T/T_p, d] out_dtype: rank t's rows of the residual stream (sharded
 *                  by rows as well), or NULL; may equal y_rows
 *   y_rows         [T/T_p, d] out_dtype: rank t's rows of the sum
 * T_p must divide T (TP_ERR_NOT_DIVISIBLE) and d must be a multiple of 8.
 * The values equal rows [t*T/T_p, ...) of tp_partial_sum over the same inputs bit
 * for bit (same kernel, same ascending order).  The all-gather that follows, every
 * rank's rows into the [T, d] input of the next column GEMM, is a placement on one
 * GPU: pass y_rows = y + t*(T/T_p)*d.  Errors: as tp_partial_sum, plus the above.
 */
int tp_reduce_scatter_rows(const void* partials, int64_t partial_stride, int32_t T_p, int32_t t,
                           const void* residual, void* y_rows, int64_t T, int64_t d,
                           int32_t part_dtype, int32_t out_dtype, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* TPSHARD_H */
