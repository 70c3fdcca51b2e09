"""Float64 oracle of the tensor-parallel FFN and attention sublayer shards.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain definitions,
written out step by step; numpy.matmul serves as the matrix product.

Conventions (the row-vector form used by the code on "Tensor & Pipeline
Parallelism" (llminference, S17), section "Core idea": ``x @ w1``):
    X [T, d], W1/W3 [d, d_ff], W2 [d_ff, d], Wq [d, n_heads*d_h],
    Wk/Wv [d, n_kv_heads*d_h], Wo [n_heads*d_h, d]; everything row-major.
The column-vector form of "7.9 Tensor and pipeline parallelism" section 2.1
(y = W2 sigma(W1 x), W1 in R^{d_ff x d}) is the transpose of this and shards
the same d_ff hidden units.
"""
from __future__ import annotations

import math

import numpy as np
from scipy import special as _sp

ACTS = ("none", "gelu", "swiglu", "bilinear")


# ----------------------------------------------------------------------------- shards
def shard_range(extent: int, T_p: int, t: int) -> tuple[int, int]:
    """Block of ``extent`` owned by rank t of T_p: (begin, length).

    "7.9 Tensor and pipeline parallelism" section 2.1: the d_ff hidden units
    are divided into T_p groups and device t holds group t.  An extent that
    T_p does not divide is an error (the pages only divide evenly).
    """
    if T_p < 1 or not (0 <= t < T_p):
        raise ValueError(f"rank {t} out of range for T_p={T_p}")
    if extent < 0:
        raise ValueError("negative extent")
    if extent % T_p:
        raise ValueError(f"extent {extent} not divisible by T_p={T_p}")
    n = extent // T_p
    return t * n, n


def head_shard(n_heads: int, n_kv_heads: int, head_dim: int, T_p: int, t: int) -> dict:
    """Heads owned by rank t, and the column (Wq/Wk/Wv) / row (Wo) blocks they index.

    "7.9 Tensor and pipeline parallelism" section 2.2 (device t owns h/T_p
    heads) and the ShardedAttention listing on "Tensor & Pipeline
    Parallelism" (llminference, S17), section "Implementation": T_p must
    divide both the query-head and the KV-head counts.
    """
    if n_heads % T_p:
        raise ValueError(f"n_heads={n_heads} is not a multiple of T_p={T_p}")
    if n_kv_heads % T_p:
        raise ValueError(f"n_kv_heads={n_kv_heads} is not a multiple of T_p={T_p}")
    h_t = n_heads // T_p
    kv_t = n_kv_heads // T_p
    return {
        "h_t": h_t,
        "kv_t": kv_t,
        "q_cols": (t * h_t * head_dim, (t + 1) * h_t * head_dim),
        "kv_cols": (t * kv_t * head_dim, (t + 1) * kv_t * head_dim),
        "o_rows": (t * h_t * head_dim, (t + 1) * h_t * head_dim),
    }


def head_shard_kv_replicated(n_heads: int, n_kv_heads: int, head_dim: int, T_p: int, t: int) -> dict:
    """Head shard of rank t when T_p exceeds the KV heads: the KV heads are replicated.

    "Tensor & Pipeline Parallelism" (S17), "Attention shards by head, and GQA
    caps the degree": with fewer KV heads than ranks the degree only works if
    KV heads are replicated across ranks.  With T_p a multiple of n_kv_heads,
    each KV head serves T_p / n_kv_heads consecutive ranks, and all h_t query
    heads of rank t share KV head t // (T_p / n_kv_heads).  When T_p divides
    n_kv_heads nothing is replicated and this is head_shard.
    """
    if n_kv_heads % T_p == 0:
        return head_shard(n_heads, n_kv_heads, head_dim, T_p, t)
    if n_heads % T_p:
        raise ValueError(f"n_heads={n_heads} is not a multiple of T_p={T_p}")
    if T_p % n_kv_heads or n_heads % n_kv_heads:
        raise ValueError(f"TP{T_p} cannot replicate {n_kv_heads} KV heads evenly")
    if not (0 <= t < T_p):
        raise ValueError(f"rank {t} out of range for T_p={T_p}")
    h_t = n_heads // T_p
    kv = t // (T_p // n_kv_heads)
    return {
        "h_t": h_t,
        "kv_t": 1,
        "q_cols": (t * h_t * head_dim, (t + 1) * h_t * head_dim),
        "kv_cols": (kv * head_dim, (kv + 1) * head_dim),
        "o_rows": (t * h_t * head_dim, (t + 1) * h_t * head_dim),
    }


# ----------------------------------------------------------------------------- activations
def gelu(u: np.ndarray) -> np.ndarray:
    """GELU, erf form: u * Phi(u) = u/2 * (1 + erf(u / sqrt 2)) = u/2 * erfc(-u / sqrt 2).

    The pages name GeLU/GELU without a formula ("Tensor and Pipeline
    Parallelism" lesson on grasp.study, "A Tale of Two GEMMs"; "Parallelism II:
    model", "Tensor parallelism"); the exact (erf) form is taken.  It is
    evaluated through erfc so that the far negative tail keeps its relative
    accuracy (1 + erf cancels there).
    """
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * u * _sp.erfc(-u / math.sqrt(2.0))


def silu(u: np.ndarray) -> np.ndarray:
    """silu(u) = u / (1 + exp(-u)), as used by the ShardedFFN listing (S17, "Core idea")."""
    u = np.asarray(u, dtype=np.float64)
    return u / (1.0 + np.exp(-u))


# ----------------------------------------------------------------------------- FFN
def column_parallel(x, w1, w3, cols: tuple[int, int], act: str) -> np.ndarray:
    """H(t) = sigma(X . W1[:, cols]) -- or silu(X.W1[:,cols]) * (X.W3[:,cols]).

    "7.9 ..." section 2.1 eq. for h^(t): x is the same on every device and
    the element-wise non-linearity is applied to the rank's hidden slice with
    no communication.  S17 "Core idea": h = silu(x @ w1) * (x @ w3) with W1
    and W3 split on their output dimension.  "bilinear" is the gate with no
    non-linearity, U * V; "none" returns U (both used for exact tests).
    """
    if act not in ACTS:
        raise ValueError(act)
    b, e = cols
    x = np.asarray(x, dtype=np.float64)
    u = x @ np.asarray(w1[:, b:e], dtype=np.float64)
    if act == "none":
        return u
    if act == "gelu":
        return gelu(u)
    v = x @ np.asarray(w3[:, b:e], dtype=np.float64)
    if act == "swiglu":
        return silu(u) * v
    return u * v


def row_parallel(h, w2, rows: tuple[int, int]) -> np.ndarray:
    """y(t) = H(t) . W2[rows, :] -- the rank's partial sum of the output.

    "7.9 ..." section 2.1 eq. for y^(t) (row shard of W2 over the same
    groups); S17 "Core idea": y = h @ w2 is a PARTIAL sum.
    """
    b, e = rows
    return np.asarray(h, dtype=np.float64) @ np.asarray(w2[b:e, :], dtype=np.float64)


def ffn_shard(x, w1, w3, w2, T_p: int, t: int, act: str):
    """Rank t's FFN share: returns (H(t), y(t))."""
    d_ff = w1.shape[1]
    b, n = shard_range(d_ff, T_p, t)
    h = column_parallel(x, w1, w3, (b, b + n), act)
    return h, row_parallel(h, w2, (b, b + n))


def ffn_unsharded(x, w1, w3, w2, act: str) -> np.ndarray:
    """The full sublayer y = sigma(X W1) W2 (or (silu(XW1) * XW3) W2), no sharding."""
    h = column_parallel(x, w1, w3, (0, w1.shape[1]), act)
    return row_parallel(h, w2, (0, w2.shape[0]))


# ----------------------------------------------------------------------------- FFN backward
def gelu_grad(u: np.ndarray) -> np.ndarray:
    """d/du of u * Phi(u): Phi(u) + u * phi(u), phi the standard normal density."""
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * _sp.erfc(-u / math.sqrt(2.0)) + u * np.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)


def silu_grad(u: np.ndarray) -> np.ndarray:
    """d/du of u * s(u), s the logistic function: s(u) * (1 + u * (1 - s(u)))."""
    u = np.asarray(u, dtype=np.float64)
    s = 1.0 / (1.0 + np.exp(-u))
    return s * (1.0 + u * (1.0 - s))


def act_backward(dh, u, v, act: str):
    """(dU, dV) from dH and the saved pre-activations U = X W1(t), V = X W3(t).

    The chain rule through the element-wise activation of the column shard:
    gelu: dU = dH * gelu'(U); swiglu (H = silu(U) * V): dU = dH * V * silu'(U),
    dV = dH * silu(U); bilinear (H = U * V): dU = dH * V, dV = dH * U; none: dU = dH.
    dV is None for the ungated kinds.
    """
    dh = np.asarray(dh, dtype=np.float64)
    if act == "none":
        return dh, None
    if act == "gelu":
        return dh * gelu_grad(u), None
    if act == "swiglu":
        return dh * v * silu_grad(u), dh * silu(u)
    if act == "bilinear":
        return dh * v, dh * u
    raise ValueError(act)


def ffn_shard_bwd(x, w1, w3, w2, dy, T_p: int, t: int, act: str) -> dict:
    """Rank t's share of the FFN backward, given dY = dL/dy for the full output y.

    "7.9 Tensor and pipeline parallelism" section 2.1 (the f-g pattern): g, the
    all-reduce after the row shard, is the identity going backward, so every
    rank receives the whole dY; f, the identity before the column shard, becomes
    an all-reduce, so rank t's input gradient dX(t) is a partial sum and
    dX = sum_t dX(t).  The weight gradients of a rank touch only its own blocks.
    With U = X W1(t), V = X W3(t), H = sigma(U[, V]) and y(t) = H W2(t):
        dH = dY W2(t)^T          dW2(t) = H^T dY          (rows cols(t) of dW2)
        (dU, dV) = act_backward(dH, U, V)
        dX(t) = dU W1(t)^T [+ dV W3(t)^T]
        dW1(t) = X^T dU [, dW3(t) = X^T dV]             (columns cols(t))
    Returns every intermediate: u, v, h, dh, du, dv, dx_t, dw1, dw3, dw2.
    """
    d_ff = w1.shape[1]
    b, n = shard_range(d_ff, T_p, t)
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    w1c = np.asarray(w1[:, b:b + n], dtype=np.float64)
    w2r = np.asarray(w2[b:b + n, :], dtype=np.float64)
    gated = act in ("swiglu", "bilinear")
    w3c = np.asarray(w3[:, b:b + n], dtype=np.float64) if gated else None
    u = x @ w1c
    v = x @ w3c if gated else None
    h = column_parallel(x, w1, w3, (b, b + n), act)
    dh = dy @ w2r.T
    dw2 = h.T @ dy
    du, dv = act_backward(dh, u, v, act)
    dx_t = du @ w1c.T
    if gated:
        dx_t = dx_t + dv @ w3c.T
    return {"u": u, "v": v, "h": h, "dh": dh, "du": du, "dv": dv, "dx_t": dx_t,
            "dw1": x.T @ du, "dw3": x.T @ dv if gated else None, "dw2": dw2}


def partial_sum(parts, residual=None) -> np.ndarray:
    """y = sum_t y(t) [+ residual] -- what the all-reduce g computes.

    "7.9 ..." section 2.1: the full output is the sum over devices of the
    partial sums; one all-reduce at the end of the FFN gives every device y.
    Summed in ascending t; the residual (used by the block) is added last.
    """
    acc = np.zeros_like(np.asarray(parts[0], dtype=np.float64))
    for p in parts:
        acc = acc + np.asarray(p, dtype=np.float64)
    if residual is not None:
        acc = acc + np.asarray(residual, dtype=np.float64)
    return acc


# ----------------------------------------------------------------------------- attention
def reduce_scatter_rows(parts, T_p: int, t: int, residual_rows=None) -> np.ndarray:
    """Rank t's token rows of the sum, the sequence-parallel reduce-scatter.

    "7.9 Tensor and pipeline parallelism" section 2.5 and "Parallelism II:
    model", "Sequence and context parallelism": the all-reduce after the row
    shard becomes a reduce-scatter over the sequence, rank t keeping rows
    [t*T/T_p, (t+1)*T/T_p) (T_p must divide T), with its rows of the residual
    stream added; an all-gather restores the full rows for the next column shard.
    """
    parts = [np.asarray(p_, dtype=np.float64) for p_ in parts]
    T = parts[0].shape[0]
    b, m = shard_range(T, T_p, t)
    acc = np.zeros_like(parts[0][b:b + m])
    for p_ in parts:
        acc = acc + p_[b:b + m]
    return acc if residual_rows is None else acc + np.asarray(residual_rows, dtype=np.float64)


def attn_outproj_shard(o_t, wo, n_heads: int, n_kv_heads: int, head_dim: int, T_p: int,
                       t: int) -> np.ndarray:
    """a(t) = O(t) . Wo[rows(t), :] -- row-sharded output projection.

    "7.9 ..." section 2.2 eq. attn-out^(t) = W_O^(t) head-output^(t), then an
    all-reduce; S17 "Implementation": ``self.wo = w.wo[h, :]`` (row shard by
    the rank's heads).
    """
    hs = head_shard(n_heads, n_kv_heads, head_dim, T_p, t)
    b, e = hs["o_rows"]
    o_t = np.asarray(o_t, dtype=np.float64)
    if o_t.shape[1] != e - b:
        raise ValueError("O(t) width must be h_t * head_dim")
    return o_t @ np.asarray(wo[b:e, :], dtype=np.float64)


def attn_outproj_shard_bwd(o_t, wo, dy, n_heads: int, n_kv_heads: int, head_dim: int, T_p: int,
                           t: int) -> dict:
    """Backward of the row-sharded out-projection a(t) = O(t) . Wo[rows(t), :].

    The same f-g pattern as the FFN ("7.9 ..." section 2.2 with 2.1): the sum
    over ranks (g) passes dY unchanged to every rank; O(t) holds only rank t's
    heads, so its gradient dO(t) = dY Wo(t)^T stays on the rank, and dWo(t) =
    O(t)^T dY is rank t's block of rows of dWo.
    """
    hs = head_shard(n_heads, n_kv_heads, head_dim, T_p, t)
    b, e = hs["o_rows"]
    o_t = np.asarray(o_t, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    wr = np.asarray(wo[b:e, :], dtype=np.float64)
    return {"do_t": dy @ wr.T, "dwo": o_t.T @ dy}


def attention_head(q, k, v, causal: bool = True, rows=None) -> np.ndarray:
    """softmax(Q K^T / sqrt(d_h) [+ causal mask]) V for one head.

    Scaled dot-product attention, computed per head with no communication
    ("7.9 ..." section 2.2: Q, K, V projections, softmax and value mixing are
    local to the device owning the head).  Causal: query i sees keys k <= i.
    ``rows`` restricts the computed query rows (q is then the full Q, and only
    those rows are returned).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, dh = q.shape
    idx = np.arange(T) if rows is None else np.asarray(rows)
    s = (q[idx] @ k.T) / math.sqrt(dh)
    if causal:
        mask = np.arange(k.shape[0])[None, :] > idx[:, None]
        s = np.where(mask, -np.inf, s)
    s = s - np.max(s, axis=1, keepdims=True)
    p = np.exp(s)
    p = p / np.sum(p, axis=1, keepdims=True)
    return p @ v


def ring_attention_step(q, k, v, o_state, lse_state, q_pos0: int, k_pos0: int,
                        causal: bool = True):
    """Fold one K/V chunk into the running attention state of a query chunk (one head).

    Context parallelism ("7.9 Tensor and pipeline parallelism" section 6; "Parallelism
    II: model", "Sequence and context parallelism"; "Tensor & Pipeline Parallelism" (S17),
    which passes the FlashAttention running state round a ring): the sequence is split
    into chunks over the devices, each keeps its own queries and takes in every chunk's
    keys and values in turn.  The running state of a query row is (O, lse): O the
    softmax-weighted mean of the values of the keys seen so far, lse the natural log of
    the softmax denominator over them (-inf and 0 before any key).  Positions: query row
    i is at q_pos0 + i, key row k at k_pos0 + k; causal lets a query see keys at or
    before its own position.  Returns the new (O, lse); rows that see no key of this
    chunk keep their state unchanged.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    o_state = np.asarray(o_state, dtype=np.float64)
    lse_state = np.asarray(lse_state, dtype=np.float64)
    dh = q.shape[1]
    s = (q @ k.T) / math.sqrt(dh)
    if causal:
        qpos = q_pos0 + np.arange(q.shape[0])
        kpos = k_pos0 + np.arange(k.shape[0])
        s = np.where(kpos[None, :] > qpos[:, None], -np.inf, s)
    seen = np.isfinite(s).any(axis=1)
    # this chunk's own softmax over its visible keys
    m = np.where(seen, np.max(np.where(np.isfinite(s), s, -np.inf), axis=1), 0.0)
    e = np.exp(s - m[:, None])                 # exp(-inf) = 0 for masked keys
    den = e.sum(axis=1)
    lse_c = np.where(seen, m + np.log(np.where(seen, den, 1.0)), -np.inf)
    o_c = (e @ v) / np.where(seen, den, 1.0)[:, None]
    # merge: lse' = ln(e^lse + e^lse_c), O' = e^(lse - lse') O + e^(lse_c - lse') O_c
    big = np.maximum(lse_state, lse_c)
    big_f = np.where(np.isfinite(big), big, 0.0)
    w_old = np.exp(lse_state - big_f)
    w_new = np.exp(lse_c - big_f)
    lse_new = big_f + np.log(np.where(seen, w_old + w_new, 1.0))
    o_new = (w_old[:, None] * o_state + w_new[:, None] * o_c) / np.where(seen, w_old + w_new, 1.0)[:, None]
    return np.where(seen[:, None], o_new, o_state), np.where(seen, lse_new, lse_state)


def attn_heads_shard(x, wq, wk, wv, n_heads: int, n_kv_heads: int, head_dim: int, T_p: int,
                     t: int, causal: bool = True, rows=None, kv_replicate: bool = False) -> np.ndarray:
    """O(t): the rank's heads' outputs concatenated, [T (or len(rows)), h_t*head_dim].

    Column shards of Wq (and of Wk/Wv by KV head) by head, per S17
    "Implementation" (``w.wq[:, h]``, KV sharded by KV head); local query head
    j of rank t reads KV head j // (h_t / kv_t) of that rank (grouped-query
    attention; with n_kv_heads == n_heads this is ordinary multi-head
    attention).  kv_replicate takes head_shard_kv_replicated's blocks.
    """
    hs = (head_shard_kv_replicated if kv_replicate else head_shard)(n_heads, n_kv_heads, head_dim, T_p, t)
    x = np.asarray(x, dtype=np.float64)
    qb, _ = hs["q_cols"]
    kb, _ = hs["kv_cols"]
    group = hs["h_t"] // hs["kv_t"]
    outs = []
    # a causal query row i needs only the keys and values of rows <= i; without the mask
    # every row sees the whole sequence
    need = x if (rows is None or not causal) else x[: int(np.max(rows)) + 1]
    for j in range(hs["h_t"]):
        c0 = qb + j * head_dim
        kc = kb + (j // group) * head_dim
        q = need @ np.asarray(wq[:, c0:c0 + head_dim], dtype=np.float64)
        k = need @ np.asarray(wk[:, kc:kc + head_dim], dtype=np.float64)
        v = need @ np.asarray(wv[:, kc:kc + head_dim], dtype=np.float64)
        outs.append(attention_head(q, k, v, causal=causal, rows=rows))
    return np.concatenate(outs, axis=1)


def block_sequence(x_s, w, n_heads: int, n_kv_heads: int, head_dim: int, T_p: int,
                   act: str = "gelu", rows=None):
    """One sequence through a TP block shard set, all T_p ranks: returns (x1, y).

    Attention sublayer (heads sharded, row-sharded Wo) -> sum over ranks
    (g) + residual -> FFN sublayer (column/row sharded) -> sum over ranks (g)
    + residual.  "7.9 ..." section 2.2: two all-reduces per block; LayerNorm,
    dropout and biases are outside the sharded matmuls and are not part of
    this computation.  ``w`` holds full wq, wk, wv, wo, w1, w3 (or None), w2.
    With ``rows`` only those token rows of x1 and y are returned.
    """
    x_s = np.asarray(x_s, dtype=np.float64)
    a_parts = []
    for t in range(T_p):
        o_t = attn_heads_shard(x_s, w["wq"], w["wk"], w["wv"], n_heads, n_kv_heads, head_dim,
                               T_p, t, causal=True, rows=rows)
        a_parts.append(attn_outproj_shard(o_t, w["wo"], n_heads, n_kv_heads, head_dim, T_p, t))
    res = x_s if rows is None else x_s[np.asarray(rows)]
    x1 = partial_sum(a_parts, residual=res)
    y_parts = [ffn_shard(x1, w["w1"], w.get("w3"), w["w2"], T_p, t, act)[1] for t in range(T_p)]
    return x1, partial_sum(y_parts, residual=x1)


# ----------------------------------------------------------------------------- comparison
def normwise_max_rel_err(got, ref) -> float:
    """max|G - R| / max|R| (0 when both are all zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den
