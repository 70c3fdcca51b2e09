"""Seeded synthetic inputs for the tensor-parallel shard workloads.

This module is shared by the GPU path's tests/bench and by the CPU oracle's
tests.  It holds none of the sublayer's arithmetic: it only draws Gaussian
numbers, scales them by an initialisation standard deviation, optionally
RMS-normalises token rows (part of the input recipe of the Llama-shaped
workloads), and encodes float32 values as bfloat16 bit patterns with
round-to-nearest-even.  Both sides receive exactly the same bits.

Workload shapes follow the pages' problem statement of one FFN sublayer
(d, d_ff, T_p, rank t, activation) and the shapes of GPT-2-medium,
Llama-3-8B, Llama-3-70B and a GPT-style d=6144 block.

Seeds: tensor ``i`` of workload ``c`` is drawn from
``numpy.random.Generator(PCG64(1000 * c + i))`` as float32 standard normals,
then multiplied (in float32) by its std.  Tensor indices: x=0, W1=1, W3=2,
W2=3, Wq=4, Wk=5, Wv=6, Wo=7, O (concatenated head outputs)=8.
Full (unsharded) matrices are drawn; ranks take slices of them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F32 = "f32"
BF16 = "bf16"

T_X, T_W1, T_W3, T_W2, T_WQ, T_WK, T_WV, T_WO, T_O, T_DY = range(10)


@dataclass(frozen=True)
class Workload:
    """Shapes and input recipe of one synthetic workload."""

    cid: int                 # 1-based workload number (seed namespace)
    name: str
    T: int                   # tokens per pass (batch x sequence)
    d: int
    d_ff: int
    T_p: int
    act: str                 # "gelu" | "swiglu"
    dtype: str               # F32 | BF16
    x_std: float = 1.0
    x_rms_norm: bool = False
    w1_std: float = 0.02
    w2_std: float = 0.02
    n_heads: int = 0         # attention (0 = FFN only)
    n_kv_heads: int = 0
    head_dim: int = 0
    wqkv_std: float = 0.02
    wo_std: float = 0.02
    seq_len: int = 0         # >0: T is n_seq sequences of seq_len tokens (causal block)
    has_attn_outproj: bool = False
    has_block: bool = False
    notes: str = ""

    @property
    def n(self) -> int:
        """Hidden units per rank: d_ff / T_p."""
        return self.d_ff // self.T_p

    @property
    def n_seq(self) -> int:
        return self.T // self.seq_len if self.seq_len else 1


WORKLOADS = {
    1: Workload(1, "tiny_gelu_fp32", T=64, d=256, d_ff=1024, T_p=2, act="gelu", dtype=F32,
                x_std=1.0, w1_std=1.0 / math.sqrt(256), w2_std=1.0 / math.sqrt(1024)),
    2: Workload(2, "gpt2_medium_gelu_bf16", T=8 * 512, d=1024, d_ff=4096, T_p=4, act="gelu",
                dtype=BF16, x_std=1.0, w1_std=0.02, w2_std=0.02),
    3: Workload(3, "llama3_8b_swiglu_bf16", T=8192, d=4096, d_ff=14336, T_p=8, act="swiglu",
                dtype=BF16, x_std=1.0, x_rms_norm=True, w1_std=1.0 / math.sqrt(4096),
                w2_std=1.0 / math.sqrt(14336)),
    4: Workload(4, "llama3_70b_swiglu_bf16", T=16384, d=8192, d_ff=28672, T_p=8, act="swiglu",
                dtype=BF16, x_std=1.0, x_rms_norm=True, w1_std=1.0 / math.sqrt(8192),
                w2_std=1.0 / math.sqrt(28672), n_heads=64, n_kv_heads=8, head_dim=128,
                wo_std=1.0 / math.sqrt(64 * 128), has_attn_outproj=True),
    5: Workload(5, "gpt_block_tp8_bf16", T=4 * 2048, d=6144, d_ff=24576, T_p=8, act="gelu",
                dtype=BF16, x_std=1.0, w1_std=0.02, w2_std=0.02, n_heads=48, n_kv_heads=48,
                head_dim=128, wqkv_std=0.02, wo_std=0.02, seq_len=2048, has_block=True),
}


# ----------------------------------------------------------------------------- encoding
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    Inputs must be finite (the generators only produce finite values).
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = (u + bias) >> np.uint32(16)
    return out.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> the exact float32 values they encode."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of a generated tensor (bf16 bits or float32)."""
    if dtype == BF16:
        return bf16_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------------------- drawing
def draw(cid: int, index: int, shape, std: float) -> np.ndarray:
    """float32 N(0,1) draws from PCG64(1000*cid + index), multiplied by std in float32."""
    g = np.random.Generator(np.random.PCG64(1000 * cid + index))
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def rms_normalise_rows(a: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """Input recipe: scale each token row to unit RMS (gain 1), in float32."""
    a = np.asarray(a, dtype=np.float32)
    ms = np.mean(np.square(a, dtype=np.float32), axis=-1, keepdims=True, dtype=np.float32)
    return (a / np.sqrt(ms + np.float32(eps))).astype(np.float32)


def encode(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(a) if dtype == BF16 else np.ascontiguousarray(a, dtype=np.float32)


def make_tensor(w: Workload, name: str) -> np.ndarray:
    """Generate one full tensor of a workload, encoded in the workload's dtype.

    name in {"x", "w1", "w3", "w2", "wq", "wk", "wv", "wo", "o", "dy"}; "dy" is the
    gradient of the loss with respect to the sublayer output, N(0, 1), for the backward.
    """
    if name == "x":
        a = draw(w.cid, T_X, (w.T, w.d), w.x_std)
        if w.x_rms_norm:
            a = rms_normalise_rows(a)
    elif name == "w1":
        a = draw(w.cid, T_W1, (w.d, w.d_ff), w.w1_std)
    elif name == "w3":
        if w.act != "swiglu":
            raise ValueError(f"{w.name} has no W3")
        a = draw(w.cid, T_W3, (w.d, w.d_ff), w.w1_std)
    elif name == "w2":
        a = draw(w.cid, T_W2, (w.d_ff, w.d), w.w2_std)
    elif name in ("wq", "wk", "wv"):
        if not w.has_block:
            raise ValueError(f"{w.name} has no QKV projection")
        heads = w.n_heads if name == "wq" else w.n_kv_heads
        idx = {"wq": T_WQ, "wk": T_WK, "wv": T_WV}[name]
        a = draw(w.cid, idx, (w.d, heads * w.head_dim), w.wqkv_std)
    elif name == "wo":
        if not w.n_heads:
            raise ValueError(f"{w.name} has no attention")
        a = draw(w.cid, T_WO, (w.n_heads * w.head_dim, w.d), w.wo_std)
    elif name == "o":
        if not w.has_attn_outproj:
            raise ValueError(f"{w.name} has no synthetic head outputs")
        a = draw(w.cid, T_O, (w.T, w.n_heads * w.head_dim), 1.0)
    elif name == "dy":
        a = draw(w.cid, T_DY, (w.T, w.d), 1.0)
    else:
        raise KeyError(name)
    return encode(a, w.dtype)


def small_ffn_case(seed: int, T: int, d: int, d_ff: int, act: str, dtype: str,
                   x_std: float = 1.0, w1_std: float | None = None,
                   w2_std: float | None = None) -> dict:
    """Seeded small/ragged FFN inputs for parity and edge-case tests.

    Returns encoded x [T,d], w1/w3 [d,d_ff], w2 [d_ff,d] (w3 only for the gated kinds)
    and dy [T,d] (N(0,1), the output gradient for the backward).
    Default stds are 1/sqrt(fan_in) of the full matrices.
    """
    w1_std = 1.0 / math.sqrt(d) if w1_std is None else w1_std
    w2_std = 1.0 / math.sqrt(d_ff) if w2_std is None else w2_std
    cid = 100000 + seed
    out = {
        "x": encode(draw(cid, T_X, (T, d), x_std), dtype),
        "w1": encode(draw(cid, T_W1, (d, d_ff), w1_std), dtype),
        "w2": encode(draw(cid, T_W2, (d_ff, d), w2_std), dtype),
    }
    if act in ("swiglu", "bilinear"):
        out["w3"] = encode(draw(cid, T_W3, (d, d_ff), w1_std), dtype)
    out["dy"] = encode(draw(cid, T_DY, (T, d), 1.0), dtype)
    return out


def integer_offset_case(T: int, d: int, d_ff: int, seed: int = 7) -> dict:
    """Integer-valued inputs whose sharded FFN (activation NONE) is exact in bf16/fp32.

    x: integers in [-8, 8].  W1 (and W3): column j has a single entry
    (+1 or -1) at row (7*j) mod d, so U = X.W1 is a signed copy of x columns,
    |U| <= 8 (exact in bf16).  W2: entries in {-1, 0, 1}.  With activation NONE
    and float32 output, every sum is an integer of magnitude <= 8*d_ff < 2^24,
    so any correct summation order gives the same bits, and a wrong shard
    offset selects different columns and shows up as a different integer.
    Returned as bf16 bit patterns.
    """
    g = np.random.Generator(np.random.PCG64(424242 + seed))
    x = g.integers(-8, 9, size=(T, d)).astype(np.float32)
    w1 = np.zeros((d, d_ff), dtype=np.float32)
    w3 = np.zeros((d, d_ff), dtype=np.float32)
    cols = np.arange(d_ff)
    w1[(7 * cols) % d, cols] = g.choice([-1.0, 1.0], size=d_ff)
    w3[(5 * cols + 3) % d, cols] = g.choice([-1.0, 1.0], size=d_ff)
    w2 = g.integers(-1, 2, size=(d_ff, d)).astype(np.float32)
    return {"x": bf16_bits(x), "w1": bf16_bits(w1), "w3": bf16_bits(w3), "w2": bf16_bits(w2)}


def integer_backward_case(T: int, d: int, d_ff: int, seed: int = 7) -> dict:
    """Integer-valued inputs whose sharded FFN backward is exact (activation NONE or
    BILINEAR, float32 gradients).

    x: integers in [-8, 8]; W1 and W3 as in integer_offset_case (one +-1 per
    column, so U and V are signed copies of x columns, |U|, |V| <= 8).  W2: one
    +-1 per row (hidden unit j) at column (3*j + 1) mod d, so dH = dY W2(t)^T is a
    signed copy of dY columns.  dy: integers in [-4, 4].  Then |dU|, |dV| <= 32 and
    |H| <= 64 (exact in bf16) and every gradient entry is an integer below 2^24 for
    T < 65536: any summation order gives the same bits, and a wrong block offset
    shows up as different integers.  Returned as bf16 bit patterns.
    """
    g = np.random.Generator(np.random.PCG64(525252 + seed))
    x = g.integers(-8, 9, size=(T, d)).astype(np.float32)
    w1 = np.zeros((d, d_ff), dtype=np.float32)
    w3 = np.zeros((d, d_ff), dtype=np.float32)
    w2 = np.zeros((d_ff, d), dtype=np.float32)
    cols = np.arange(d_ff)
    w1[(7 * cols) % d, cols] = g.choice([-1.0, 1.0], size=d_ff)
    w3[(5 * cols + 3) % d, cols] = g.choice([-1.0, 1.0], size=d_ff)
    w2[cols, (3 * cols + 1) % d] = g.choice([-1.0, 1.0], size=d_ff)
    dy = g.integers(-4, 5, size=(T, d)).astype(np.float32)
    return {"x": bf16_bits(x), "w1": bf16_bits(w1), "w3": bf16_bits(w3), "w2": bf16_bits(w2),
            "dy": bf16_bits(dy)}


def bf16_grid(lo_exp: int, hi_exp: int, limit: float) -> np.ndarray:
    """Every bfloat16 value v with 2^lo_exp <= |v| < 2^(hi_exp+1) and |v| <= limit, both
    signs, plus +0 and -0, as float32 (each exactly a bf16 value)."""
    mags = []
    for e in range(lo_exp, hi_exp + 1):
        mags.append(np.float32(2.0 ** e) * (1.0 + np.arange(128, dtype=np.float32) / 128.0))
    m = np.concatenate(mags).astype(np.float32)
    m = m[m <= limit]
    return np.concatenate([m, -m, np.array([0.0, -0.0], dtype=np.float32)])


def activation_grid_case(T: int, n: int, T_p: int, seed: int = 3) -> dict:
    """Inputs that put chosen pre-activations into the column product exactly.

    d = 2n.  x[:, :n] holds every bfloat16 value in [-12, 12] with magnitude at least
    2^-20 (and +-0), tiled over the T x n cells in a seeded random order; x[:, n:] holds
    the gate values: 1.0 in a seeded half of the cells, other bf16 values in [-4, 4]
    elsewhere.  Every rank's block of W1 is [I_n; 0] and of W3 is [0; I_n], so each
    rank's U = X W1(t) and V = X W3(t) are exactly x[:, :n] and x[:, n:] (one non-zero
    product per sum).  Every rank's row block of W2 is [I_n | 0], so y(t) = [H | 0] and,
    in the backward, dH = dY W2(t)^T = dy[:, :n] exactly.  dy holds bf16 values in
    [-4, 4] (1.0 in a seeded quarter of the cells).  Returned as bf16 bit patterns."""
    g = np.random.Generator(np.random.PCG64(636363 + seed))
    grid = bf16_grid(-20, 3, 12.0)
    reps = -(-T * n // grid.size)
    u = np.concatenate([g.permutation(grid) for _ in range(reps)])[: T * n].reshape(T, n)
    small = bf16_grid(-20, 1, 4.0)
    v = g.choice(small, size=(T, n)).astype(np.float32)
    v[g.random((T, n)) < 0.5] = 1.0
    dy = g.choice(small, size=(T, 2 * n)).astype(np.float32)
    dy[g.random((T, 2 * n)) < 0.25] = 1.0
    eye = np.eye(n, dtype=np.float32)
    zero = np.zeros((n, n), dtype=np.float32)
    w1 = np.tile(np.vstack([eye, zero]), (1, T_p))
    w3 = np.tile(np.vstack([zero, eye]), (1, T_p))
    w2 = np.tile(np.hstack([eye, zero]), (T_p, 1))
    x = np.hstack([u, v]).astype(np.float32)
    return {"x": bf16_bits(x), "w1": bf16_bits(w1), "w3": bf16_bits(w3), "w2": bf16_bits(w2),
            "dy": bf16_bits(dy)}
