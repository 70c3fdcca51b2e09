"""Split-K path of the forward products (a few thousand tokens, too few output tiles to fill
the GPU): the k range is split over several workgroups per tile, each writes an fp32 partial
product into the caller's workspace, and a second kernel adds them in split order and
applies the activation.  The library takes this path when the workspace holds more than
H(t) (or Q, K, V): the queries return the size that enables it.

Checked against the oracle ("7.9 Tensor and pipeline parallelism", section 2.1, h^(t) and
y^(t); section 2.2 for the Q, K, V projections), bit for bit on integer inputs, against
the unsplit path, and for bitwise repeatability.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from _gpu_util import BF16_TOL, dev, f64, host64, log, nerr, requires_gpu, sample_rows
from megatron_tensor_transformer_gemm_amd import inputs as I
from megatron_tensor_transformer_gemm_amd import tpshard as S
from oracle import tp_oracle as O

pytestmark = [pytest.mark.gpu, requires_gpu]


def _shard(dd, T, d, d_ff, T_p, t, act, out_code, split: bool):
    """tp_ffn_shard_fwd with the full workspace (split-K allowed) or just H(t) (no split)."""
    n = d_ff // T_p
    full = S.tp_ffn_workspace_bytes(T, d_ff, T_p, S.TP_BF16)
    hbytes = (T * n * 2 + 255) // 256 * 256
    nb = full if split else hbytes
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
    y = torch.full((T, d), float("nan"), dtype=torch.float32 if out_code == S.TP_F32 else torch.bfloat16,
                   device="cuda:0")
    S.tp_ffn_shard_fwd(dd["x"], dd["w1"], dd.get("w3"), dd["w2"], y, ws, nb, T, d, d_ff, T_p, t, act,
                       S.TP_BF16, out_code)
    torch.cuda.synchronize()
    return y, ws[: T * n * 2].view(torch.bfloat16).view(T, n).clone()


def test_workspace_query_enables_split_for_block_sized_products():
    full = S.tp_ffn_workspace_bytes(2000, 6144, 2, S.TP_BF16)
    assert full > 2000 * 3072 * 2, "the 2000-token product should get split-K scratch"
    assert S.tp_ffn_workspace_bytes(16384, 28672, 8, S.TP_BF16) == 16384 * 3584 * 2


@pytest.mark.parametrize("act", ["none", "bilinear"])
@pytest.mark.parametrize("shape", [(2000, 4096, 2, 3072), (1500, 4104, 4, 1536)],
                         ids=["2-splits-192col", "4-splits-ragged-k"])
def test_split_integer_bit_exact(act, shape):
    """Integer inputs: every partial sum is an exact integer, so H(t) (bf16) and y(t) (fp32)
    equal the oracle bit for bit, and equal the unsplit path's."""
    T, d, T_p, n = shape
    d_ff = T_p * n
    log(f"[splitk-integer] act={act} T={T} d={d} d_ff={d_ff} T_p={T_p}")
    c = I.integer_offset_case(T, d, d_ff)
    keys = ("x", "w1", "w3", "w2") if act == "bilinear" else ("x", "w1", "w2")
    dd = {k: dev(c[k], I.BF16) for k in keys}
    x, w1, w3, w2 = (f64(c[k], I.BF16) for k in ("x", "w1", "w3", "w2"))
    for t in (0, T_p - 1):
        y, h = _shard(dd, T, d, d_ff, T_p, t, act, S.TP_F32, split=True)
        y0, h0 = _shard(dd, T, d, d_ff, T_p, t, act, S.TP_F32, split=False)
        h_ref, y_ref = O.ffn_shard(x, w1, w3, w2, T_p, t, act)
        assert np.array_equal(host64(h), h_ref), f"H({t}) differs"
        assert np.array_equal(host64(y), y_ref), f"y({t}) differs"
        assert torch.equal(h, h0) and torch.equal(y, y0)


@pytest.mark.parametrize("act,n", [("gelu", 3072), ("swiglu", 1536)])
def test_split_float_parity_and_repeatability(act, n):
    """GPT-block-sized ranks (2048 tokens, d = 6144; GELU with n = 3072 splits 2 ways over 256 x
    192 tiles, SwiGLU with n = 1536 2 ways over the gated pair's tiles): H(t) and y(t) against
    the oracle on sampled rows, against the unsplit path normwise, and two calls bitwise equal
    (the partials are added in split order, no atomics)."""
    T, d, T_p, t = 2048, 6144, 8, 5
    d_ff = n * T_p
    log(f"[splitk-float] act={act} T={T} d={d} n={n}")
    c = I.small_ffn_case(77, T, d, d_ff, act, I.BF16)
    keys = ("x", "w1", "w3", "w2") if act == "swiglu" else ("x", "w1", "w2")
    dd = {k: dev(c[k], I.BF16) for k in keys}
    y, h = _shard(dd, T, d, d_ff, T_p, t, act, S.TP_BF16, split=True)
    y2, h2 = _shard(dd, T, d, d_ff, T_p, t, act, S.TP_BF16, split=True)
    y0, h0 = _shard(dd, T, d, d_ff, T_p, t, act, S.TP_BF16, split=False)
    assert torch.equal(h, h2) and torch.equal(y, y2), "split-K is not bitwise repeatable"
    rows = sample_rows(T, 512, seed=12)
    b = t * n
    xs = f64(c["x"][rows], I.BF16)
    w1s = f64(c["w1"][:, b:b + n], I.BF16)
    w3s = f64(c["w3"][:, b:b + n], I.BF16) if act == "swiglu" else None
    w2s = f64(c["w2"][b:b + n], I.BF16)
    h_ref, y_ref = O.ffn_shard(xs, w1s, w3s, w2s, 1, 0, act)
    eh, ey = nerr(host64(h[rows]), h_ref), nerr(host64(y[rows]), y_ref)
    log(f"   err(H)={eh:.3e} err(y)={ey:.3e}; vs unsplit {nerr(host64(h), host64(h0)):.3e}")
    assert eh <= BF16_TOL and ey <= BF16_TOL
    assert nerr(host64(h), host64(h0)) <= 2 ** -7


def test_split_qkv_projection_against_unsplit_and_oracle():
    """The GPT block's fused Q, K, V projection of one rank (2048 tokens, 6 query heads)
    through tp_attn_heads_shard_fwd: with the full workspace it splits k three ways; O(t)
    against the unsplit call and against the oracle on sampled rows."""
    L, d, H, dh, T_p, t = 2048, 6144, 48, 128, 8, 2
    g = np.random.default_rng(31)
    x = I.bf16_bits(g.standard_normal((L, d)).astype(np.float32))
    wq, wk, wv = (I.bf16_bits((g.standard_normal((d, H * dh)) * 0.02).astype(np.float32)) for _ in range(3))
    xd, wqd, wkd, wvd = (dev(a, I.BF16) for a in (x, wq, wk, wv))
    h_t = H // T_p
    full = S.tp_attn_heads_workspace_bytes(1, L, H, H, dh, T_p)
    qkv = L * 3 * h_t * dh * 2
    assert full > qkv
    outs = []
    for nb in (full, qkv):
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
        o = torch.full((L, h_t * dh), float("nan"), dtype=torch.bfloat16, device="cuda:0")
        S.tp_attn_heads_shard_fwd(xd, wqd, wkd, wvd, o, ws, nb, 1, L, d, H, H, dh, T_p, t, True)
        torch.cuda.synchronize()
        outs.append(o)
    e_split = nerr(host64(outs[0]), host64(outs[1]))
    rows = sample_rows(L, 256, seed=3)
    ref = O.attn_heads_shard(f64(x, I.BF16), f64(wq, I.BF16), f64(wk, I.BF16), f64(wv, I.BF16), H, H, dh,
                             T_p, t, causal=True, rows=rows)
    e = nerr(host64(outs[0][rows]), ref)
    log(f"   err(O) vs oracle {e:.3e}, vs unsplit {e_split:.3e}")
    assert e <= BF16_TOL and e_split <= BF16_TOL
