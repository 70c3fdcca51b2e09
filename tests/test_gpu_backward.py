"""GPU parity of the FFN shard backward (and of the training forward that keeps U, V
and H for it), against the CPU oracle, through the C ABI."""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

from _gpu_util import BF16_TOL, dev, f64, host64, log, nerr, requires_gpu, sample_rows
from megatron_tensor_transformer_gemm_amd import inputs as I
from megatron_tensor_transformer_gemm_amd import tpshard as S
from oracle import tp_oracle as O

pytestmark = [pytest.mark.gpu, requires_gpu]

GATED = ("swiglu", "bilinear")
SENTINEL = 1536.0   # exact in bf16; written before the call: entries outside rank t's blocks must keep it


def _tdt(code):
    return torch.float32 if code == S.TP_F32 else torch.bfloat16


def _train_fwd(xd, w1d, w3d, w2d, T, d, d_ff, T_p, t, act, out_code=S.TP_BF16):
    n = d_ff // T_p
    y = torch.full((T, d), float("nan"), dtype=_tdt(out_code), device="cuda:0")
    h = torch.full((T, n), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    u = torch.full((T, n), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    v = torch.full((T, n), float("nan"), dtype=torch.bfloat16, device="cuda:0") if act in GATED else None
    S.tp_ffn_shard_fwd_train(xd, w1d, w3d if act in GATED else None, w2d, y, h, u, v, T, d, d_ff, T_p, t,
                             act, out_code)
    return y, h, u, v


def _bwd(xd, w1d, w3d, w2d, dyd, h, u, v, T, d, d_ff, T_p, t, act, dx_code, g_code):
    gated = act in GATED
    dx = torch.full((T, d), float("nan"), dtype=_tdt(dx_code), device="cuda:0")
    dw1 = torch.full((d, d_ff), SENTINEL, dtype=_tdt(g_code), device="cuda:0")
    dw3 = torch.full((d, d_ff), SENTINEL, dtype=_tdt(g_code), device="cuda:0") if gated else None
    dw2 = torch.full((d_ff, d), SENTINEL, dtype=_tdt(g_code), device="cuda:0")
    nbytes = S.tp_ffn_bwd_workspace_bytes(T, d_ff, T_p, act)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda:0")
    S.tp_ffn_shard_bwd(xd, w1d, w3d if gated else None, w2d, dyd, h, u, v, dx, dw1, dw3, dw2, ws,
                       ws.numel(), T, d, d_ff, T_p, t, act, dx_code, g_code)
    torch.cuda.synchronize()
    return dx, dw1, dw3, dw2


def _check_untouched(full: np.ndarray, lo: int, hi: int, axis: int, name: str):
    """Entries outside [lo, hi) along `axis` still hold the sentinel."""
    outside = np.delete(full, np.arange(lo, hi), axis=axis)
    assert np.all(outside == SENTINEL), f"{name}: entries outside rank's block were written"


# ----------------------------------------------------------------------------- bit-exact offsets
@pytest.mark.parametrize("act", ["none", "bilinear"])
@pytest.mark.parametrize("shape", [(300, 264, 4, 136), (4100, 1032, 2, 1288), (4100, 264, 1, 4000),
                                   (4000, 4000, 1, 4000)],
                         ids=["small-tiles", "large-tiles", "dH-128x256-3-stage", "full-wave-256x256"])
def test_backward_integer_bit_exact(act, shape):
    """Integer inputs: dX(t) and the weight-gradient blocks (fp32) equal the oracle bit for bit,
    and nothing outside the rank's blocks is written.  The last shape gives every product a
    full wave of 256 x 256 tiles (16 x 16, ragged at 4000), the dispatch of the full-size
    backward (8 waves; dW with four 32-deep stages)."""
    T, d, T_p, n = shape
    d_ff = T_p * n
    log(f"[bwd-integer] act={act} T={T} d={d} d_ff={d_ff} T_p={T_p}")
    c = I.integer_backward_case(T, d, d_ff)
    xd, w1d, w3d, w2d, dyd = (dev(c[k], I.BF16) for k in ("x", "w1", "w3", "w2", "dy"))
    x, w1, w3, w2, dy = (f64(c[k], I.BF16) for k in ("x", "w1", "w3", "w2", "dy"))
    for t in range(T_p):
        b = t * n
        if act == "none":
            h = torch.empty((T, n), dtype=torch.bfloat16, device="cuda:0")
            S.tp_ffn_column_fwd(xd, w1d, None, h, T, d, d_ff, T_p, t, "none", S.TP_BF16)
            u, v = None, None
        else:
            _, h, u, v = _train_fwd(xd, w1d, w3d, w2d, T, d, d_ff, T_p, t, act)
        dx, dw1, dw3, dw2 = _bwd(xd, w1d, w3d, w2d, dyd, h, u, v, T, d, d_ff, T_p, t, act, S.TP_F32,
                                 S.TP_F32)
        ref = O.ffn_shard_bwd(x, w1, w3, w2, dy, T_p, t, act)
        assert np.array_equal(host64(dx), ref["dx_t"]), f"dX({t}) differs"
        g1, g2 = host64(dw1), host64(dw2)
        assert np.array_equal(g1[:, b:b + n], ref["dw1"]), f"dW1 block {t} differs"
        assert np.array_equal(g2[b:b + n, :], ref["dw2"]), f"dW2 block {t} differs"
        _check_untouched(g1, b, b + n, 1, "dW1")
        _check_untouched(g2, b, b + n, 0, "dW2")
        if act in GATED:
            g3 = host64(dw3)
            assert np.array_equal(g3[:, b:b + n], ref["dw3"]), f"dW3 block {t} differs"
            _check_untouched(g3, b, b + n, 1, "dW3")


# ----------------------------------------------------------------------------- training forward
@pytest.mark.parametrize("act", ["gelu", "swiglu", "bilinear"])
@pytest.mark.parametrize("shape", [(520, 264, 1056, 4, 2), (2000, 2048, 6144, 2, 1)],
                         ids=["small", "192-col-tiles"])
def test_train_forward_keeps_preactivations(act, shape):
    """y and H equal the plain forward bit for bit; U (V) equal the column product with no
    activation bit for bit (same kernels, same accumulation), and the oracle within tolerance.
    The second shape's ungated column products run as 256 tiles of 128 x 192."""
    T, d, d_ff, T_p, t = shape
    n = d_ff // T_p
    log(f"[train-fwd] act={act} shape={shape}")
    c = I.small_ffn_case(11, T, d, d_ff, act, I.BF16)
    xd, w1d, w2d = dev(c["x"], I.BF16), dev(c["w1"], I.BF16), dev(c["w2"], I.BF16)
    w3d = dev(c["w3"], I.BF16) if act in GATED else None
    y, h, u, v = _train_fwd(xd, w1d, w3d, w2d, T, d, d_ff, T_p, t, act)
    y0 = torch.empty((T, d), dtype=torch.bfloat16, device="cuda:0")
    # a workspace of exactly H(t): the plain forward then runs the same (unsplit) kernels
    ws = torch.empty((T * n * 2 + 255) // 256 * 256, dtype=torch.uint8, device="cuda:0")
    S.tp_ffn_shard_fwd(xd, w1d, w3d, w2d, y0, ws, ws.numel(), T, d, d_ff, T_p, t, act, S.TP_BF16, S.TP_BF16)
    u0 = torch.empty((T, n), dtype=torch.bfloat16, device="cuda:0")
    S.tp_ffn_column_fwd(xd, w1d, None, u0, T, d, d_ff, T_p, t, "none", S.TP_BF16)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    assert torch.equal(h, ws[: T * n * 2].view(torch.bfloat16).view(T, n))
    assert torch.equal(u, u0)
    x, w1 = f64(c["x"], I.BF16), f64(c["w1"], I.BF16)
    assert nerr(host64(u), x @ w1[:, t * n:(t + 1) * n]) < BF16_TOL
    if act in GATED:
        v0 = torch.empty((T, n), dtype=torch.bfloat16, device="cuda:0")
        S.tp_ffn_column_fwd(xd, w3d, None, v0, T, d, d_ff, T_p, t, "none", S.TP_BF16)
        torch.cuda.synchronize()
        assert torch.equal(v, v0)


# ----------------------------------------------------------------------------- float parity
CASES = [
    # T, d, d_ff, T_p, act, dx dtype, grad dtype
    (300, 264, 272, 2, "gelu", S.TP_BF16, S.TP_F32),
    (257, 136, 544, 4, "swiglu", S.TP_F32, S.TP_F32),
    (1000, 328, 800, 4, "bilinear", S.TP_BF16, S.TP_BF16),
    (64, 64, 128, 1, "gelu", S.TP_BF16, S.TP_F32),
    (3000, 1024, 4096, 4, "swiglu", S.TP_BF16, S.TP_F32),
    (1, 64, 64, 1, "swiglu", S.TP_BF16, S.TP_BF16),
    (700, 520, 1040, 2, "none", S.TP_F32, S.TP_BF16),
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}-d{c[1]}-dff{c[2]}-tp{c[3]}-{c[4]}-dx{c[5]}-g{c[6]}"
                                             for c in CASES])
def test_backward_parity(case):
    """Every rank: dX(t), dW1/dW3/dW2 blocks against the oracle; the ranks' dX(t) reduced by
    tp_partial_sum against the unsharded dX."""
    T, d, d_ff, T_p, act, dxc, gc = case
    n = d_ff // T_p
    log(f"[bwd] {case}")
    c = I.small_ffn_case(zlib.crc32(repr(case).encode()) % 1000, T, d, d_ff, act, I.BF16)
    xd, w1d, w2d, dyd = (dev(c[k], I.BF16) for k in ("x", "w1", "w2", "dy"))
    w3d = dev(c["w3"], I.BF16) if act in GATED else None
    x, w1, w2, dy = (f64(c[k], I.BF16) for k in ("x", "w1", "w2", "dy"))
    w3 = f64(c["w3"], I.BF16) if act in GATED else None
    parts = torch.empty((T_p, T, d), dtype=_tdt(dxc), device="cuda:0")
    for t in range(T_p):
        b = t * n
        if act == "none":
            h = torch.empty((T, n), dtype=torch.bfloat16, device="cuda:0")
            S.tp_ffn_column_fwd(xd, w1d, None, h, T, d, d_ff, T_p, t, "none", S.TP_BF16)
            u, v = None, None
        else:
            _, h, u, v = _train_fwd(xd, w1d, w3d, w2d, T, d, d_ff, T_p, t, act)
        dx, dw1, dw3, dw2 = _bwd(xd, w1d, w3d, w2d, dyd, h, u, v, T, d, d_ff, T_p, t, act, dxc, gc)
        parts[t].copy_(dx)
        ref = O.ffn_shard_bwd(x, w1, w3, w2, dy, T_p, t, act)
        errs = {"dx": nerr(host64(dx), ref["dx_t"]),
                "dw1": nerr(host64(dw1)[:, b:b + n], ref["dw1"]),
                "dw2": nerr(host64(dw2)[b:b + n, :], ref["dw2"])}
        if act in GATED:
            errs["dw3"] = nerr(host64(dw3)[:, b:b + n], ref["dw3"])
        log(f"  t={t} " + " ".join(f"{k}={e:.2e}" for k, e in errs.items()))
        assert all(e < BF16_TOL for e in errs.values()), errs
        _check_untouched(host64(dw1), b, b + n, 1, "dW1")
        _check_untouched(host64(dw2), b, b + n, 0, "dW2")
    dx_all = torch.empty((T, d), dtype=torch.float32, device="cuda:0")
    S.tp_partial_sum(parts, T * d, T_p, None, dx_all, T * d, dxc, S.TP_F32)
    torch.cuda.synchronize()
    full = O.ffn_shard_bwd(x, w1, w3, w2, dy, 1, 0, act)["dx_t"]
    assert nerr(host64(dx_all), full) < BF16_TOL


def test_backward_zero_tokens_zeroes_weight_blocks():
    T, d, d_ff, T_p, t = 0, 64, 256, 2, 1
    n = d_ff // T_p
    x = torch.empty((1, d), dtype=torch.bfloat16, device="cuda:0")
    w1 = torch.ones((d, d_ff), dtype=torch.bfloat16, device="cuda:0")
    w3 = torch.ones((d, d_ff), dtype=torch.bfloat16, device="cuda:0")
    w2 = torch.ones((d_ff, d), dtype=torch.bfloat16, device="cuda:0")
    one = torch.empty((1, n), dtype=torch.bfloat16, device="cuda:0")
    dx = torch.empty((1, d), dtype=torch.bfloat16, device="cuda:0")
    dw1 = torch.full((d, d_ff), SENTINEL, dtype=torch.float32, device="cuda:0")
    dw3 = torch.full((d, d_ff), SENTINEL, dtype=torch.float32, device="cuda:0")
    dw2 = torch.full((d_ff, d), SENTINEL, dtype=torch.float32, device="cuda:0")
    S.tp_ffn_shard_bwd(x, w1, w3, w2, x, one, one, one, dx, dw1, dw3, dw2, None, 0, T, d, d_ff, T_p,
                       t, "swiglu", S.TP_BF16, S.TP_F32)
    torch.cuda.synchronize()
    for g, ax in ((dw1, 1), (dw3, 1), (dw2, 0)):
        a = host64(g)
        blk = a[:, t * n:(t + 1) * n] if ax == 1 else a[t * n:(t + 1) * n, :]
        assert np.all(blk == 0.0)
        _check_untouched(a, t * n, (t + 1) * n, ax, "grad")


# ----------------------------------------------------------------------------- full-size workloads
def _sampled_backward(w: I.Workload, t: int, n_rows: int, n_cols: int):
    """Rank t's backward at the workload's full shape; dX(t) on sampled rows, dW1/dW3 on
    sampled columns (all d rows), dW2 on sampled rows (all d columns), each computed by the
    oracle's definitions on just the slices it needs."""
    T, d, d_ff, T_p, act = w.T, w.d, w.d_ff, w.T_p, w.act
    n = d_ff // T_p
    b = t * n
    gated = act in GATED
    log(f"[bwd-full] {w.name} t={t}: generating inputs")
    host = {k: I.make_tensor(w, k) for k in ("x", "w1", "w2", "dy") + (("w3",) if gated else ())}
    D = {k: dev(a, w.dtype) for k, a in host.items()}
    log(f"[bwd-full] {w.name} t={t}: forward + backward on the GPU")
    _, h, u, v = _train_fwd(D["x"], D["w1"], D.get("w3"), D["w2"], T, d, d_ff, T_p, t, act)
    dx, dw1, dw3, dw2 = _bwd(D["x"], D["w1"], D.get("w3"), D["w2"], D["dy"], h, u, v, T, d, d_ff, T_p,
                             t, act, S.TP_BF16, S.TP_F32)
    del D, h, u, v
    x = f64(host["x"], w.dtype)
    dy = f64(host["dy"], w.dtype)
    w1c = f64(host["w1"][:, b:b + n], w.dtype)
    w2r = f64(host["w2"][b:b + n, :], w.dtype)
    w3c = f64(host["w3"][:, b:b + n], w.dtype) if gated else None
    errs = {}
    # dX(t) rows: the oracle's whole chain on those token rows
    rows = sample_rows(T, n_rows, 123 + t)
    xr, dyr = x[rows], dy[rows]
    ur = xr @ w1c
    vr = xr @ w3c if gated else None
    du, dv = O.act_backward(dyr @ w2r.T, ur, vr, act)
    dx_ref = du @ w1c.T + (dv @ w3c.T if gated else 0.0)
    errs["dx"] = nerr(host64(dx[torch.as_tensor(rows, device="cuda:0")]), dx_ref)
    # dW1 / dW3 columns j and dW2 rows j of the block: need U, V, dU, dV of hidden unit j, all tokens
    cols = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(99 + t).choice(n, n_cols, False)]))
    U = x @ w1c[:, cols]
    V = x @ w3c[:, cols] if gated else None
    dH = dy @ w2r[cols, :].T
    dU, dV = O.act_backward(dH, U, V, act)
    k = len(cols)
    Hc = O.column_parallel(x, w1c[:, cols], w3c[:, cols] if gated else None, (0, k), act)
    g1 = host64(dw1)[:, b + cols]
    errs["dw1"] = nerr(g1, x.T @ dU)
    errs["dw2"] = nerr(host64(dw2)[b + cols, :], Hc.T @ dy)
    if gated:
        errs["dw3"] = nerr(host64(dw3)[:, b + cols], x.T @ dV)
    log(f"[bwd-full] {w.name} t={t}: " + " ".join(f"{k}={e:.2e}" for k, e in errs.items()))
    assert all(e < BF16_TOL for e in errs.values()), errs


@pytest.mark.slow
def test_backward_llama3_8b_shape_sampled():
    _sampled_backward(I.WORKLOADS[3], t=5, n_rows=1024, n_cols=16)


@pytest.mark.slow
def test_backward_llama3_70b_shape_sampled():
    _sampled_backward(I.WORKLOADS[4], t=3, n_rows=1024, n_cols=8)


# ----------------------------------------------------------------------------- out-projection backward
def _outproj_bwd(od, wod, dyd, T, d, H, KV, dh, T_p, t, gc):
    k = H // T_p * dh
    do = torch.full((T, k), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    dwo = torch.full((H * dh, d), SENTINEL, dtype=_tdt(gc), device="cuda:0")
    S.tp_attn_outproj_shard_bwd(od, wod, dyd, do, dwo, T, d, H, KV, dh, T_p, t, gc)
    torch.cuda.synchronize()
    return do, dwo


def test_outproj_backward_integer_bit_exact():
    """O(t) integers in [-8, 8], Wo with one +-1 per row, dY integers in [-4, 4]: dO(t) (bf16)
    and the fp32 dWo block are exact integers, equal to the oracle bit for bit."""
    T, d, H, KV, dh, T_p = 1000, 520, 16, 8, 64, 4
    k = H // T_p * dh
    g = np.random.default_rng(31)
    o = g.integers(-8, 9, (T, H * dh)).astype(np.float32)
    wo = np.zeros((H * dh, d), dtype=np.float32)
    rows = np.arange(H * dh)
    wo[rows, (5 * rows + 2) % d] = g.choice([-1.0, 1.0], H * dh)
    dy = g.integers(-4, 5, (T, d)).astype(np.float32)
    wod, dyd = dev(I.bf16_bits(wo), I.BF16), dev(I.bf16_bits(dy), I.BF16)
    for t in range(T_p):
        od = dev(I.bf16_bits(np.ascontiguousarray(o[:, t * k:(t + 1) * k])), I.BF16)
        do, dwo = _outproj_bwd(od, wod, dyd, T, d, H, KV, dh, T_p, t, S.TP_F32)
        ref = O.attn_outproj_shard_bwd(o[:, t * k:(t + 1) * k], wo, dy, H, KV, dh, T_p, t)
        assert np.array_equal(host64(do), ref["do_t"]), f"dO({t}) differs"
        gw = host64(dwo)
        assert np.array_equal(gw[t * k:(t + 1) * k], ref["dwo"]), f"dWo block {t} differs"
        _check_untouched(gw, t * k, (t + 1) * k, 0, "dWo")


@pytest.mark.parametrize("gc", [S.TP_F32, S.TP_BF16])
def test_outproj_backward_parity(gc):
    T, d, H, KV, dh, T_p, t = 777, 392, 12, 6, 128, 3, 2
    k = H // T_p * dh
    g = np.random.default_rng(41 + gc)
    o = I.bf16_bits(g.standard_normal((T, k)).astype(np.float32))
    wo = I.bf16_bits((g.standard_normal((H * dh, d)) / np.sqrt(H * dh)).astype(np.float32))
    dy = I.bf16_bits(g.standard_normal((T, d)).astype(np.float32))
    do, dwo = _outproj_bwd(dev(o, I.BF16), dev(wo, I.BF16), dev(dy, I.BF16), T, d, H, KV, dh, T_p, t, gc)
    ref = O.attn_outproj_shard_bwd(f64(o, I.BF16), f64(wo, I.BF16), f64(dy, I.BF16), H, KV, dh, T_p, t)
    e1 = nerr(host64(do), ref["do_t"])
    e2 = nerr(host64(dwo)[t * k:(t + 1) * k], ref["dwo"])
    log(f"[outproj-bwd] grad dtype {gc}: dO {e1:.2e} dWo {e2:.2e}")
    assert e1 < BF16_TOL and e2 < BF16_TOL
    _check_untouched(host64(dwo), t * k, (t + 1) * k, 0, "dWo")


@pytest.mark.slow
def test_outproj_backward_llama3_70b_shape_sampled():
    w = I.WORKLOADS[4]
    T, d, H, KV, dh, T_p, t = w.T, w.d, w.n_heads, w.n_kv_heads, w.head_dim, w.T_p, 6
    k = H // T_p * dh
    log(f"[outproj-bwd-full] {w.name} t={t}")
    o_full = I.make_tensor(w, "o")
    o = np.ascontiguousarray(o_full[:, t * k:(t + 1) * k])
    wo = I.make_tensor(w, "wo")
    dy = I.make_tensor(w, "dy")
    do, dwo = _outproj_bwd(dev(o, w.dtype), dev(wo, w.dtype), dev(dy, w.dtype), T, d, H, KV, dh, T_p, t,
                           S.TP_F32)
    dy64 = f64(dy, w.dtype)
    wr = f64(wo[t * k:(t + 1) * k], w.dtype)
    rows = sample_rows(T, 1024, 77)
    e1 = nerr(host64(do[torch.as_tensor(rows, device="cuda:0")]), dy64[rows] @ wr.T)
    cols = np.unique(np.concatenate([[0, k - 1], np.random.default_rng(5).choice(k, 16, False)]))
    e2 = nerr(host64(dwo)[t * k + cols], f64(o[:, cols], w.dtype).T @ dy64)
    log(f"[outproj-bwd-full] dO {e1:.2e} dWo {e2:.2e}")
    assert e1 < BF16_TOL and e2 < BF16_TOL


def test_new_entry_points_with_no_tokens():
    """T = 0: the training forward and the reduce-scatter are no-ops; the out-projection
    backward zeroes rank t's rows of dWo and touches nothing else."""
    d, H, dh, T_p, t = 64, 8, 64, 4, 2
    k = H // T_p * dh
    z = torch.zeros((1, 1024), dtype=torch.bfloat16, device="cuda:0")
    y = torch.full((8, d), 7.0, dtype=torch.bfloat16, device="cuda:0")
    S.tp_ffn_shard_fwd_train(z, z, None, z, y, z, z, None, 0, d, 256, T_p, t, "gelu", S.TP_BF16)
    S.tp_reduce_scatter_rows(z, 0, T_p, t, None, y, 0, d, S.TP_BF16, S.TP_BF16)
    dwo = torch.full((H * dh, d), SENTINEL, dtype=torch.float32, device="cuda:0")
    S.tp_attn_outproj_shard_bwd(z, z, z, z, dwo, 0, d, H, H, dh, T_p, t, S.TP_F32)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
    g = host64(dwo)
    assert np.all(g[t * k:(t + 1) * k] == 0.0)
    _check_untouched(g, t * k, (t + 1) * k, 0, "dWo")


@pytest.mark.slow
def test_backward_gpt2_medium_shape_every_rank():
    """GELU workload at full size (4096 tokens, d 1024, d_ff 4096, TP4): every rank's dX(t) and
    weight-gradient blocks against the oracle, and the reduced dX against the unsharded one."""
    w = I.WORKLOADS[2]
    T, d, d_ff, T_p, act = w.T, w.d, w.d_ff, w.T_p, w.act
    n = d_ff // T_p
    host = {k: I.make_tensor(w, k) for k in ("x", "w1", "w2", "dy")}
    D = {k: dev(a, w.dtype) for k, a in host.items()}
    x, w1, w2, dy = (f64(host[k], w.dtype) for k in ("x", "w1", "w2", "dy"))
    parts = torch.empty((T_p, T, d), dtype=torch.float32, device="cuda:0")
    for t in range(T_p):
        b = t * n
        _, h, u, v = _train_fwd(D["x"], D["w1"], None, D["w2"], T, d, d_ff, T_p, t, act)
        dx, dw1, _, dw2 = _bwd(D["x"], D["w1"], None, D["w2"], D["dy"], h, u, v, T, d, d_ff, T_p, t, act,
                               S.TP_F32, S.TP_F32)
        parts[t].copy_(dx)
        ref = O.ffn_shard_bwd(x, w1, None, w2, dy, T_p, t, act)
        errs = (nerr(host64(dx), ref["dx_t"]), nerr(host64(dw1)[:, b:b + n], ref["dw1"]),
                nerr(host64(dw2)[b:b + n, :], ref["dw2"]))
        log(f"[bwd-gpt2] t={t} dx={errs[0]:.2e} dw1={errs[1]:.2e} dw2={errs[2]:.2e}")
        assert max(errs) < BF16_TOL
    dx_all = torch.empty((T, d), dtype=torch.float32, device="cuda:0")
    S.tp_partial_sum(parts, T * d, T_p, None, dx_all, T * d, S.TP_F32, S.TP_F32)
    torch.cuda.synchronize()
    full = O.ffn_shard_bwd(x, w1, None, w2, dy, 1, 0, act)["dx_t"]
    assert nerr(host64(dx_all), full) < BF16_TOL
