"""Element-wise pins of the fused activation epilogues, forward and backward.

The column product H(t) = sigma(X W1(t)) [* X W3(t)] ("7.9 Tensor and pipeline
parallelism", section 2.1, the equation for h^(t); "Tensor & Pipeline Parallelism"
(S17), "Core idea": silu(x @ w1) * (x @ w3)) applies its activation on the GPU to the
fp32 accumulators and rounds once to bf16.  With activation_grid_case the
pre-activations U (and V) are exactly every bf16 value in [-12, 12] (GELU's far tail
included), so every element of H can be compared with the float64 oracle rounded to
bf16: the two may differ only where the kernel's fp32 value and the exact one fall on
either side of a bf16 rounding boundary, i.e. by at most one bf16 step.  The backward's
dU (and dV) are pinned the same way, with dH = dY W2(t)^T exact and the derivative
evaluated at the saved bf16 U, V.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from _gpu_util import dev, f64, host64, log, requires_gpu
from megatron_tensor_transformer_gemm_amd import inputs as I
from megatron_tensor_transformer_gemm_amd import tpshard as S
from oracle import tp_oracle as O

pytestmark = [pytest.mark.gpu, requires_gpu]


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _ordered(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> integers in the order of the values they encode (+0 = -0)."""
    b = bits.astype(np.int64)
    return np.where(b < 0x8000, b, -(b & 0x7FFF))


def _rne_bf16(ref: np.ndarray) -> np.ndarray:
    return I.bf16_bits(np.asarray(ref, dtype=np.float64).astype(np.float32))


def _assert_within_one_step(got: torch.Tensor, ref: np.ndarray, what: str):
    g, r = _ordered(_bits(got)), _ordered(_rne_bf16(ref))
    diff = np.abs(g - r)
    worst = int(diff.max())
    log(f"   {what}: {np.count_nonzero(diff)} of {diff.size} elements one bf16 step apart, "
        f"largest difference {worst} steps")
    assert worst <= 1, f"{what}: {np.count_nonzero(diff > 1)} elements more than one bf16 step off"


def _case(T, n, T_p):
    c = I.activation_grid_case(T, n, T_p)
    d = {k: dev(v, I.BF16) for k, v in c.items()}
    h = {k: f64(v, I.BF16) for k, v in c.items()}
    return c, d, h


SHAPES = [(1000, 256, 2, None), (4160, 4096, 2, 1)]
SHAPE_IDS = ["small-tiles-both-ranks", "256x256-tiles-rank1"]


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
def test_forward_epilogue_elementwise(act, shape):
    """tp_ffn_shard_fwd (H staged through LDS, then row segments stored) and
    tp_ffn_shard_fwd_train (H, U, V stored from the registers on small tiles, staged through
    LDS one after another on 8-wave 256 x 256 tiles): every H element within one bf16 step
    of the oracle; U, V equal the chosen pre-activations; y(t) = [H | 0]."""
    T, n, T_p, only = shape
    d, d_ff = 2 * n, T_p * n
    log(f"[epilogue-fwd] act={act} T={T} n={n} T_p={T_p}")
    c, dd, hh = _case(T, n, T_p)
    w3d = dd["w3"] if act == "swiglu" else None
    u_ref, v_ref = hh["x"][:, :n], hh["x"][:, n:]
    h_ref = O.gelu(u_ref) if act == "gelu" else O.silu(u_ref) * v_ref
    assert np.array_equal(O.column_parallel(hh["x"], hh["w1"], hh["w3"], (0, n), act), h_ref)
    ranks = range(T_p) if only is None else [only]
    for t in ranks:
        nb = S.tp_ffn_workspace_bytes(T, d_ff, T_p, S.TP_BF16)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
        y = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device="cuda:0")
        S.tp_ffn_shard_fwd(dd["x"], dd["w1"], w3d, dd["w2"], y, ws, nb, T, d, d_ff, T_p, t, act,
                           S.TP_BF16, S.TP_BF16)
        torch.cuda.synchronize()
        h = ws[: T * n * 2].view(torch.bfloat16).view(T, n)
        _assert_within_one_step(h, h_ref, f"H({t}) staged")
        assert torch.equal(y[:, :n], h) and not torch.any(y[:, n:] != 0), "y(t) is not [H | 0]"

        yt = torch.empty((T, d), dtype=torch.bfloat16, device="cuda:0")
        h2, u2 = (torch.empty((T, n), dtype=torch.bfloat16, device="cuda:0") for _ in range(2))
        v2 = torch.empty((T, n), dtype=torch.bfloat16, device="cuda:0") if act == "swiglu" else None
        S.tp_ffn_shard_fwd_train(dd["x"], dd["w1"], w3d, dd["w2"], yt, h2, u2, v2, T, d, d_ff,
                                 T_p, t, act, S.TP_BF16)
        torch.cuda.synchronize()
        _assert_within_one_step(h2, h_ref, f"H({t}) of the training forward")
        assert np.array_equal(host64(u2), u_ref), "saved U is not the pre-activation"
        if v2 is not None:
            assert np.array_equal(host64(v2), v_ref), "saved V is not the gate"
        # GELU's negative tail is checked on its own, relative to its own size
        if act == "gelu":
            tail = u_ref <= -3.0
            assert np.count_nonzero(tail) > 1000
            rel = np.abs(host64(h)[tail] - h_ref[tail]) / np.abs(h_ref[tail])
            log(f"   GELU tail u <= -3: {np.count_nonzero(tail)} elements, max relative "
                f"error {rel.max():.2e}")
            assert rel.max() <= 2.0 ** -7


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
@pytest.mark.parametrize("shape", [(1000, 256, 2, None), (4100, 1032, 2, 1), (4160, 4096, 1, 0),
                                   (4096, 4096, 1, 0)],
                         ids=["small-tiles-both-ranks", "large-tiles-rank1", "128x256-tiles",
                              "256x256-tiles"])
def test_backward_epilogue_elementwise(act, shape):
    """tp_ffn_shard_bwd's dU (and dV), which it leaves in its workspace: dH = dY W2(t)^T
    is exactly dy[:, :n], so every element is the derivative formula at the saved bf16
    U, V times an exact dH; within one bf16 step of the oracle's act_backward.  The dH
    product's tiles: 128 x 128 (first two shapes) and 128 x 256 (8 waves; U, V loaded
    before the k-loop) stage the epilogue through LDS; 256 x 256 stages it for GELU and
    keeps direct accesses for SwiGLU (U and V of all waves do not fit in LDS)."""
    T, n, T_p, only = shape
    d, d_ff = 2 * n, T_p * n
    log(f"[epilogue-bwd] act={act} T={T} n={n} T_p={T_p}")
    c, dd, hh = _case(T, n, T_p)
    gated = act == "swiglu"
    w3d = dd["w3"] if gated else None
    ranks = range(T_p) if only is None else [only]
    for t in ranks:
        yt = torch.empty((T, d), dtype=torch.bfloat16, device="cuda:0")
        h, u = (torch.empty((T, n), dtype=torch.bfloat16, device="cuda:0") for _ in range(2))
        v = torch.empty((T, n), dtype=torch.bfloat16, device="cuda:0") if gated else None
        S.tp_ffn_shard_fwd_train(dd["x"], dd["w1"], w3d, dd["w2"], yt, h, u, v, T, d, d_ff, T_p, t,
                                 act, S.TP_BF16)
        nb = S.tp_ffn_bwd_workspace_bytes(T, d_ff, T_p, act)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
        dx = torch.empty((T, d), dtype=torch.float32, device="cuda:0")
        dw1 = torch.empty((d, d_ff), dtype=torch.float32, device="cuda:0")
        dw3 = torch.empty((d, d_ff), dtype=torch.float32, device="cuda:0") if gated else None
        dw2 = torch.empty((d_ff, d), dtype=torch.float32, device="cuda:0")
        S.tp_ffn_shard_bwd(dd["x"], dd["w1"], w3d, dd["w2"], dd["dy"], h, u, v, dx, dw1, dw3, dw2,
                           ws, nb, T, d, d_ff, T_p, t, act, S.TP_F32, S.TP_F32)
        torch.cuda.synchronize()
        plane = nb // 2 if gated else nb
        du = ws[: T * n * 2].view(torch.bfloat16).view(T, n)
        u_ref, v_ref = hh["x"][:, :n], (hh["x"][:, n:] if gated else None)
        assert np.array_equal(host64(u), u_ref)
        dh = hh["dy"][:, :n]
        du_ref, dv_ref = O.act_backward(dh, u_ref, v_ref, act)
        _assert_within_one_step(du, du_ref, f"dU({t})")
        if gated:
            dv = ws[plane: plane + T * n * 2].view(torch.bfloat16).view(T, n)
            _assert_within_one_step(dv, dv_ref, f"dV({t})")
