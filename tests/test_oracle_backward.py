"""Pins of the oracle's backward of the row-sharded products (FFN, out-projection; CPU only).

The pages give the f-g pattern ("7.9 Tensor and pipeline parallelism", section
2.1): the rank's input gradient is a partial sum that f all-reduces, the
weight gradients stay on the rank.  The derivative formulas themselves are
plain calculus, so they are pinned against things other than the oracle:
closed forms of the activation derivatives, central finite differences of the
forward oracle, PyTorch autograd in float64 on the CPU, and the sharding
identities (the ranks' gradients assemble into the unsharded gradients).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import tp_oracle as O

GATED = ("swiglu", "bilinear")
ACTS = ("none", "gelu", "swiglu", "bilinear")


def _case(T=3, d=4, d_ff=8, seed=0):
    r = np.random.default_rng(seed)
    x = r.standard_normal((T, d))
    w1 = r.standard_normal((d, d_ff)) * 0.7
    w3 = r.standard_normal((d, d_ff)) * 0.7
    w2 = r.standard_normal((d_ff, d)) * 0.5
    dy = r.standard_normal((T, d))
    return x, w1, w3, w2, dy


def _assemble(x, w1, w3, w2, dy, T_p, act):
    """Full gradients assembled from the T_p ranks: dX = sum_t dX(t), weight grads by block."""
    d_ff = w1.shape[1]
    dx = np.zeros_like(x)
    dw1 = np.zeros_like(w1)
    dw3 = np.zeros_like(w3)
    dw2 = np.zeros_like(w2)
    for t in range(T_p):
        b, n = O.shard_range(d_ff, T_p, t)
        g = O.ffn_shard_bwd(x, w1, w3, w2, dy, T_p, t, act)
        dx += g["dx_t"]
        dw1[:, b:b + n] = g["dw1"]
        dw2[b:b + n, :] = g["dw2"]
        if act in GATED:
            dw3[:, b:b + n] = g["dw3"]
    return dx, dw1, dw3, dw2


def _loss(x, w1, w3, w2, dy, act):
    """L = <y, dY> with y the unsharded forward oracle, so dL/d(anything) is what the backward returns."""
    return float(np.sum(O.ffn_unsharded(x, w1, w3, w2, act) * dy))


def test_activation_derivative_closed_forms():
    u = np.linspace(-6.0, 6.0, 97)
    # gelu(u) - gelu(-u) = u and silu(u) - silu(-u) = u, so the derivatives at u and -u sum to 1
    assert np.allclose(O.gelu_grad(u) + O.gelu_grad(-u), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(O.silu_grad(u) + O.silu_grad(-u), 1.0, rtol=0, atol=1e-14)
    assert abs(O.gelu_grad(np.array(0.0)) - 0.5) < 1e-15
    assert abs(O.silu_grad(np.array(0.0)) - 0.5) < 1e-15
    # gelu'(u) -> 1 (u -> +inf), -> 0 (u -> -inf); silu the same
    assert abs(O.gelu_grad(np.array(12.0)) - 1.0) < 1e-12 and abs(O.gelu_grad(np.array(-12.0))) < 1e-12
    assert abs(O.silu_grad(np.array(40.0)) - 1.0) < 1e-12 and abs(O.silu_grad(np.array(-40.0))) < 1e-12


@pytest.mark.parametrize("fn,grad", [("gelu", "gelu_grad"), ("silu", "silu_grad")])
def test_activation_derivative_matches_finite_differences(fn, grad):
    u = np.linspace(-5.0, 5.0, 41) + 0.013
    f = getattr(O, fn)
    h = 1e-5
    fd = (f(u + h) - f(u - h)) / (2 * h)
    assert np.max(np.abs(getattr(O, grad)(u) - fd)) < 1e-9


@pytest.mark.parametrize("act", ACTS)
def test_backward_matches_finite_differences(act):
    """Central differences of <y, dY> in every input, at a seeded sample of entries."""
    x, w1, w3, w2, dy = _case()
    dx, dw1, dw3, dw2 = _assemble(x, w1, w3, w2, dy, 2, act)
    r = np.random.default_rng(7)
    eps = 1e-6
    mats = [("x", x, dx), ("w1", w1, dw1), ("w2", w2, dw2)]
    if act in GATED:
        mats.append(("w3", w3, dw3))
    for name, m, g in mats:
        for _ in range(6):
            idx = tuple(int(r.integers(0, s)) for s in m.shape)
            keep = m[idx]
            m[idx] = keep + eps
            lp = _loss(x, w1, w3, w2, dy, act)
            m[idx] = keep - eps
            lm = _loss(x, w1, w3, w2, dy, act)
            m[idx] = keep
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, g[idx])


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("T_p", [1, 4])
def test_backward_matches_torch_autograd_fp64(act, T_p):
    x, w1, w3, w2, dy = _case(T=5, d=6, d_ff=12, seed=3)
    tx, t1, t3, t2 = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (x, w1, w3, w2))
    u = tx @ t1
    if act == "none":
        h = u
    elif act == "gelu":
        h = torch.nn.functional.gelu(u, approximate="none")
    elif act == "swiglu":
        h = torch.nn.functional.silu(u) * (tx @ t3)
    else:
        h = u * (tx @ t3)
    ((h @ t2) * torch.tensor(dy, dtype=torch.float64)).sum().backward()
    dx, dw1, dw3, dw2 = _assemble(x, w1, w3, w2, dy, T_p, act)
    for got, ref in [(dx, tx.grad), (dw1, t1.grad), (dw2, t2.grad)] + (
            [(dw3, t3.grad)] if act in GATED else []):
        ref = ref.numpy()
        assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_backward_sharding_identities_tp1_to_tp10(act):
    """Ranks' dX(t) sum to the unsharded dX; their weight gradients are the unsharded blocks."""
    x, w1, w3, w2, dy = _case(T=4, d=5, d_ff=2520, seed=11)
    full = O.ffn_shard_bwd(x, w1, w3, w2, dy, 1, 0, act)
    for T_p in range(1, 11):
        dx, dw1, dw3, dw2 = _assemble(x, w1, w3, w2, dy, T_p, act)
        assert np.max(np.abs(dx - full["dx_t"])) <= 1e-12 * np.max(np.abs(full["dx_t"]))
        assert np.max(np.abs(dw1 - full["dw1"])) <= 1e-12 * np.max(np.abs(full["dw1"]))
        assert np.max(np.abs(dw2 - full["dw2"])) <= 1e-12 * np.max(np.abs(full["dw2"]))
        if act in GATED:
            assert np.max(np.abs(dw3 - full["dw3"])) <= 1e-12 * np.max(np.abs(full["dw3"]))


def test_backward_single_rank_input_gradient_is_partial():
    """With T_p > 1 one rank's dX(t) alone is not dX: the f all-reduce is needed."""
    x, w1, w3, w2, dy = _case(T=4, d=5, d_ff=40, seed=5)
    full = O.ffn_shard_bwd(x, w1, w3, w2, dy, 1, 0, "gelu")["dx_t"]
    part = O.ffn_shard_bwd(x, w1, w3, w2, dy, 4, 1, "gelu")["dx_t"]
    assert np.max(np.abs(part - full)) > 1e-3 * np.max(np.abs(full))


def test_outproj_backward_matches_autograd_and_assembles():
    """dO(t) and dWo(t) against float64 autograd of a = O Wo, and the ranks' pieces against the
    unsharded gradients: dO(t) is rank t's head columns of dO, dWo(t) its head rows of dWo."""
    r = np.random.default_rng(21)
    T, d, H, dh, T_p = 7, 12, 8, 4, 4
    o = r.standard_normal((T, H * dh))
    wo = r.standard_normal((H * dh, d))
    dy = r.standard_normal((T, d))
    to = torch.tensor(o, requires_grad=True)
    tw = torch.tensor(wo, requires_grad=True)
    ((to @ tw) * torch.tensor(dy)).sum().backward()
    k = H * dh // T_p
    for t in range(T_p):
        g = O.attn_outproj_shard_bwd(o[:, t * k:(t + 1) * k], wo, dy, H, H // 2, dh, T_p, t)
        assert np.max(np.abs(g["do_t"] - to.grad.numpy()[:, t * k:(t + 1) * k])) < 1e-12
        assert np.max(np.abs(g["dwo"] - tw.grad.numpy()[t * k:(t + 1) * k])) < 1e-12
    # finite differences on one entry of Wo and one of O(t)
    eps = 1e-6
    g = O.attn_outproj_shard_bwd(o[:, k:2 * k], wo, dy, H, H // 2, dh, T_p, 1)
    wp, wm = wo.copy(), wo.copy()
    wp[k + 3, 5] += eps
    wm[k + 3, 5] -= eps
    fd = (np.sum((o @ wp) * dy) - np.sum((o @ wm) * dy)) / (2 * eps)
    assert abs(fd - g["dwo"][3, 5]) < 1e-7 * max(1.0, abs(fd))
