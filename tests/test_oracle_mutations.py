"""Planted mistakes in the CPU oracle must be caught by its pins.

Each case replaces one oracle function by a plausible wrong version (on the
CPU only) and checks that at least one pin test then fails.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest

import test_oracle_backward as bpins
import test_oracle_pins as pins
import test_oracle_ring as rpins
from oracle import analytic as A
from oracle import tp_oracle as O


def _wrong_silu_sign(u):
    u = np.asarray(u, dtype=np.float64)
    return u / (1.0 + np.exp(u))


def _tanh_gelu(u):
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * u * (1 + np.tanh(math.sqrt(2 / math.pi) * (u + 0.044715 * u ** 3)))


def _reversed_ranks(extent, T_p, t):
    n = extent // T_p
    if extent % T_p or not (0 <= t < T_p):
        raise ValueError
    return (T_p - 1 - t) * n, n


def _drop_last_partial(parts, residual=None):
    acc = np.zeros_like(np.asarray(parts[0], dtype=np.float64))
    for p in parts[:-1] if len(parts) > 1 else parts:
        acc = acc + p
    return acc if residual is None else acc + residual


_orig_attention = O.attention_head


def _unscaled_attention(q, k, v, causal=True, rows=None):
    """Drops the 1/sqrt(d_h) scale (pre-multiplying Q by sqrt(d_h) cancels it)."""
    q = np.asarray(q, dtype=np.float64)
    return _orig_attention(q * math.sqrt(q.shape[1]), k, v, causal, rows)


def _mask_diagonal_too(q, k, v, causal=True, rows=None):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, dh = q.shape
    idx = np.arange(T) if rows is None else np.asarray(rows)
    s = (q[idx] @ k.T) / math.sqrt(dh)
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] >= idx[:, None], -1e300, s)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p / p.sum(axis=1, keepdims=True)) @ v


def _transposed_w2(h, w2, rows):
    b, e = rows
    w = np.asarray(w2, dtype=np.float64)
    blk = w[b:e, :]
    if blk.shape[0] == blk.shape[1]:
        blk = blk.T
    else:
        blk = blk[::-1]
    return np.asarray(h, dtype=np.float64) @ blk


def _gelu_grad_cdf_only(u):
    """Drops the u*phi(u) term of gelu'."""
    from scipy import special
    return 0.5 * special.erfc(-np.asarray(u, dtype=np.float64) / math.sqrt(2.0))


def _silu_grad_sign(u):
    u = np.asarray(u, dtype=np.float64)
    s = 1.0 / (1.0 + np.exp(-u))
    return s * (1.0 + u * s)


_orig_act_backward = O.act_backward


def _swiglu_bwd_without_gate(dh, u, v, act):
    du, dv = _orig_act_backward(dh, u, v, act)
    if act == "swiglu":
        du = np.asarray(dh, dtype=np.float64) * O.silu_grad(u)
    return du, dv


_orig_ffn_shard_bwd = O.ffn_shard_bwd


def _dx_without_w3_term(x, w1, w3, w2, dy, T_p, t, act):
    g = dict(_orig_ffn_shard_bwd(x, w1, w3, w2, dy, T_p, t, act))
    if g["dv"] is not None:
        b, n = O.shard_range(w1.shape[1], T_p, t)
        g["dx_t"] = g["du"] @ np.asarray(w1[:, b:b + n], dtype=np.float64).T
    return g


def _dw2_from_preactivation(x, w1, w3, w2, dy, T_p, t, act):
    g = dict(_orig_ffn_shard_bwd(x, w1, w3, w2, dy, T_p, t, act))
    g["dw2"] = g["u"].T @ np.asarray(dy, dtype=np.float64)
    return g


_orig_ring = O.ring_attention_step


def _ring_chunk_alone(q, k, v, o_state, lse_state, q_pos0, k_pos0, causal):
    fresh = (np.zeros_like(np.asarray(o_state, dtype=np.float64)),
             np.full_like(np.asarray(lse_state, dtype=np.float64), -np.inf))
    return _orig_ring(q, k, v, *fresh, q_pos0, k_pos0, causal)


def _ring_drops_old_state(q, k, v, o_state, lse_state, q_pos0, k_pos0, causal=True):
    """The chunk's result replaces the state instead of merging with it."""
    o_c, l_c = _ring_chunk_alone(q, k, v, o_state, lse_state, q_pos0, k_pos0, causal)
    seen = np.isfinite(l_c)
    return np.where(seen[:, None], o_c, o_state), np.where(seen, l_c, lse_state)


def _ring_lse_max(q, k, v, o_state, lse_state, q_pos0, k_pos0, causal=True):
    """Keeps the larger log-denominator instead of the log of the summed weights."""
    o_c, l_c = _ring_chunk_alone(q, k, v, o_state, lse_state, q_pos0, k_pos0, causal)
    seen = np.isfinite(l_c)
    big = np.maximum(lse_state, l_c)
    big_f = np.where(np.isfinite(big), big, 0.0)
    o = np.exp(lse_state - big_f)[:, None] * o_state + np.exp(l_c - big_f)[:, None] * o_c
    return np.where(seen[:, None], o, o_state), np.where(seen, big, lse_state)


def _ring_masks_diagonal(q, k, v, o_state, lse_state, q_pos0, k_pos0, causal=True):
    """A query no longer sees the key at its own position."""
    return _orig_ring(q, k, v, o_state, lse_state, q_pos0 - 1, k_pos0, causal)


_orig_heads = O.attn_heads_shard


def _heads_truncated_kv(x, wq, wk, wv, n_heads, n_kv_heads, head_dim, T_p, t, causal=True,
                        rows=None, kv_replicate=False):
    """Cuts the keys and values after the last requested row even without the causal mask."""
    if rows is not None:
        x = np.asarray(x)[: int(np.max(rows)) + 1]
    return _orig_heads(x, wq, wk, wv, n_heads, n_kv_heads, head_dim, T_p, t, causal, rows,
                       kv_replicate)


def _interleaved_step_squared(stages, micro_batches, v):
    """Divides by v twice."""
    return A.bubble_fraction(stages, micro_batches) / (v * v)


MUTATIONS = [
    ("silu", _wrong_silu_sign, [lambda: pins.test_silu_closed_forms_and_library(),
                                lambda: pins.test_brute_force_tiny("swiglu", 2)]),
    ("gelu", _tanh_gelu, [lambda: pins.test_gelu_closed_forms_and_library(),
                          lambda: pins.test_brute_force_tiny("gelu", 1)]),
    ("shard_range", _reversed_ranks, [lambda: pins.test_brute_force_tiny("gelu", 2),
                                      lambda: pins.test_shard_range_blocks()]),
    ("partial_sum", _drop_last_partial, [lambda: pins.test_sum_of_partials_is_unsharded_ffn_tp1_to_tp11("gelu")]),
    ("attention_head", _unscaled_attention, [lambda: pins.test_attention_vs_library_sdpa(True)]),
    ("attention_head", _mask_diagonal_too, [lambda: pins.test_attention_special_cases(),
                                            lambda: pins.test_attention_brute_force()]),
    ("row_parallel", _transposed_w2, [lambda: pins.test_brute_force_tiny("none", 2)]),
    ("gelu_grad", _gelu_grad_cdf_only, [lambda: bpins.test_activation_derivative_matches_finite_differences(
        "gelu", "gelu_grad"), lambda: bpins.test_backward_matches_torch_autograd_fp64("gelu", 1)]),
    ("silu_grad", _silu_grad_sign, [lambda: bpins.test_activation_derivative_closed_forms(),
                                    lambda: bpins.test_backward_matches_finite_differences("swiglu")]),
    ("act_backward", _swiglu_bwd_without_gate, [lambda: bpins.test_backward_matches_finite_differences("swiglu"),
                                                lambda: bpins.test_backward_matches_torch_autograd_fp64("swiglu", 4)]),
    ("ffn_shard_bwd", _dx_without_w3_term, [lambda: bpins.test_backward_matches_finite_differences("bilinear")]),
    ("ffn_shard_bwd", _dw2_from_preactivation, [lambda: bpins.test_backward_matches_torch_autograd_fp64("gelu", 4)]),
    ("ring_attention_step", _ring_drops_old_state, [lambda: rpins.test_ring_equals_full_attention(2, True),
                                                    lambda: rpins.test_ring_step_brute_force_tiny()]),
    ("ring_attention_step", _ring_lse_max, [lambda: rpins.test_ring_zero_queries_closed_form(),
                                            lambda: rpins.test_ring_equals_full_attention(3, False)]),
    ("attn_heads_shard", _heads_truncated_kv, [lambda: pins.test_heads_shard_rows_equal_the_full_result_rows(False)]),
    ("ring_attention_step", _ring_masks_diagonal, [lambda: rpins.test_ring_zero_queries_closed_form(),
                                                   lambda: rpins.test_ring_equals_full_attention(4, True)]),
]


@pytest.mark.parametrize("name,wrong,checks", MUTATIONS,
                         ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, wrong, checks):
    monkeypatch.setattr(O, name, wrong)
    for check in checks:
        with pytest.raises((AssertionError, ValueError)):
            check()


def test_planted_interleaved_bubble_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(A, "bubble_interleaved_step", _interleaved_step_squared)
    with pytest.raises(AssertionError):
        pins.test_interleaved_bubble_forms_agree()


def _ring_bytes_one_pass(n_gpus, payload_bytes):
    """Planted mistake: only the reduce-scatter's (N-1)/N of the payload."""
    return Fraction(n_gpus - 1, n_gpus) * payload_bytes


def test_planted_ring_allreduce_bytes_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(A, "ring_allreduce_bytes_per_gpu", _ring_bytes_one_pass)
    for n in (2, 8):
        with pytest.raises(AssertionError):
            pins.test_ring_allreduce_bytes_by_simulation(n)
