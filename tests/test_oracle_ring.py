"""Pins of the oracle's ring-attention step (context parallelism; CPU only).

The pages describe the method ("7.9 Tensor and pipeline parallelism" section 6;
"Parallelism II: model", "Sequence and context parallelism"; "Tensor & Pipeline
Parallelism" (S17)): a device keeps its query chunk and folds in the key/value
chunks as they come round the ring, passing a FlashAttention-style running
state.  Its result is pinned by things other than the merge formula itself:
full attention over the whole sequence (its own pins elsewhere), closed forms
with all-zero queries, brute force on tiny inputs, and invariants.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import pytest

from oracle import tp_oracle as O


def _ring(q, k, v, C, rank, order=None, causal=True):
    """Rank `rank`'s state after folding in the chunks in `order` (default: ring order)."""
    L, dh = q.shape
    c = L // C
    o = np.zeros((c, v.shape[1]))
    lse = np.full(c, -np.inf)
    order = [(rank - s) % C for s in range(C)] if order is None else order
    for src in order:
        o, lse = O.ring_attention_step(q[rank * c:(rank + 1) * c], k[src * c:(src + 1) * c],
                                       v[src * c:(src + 1) * c], o, lse, rank * c, src * c, causal)
    return o, lse


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("C", [1, 2, 3, 4])
def test_ring_equals_full_attention(C, causal):
    r = np.random.default_rng(C + 10 * causal)
    L, dh = 24, 8
    q, k, v = (r.standard_normal((L, dh)) for _ in range(3))
    full = O.attention_head(q, k, v, causal=causal)
    c = L // C
    for rank in range(C):
        o, lse = _ring(q, k, v, C, rank, causal=causal)
        assert np.max(np.abs(o - full[rank * c:(rank + 1) * c])) < 1e-12


def test_ring_order_does_not_matter():
    r = np.random.default_rng(3)
    L, C = 16, 4
    q, k, v = (r.standard_normal((L, 4)) for _ in range(3))
    ref_o, ref_l = _ring(q, k, v, C, 3)
    for order in itertools.permutations(range(C)):
        o, lse = _ring(q, k, v, C, 3, order=list(order))
        assert np.max(np.abs(o - ref_o)) < 1e-12 and np.max(np.abs(lse - ref_l)) < 1e-12


def test_ring_zero_queries_closed_form():
    """q = 0: every visible key scores 0, so lse = ln(#visible keys) and O is the mean of the
    visible values.  Causal: the row at position p sees p + 1 keys."""
    r = np.random.default_rng(5)
    L, C = 20, 4
    c = L // C
    q = np.zeros((L, 6))
    k, v = r.standard_normal((L, 6)), r.standard_normal((L, 3))
    for rank in range(C):
        o, lse = _ring(q, k, v, C, rank)
        for i in range(c):
            p = rank * c + i
            assert abs(lse[i] - math.log(p + 1)) < 1e-13
            assert np.max(np.abs(o[i] - v[:p + 1].mean(axis=0))) < 1e-13
        o, lse = _ring(q, k, v, C, rank, causal=False)
        assert np.max(np.abs(lse - math.log(L))) < 1e-13
        assert np.max(np.abs(o - v.mean(axis=0))) < 1e-13


def test_ring_step_brute_force_tiny():
    """One step from a non-empty state, against explicit loops over the scores."""
    r = np.random.default_rng(9)
    dh = 3
    q, k, v = r.standard_normal((3, dh)), r.standard_normal((4, dh)), r.standard_normal((4, 2))
    o0, l0 = r.standard_normal((3, 2)), np.array([0.3, -1.2, -np.inf])
    q_pos0, k_pos0 = 5, 3     # query positions 5..7, key positions 3..6
    o, lse = O.ring_attention_step(q, k, v, o0, l0, q_pos0, k_pos0, causal=True)
    for i in range(3):
        ws, acc = [], np.zeros(2)
        for j in range(4):
            if k_pos0 + j <= q_pos0 + i:
                w = math.exp(sum(q[i, t] * k[j, t] for t in range(dh)) / math.sqrt(dh))
                ws.append(w)
                acc += w * v[j]
        z = sum(ws)
        old = math.exp(l0[i]) if np.isfinite(l0[i]) else 0.0
        assert abs(lse[i] - math.log(old + z)) < 1e-12
        assert np.max(np.abs(o[i] - (old * o0[i] + acc) / (old + z))) < 1e-12


def test_ring_rows_and_chunks_that_see_nothing_keep_the_state():
    r = np.random.default_rng(11)
    q, k, v = r.standard_normal((8, 4)), r.standard_normal((8, 4)), r.standard_normal((8, 4))
    o0, l0 = r.standard_normal((8, 4)), r.standard_normal(8)
    # whole key chunk after the queries
    o, lse = O.ring_attention_step(q, k, v, o0, l0, 0, 8, causal=True)
    assert np.array_equal(o, o0) and np.array_equal(lse, l0)
    # keys at positions 4..11 against queries 0..7: rows 0..3 see nothing
    o, lse = O.ring_attention_step(q, k, v, o0, l0, 0, 4, causal=True)
    assert np.array_equal(o[:4], o0[:4]) and np.array_equal(lse[:4], l0[:4])
    assert np.all(lse[4:] > l0[4:])       # each seen key adds a positive term to the sum


def test_ring_two_halves_of_a_chunk_equal_the_chunk():
    """Folding a chunk in as two halves gives the state of folding it in whole."""
    r = np.random.default_rng(13)
    q, k, v = r.standard_normal((6, 4)), r.standard_normal((10, 4)), r.standard_normal((10, 5))
    o0, l0 = np.zeros((6, 5)), np.full(6, -np.inf)
    whole = O.ring_attention_step(q, k, v, o0, l0, 9, 0, causal=True)
    half = O.ring_attention_step(q, k[:5], v[:5], o0, l0, 9, 0, causal=True)
    half = O.ring_attention_step(q, k[5:], v[5:], *half, 9, 5, causal=True)
    assert np.max(np.abs(whole[0] - half[0])) < 1e-12 and np.max(np.abs(whole[1] - half[1])) < 1e-12
