"""Pins of the CPU oracle against what the pages and the mathematics fix.

No GPU.  Each test checks the oracle against something other than itself:
the sharded/unsharded identity of the column-then-row split, brute-force
loops, textbook closed forms and independent library routines, attention
special cases, and the values the pages print.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy import special

import _brute
from oracle import analytic
from oracle import tp_oracle as O

ACTS = ["none", "gelu", "swiglu", "bilinear"]


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _ffn_inputs(T, d, d_ff, seed):
    return (_rand((T, d), seed), _rand((d, d_ff), seed + 1, 1 / math.sqrt(d)),
            _rand((d, d_ff), seed + 2, 1 / math.sqrt(d)), _rand((d_ff, d), seed + 3, 1 / math.sqrt(d_ff)))


# ----------------------------------------------------------------------------- P1, P2
@pytest.mark.parametrize("act", ACTS)
def test_sum_of_partials_is_unsharded_ffn_tp1_to_tp11(act):
    """Sum over ranks of y(t) equals the unsharded sublayer, T_p = 1..11 (d_ff = lcm(1..11))."""
    T, d, d_ff = 3, 4, 27720
    x, w1, w3, w2 = _ffn_inputs(T, d, d_ff, 11)
    full = O.ffn_unsharded(x, w1, w3, w2, act)
    for T_p in range(1, 12):
        parts = [O.ffn_shard(x, w1, w3, w2, T_p, t, act)[1] for t in range(T_p)]
        y = O.partial_sum(parts)
        assert O.normwise_max_rel_err(y, full) <= 1e-12, (act, T_p)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_tp1_reproduces_full_layer(act):
    x, w1, w3, w2 = _ffn_inputs(5, 8, 16, 3)
    h, y0 = O.ffn_shard(x, w1, w3, w2, 1, 0, act)
    assert h.shape == (5, 16)
    np.testing.assert_allclose(y0, O.ffn_unsharded(x, w1, w3, w2, act), rtol=0, atol=1e-13)


# ----------------------------------------------------------------------------- P3, P4
@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_activation_commutes_with_column_split(act):
    x, w1, w3, w2 = _ffn_inputs(6, 8, 32, 5)
    h_full = O.column_parallel(x, w1, w3, (0, 32), act)
    for T_p in (2, 4, 8):
        for t in range(T_p):
            b, n = O.shard_range(32, T_p, t)
            np.testing.assert_allclose(O.column_parallel(x, w1, w3, (b, b + n), act),
                                       h_full[:, b:b + n], rtol=0, atol=1e-14)


def test_row_split_of_w1_does_not_commute():
    """The 'bad option': splitting W1 by rows would need a sum before the non-linearity."""
    x, w1, _, _ = _ffn_inputs(6, 8, 32, 9)
    u1 = x[:, :4] @ w1[:4]
    u2 = x[:, 4:] @ w1[4:]
    good = O.gelu(u1 + u2)
    bad = O.gelu(u1) + O.gelu(u2)
    assert np.max(np.abs(good - bad)) > 1e-2
    np.testing.assert_allclose(good, O.column_parallel(x, w1, None, (0, 32), "gelu"), atol=1e-14)


# ----------------------------------------------------------------------------- P5 brute force
@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("T_p", [1, 2, 4])
def test_brute_force_tiny(act, T_p):
    T, d, d_ff = 3, 4, 8
    x, w1, w3, w2 = _ffn_inputs(T, d, d_ff, 21 + T_p)
    L = lambda a: a.tolist()  # noqa: E731
    for t in range(T_p):
        h, y = O.ffn_shard(x, w1, w3, w2, T_p, t, act)
        hb, yb = _brute.ffn_rank(L(x), L(w1), L(w3), L(w2), T_p, t, act)
        np.testing.assert_allclose(h, np.array(hb), rtol=0, atol=1e-12)
        np.testing.assert_allclose(y, np.array(yb), rtol=0, atol=1e-12)


def test_shard_range_blocks():
    assert O.shard_range(14336, 8, 0) == (0, 1792)
    assert O.shard_range(14336, 8, 7) == (7 * 1792, 1792)
    assert O.shard_range(28672, 8, 3) == (3 * 3584, 3584)
    covered = []
    for t in range(11):
        b, n = O.shard_range(27720, 11, t)
        covered.extend(range(b, b + n))
    assert covered == list(range(27720))
    for bad in [(10, 3, 0), (8, 2, 2), (8, 2, -1), (8, 0, 0)]:
        with pytest.raises(ValueError):
            O.shard_range(*bad)


# ----------------------------------------------------------------------------- P6 activations
def test_gelu_closed_forms_and_library():
    u = np.linspace(-12, 12, 4801)
    g = O.gelu(u)
    assert O.gelu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(g - O.gelu(-u), u, rtol=0, atol=1e-13)       # u*Phi(u) - (-u)Phi(-u) = u
    np.testing.assert_allclose(g, u * special.ndtr(u), rtol=1e-13, atol=1e-300)
    assert O.gelu(np.array([40.0]))[0] == 40.0                               # Phi(40) = 1 in fp64
    assert abs(O.gelu(np.array([-40.0]))[0]) < 1e-300
    # Phi(1) from the standard normal table: 0.8413447460685429
    assert abs(O.gelu(np.array([1.0]))[0] - 0.8413447460685429) < 1e-15


def test_silu_closed_forms_and_library():
    u = np.linspace(-30, 30, 6001)
    s = O.silu(u)
    np.testing.assert_allclose(s - O.silu(-u), u, rtol=0, atol=1e-12)
    np.testing.assert_allclose(s, u * special.expit(u), rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert abs(O.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16


# ----------------------------------------------------------------------------- attention
def test_attention_special_cases():
    rng = np.random.default_rng(4)
    T, dh = 9, 16
    q, k, v = rng.standard_normal((3, T, dh))
    o = O.attention_head(q, k, v, causal=True)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-15)               # row 0 sees only key 0
    o0 = O.attention_head(np.zeros_like(q), k, v, causal=True)               # uniform weights
    prefix_mean = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None]
    np.testing.assert_allclose(o0, prefix_mean, rtol=0, atol=1e-14)
    ones = O.attention_head(q, k, np.ones_like(v), causal=True)              # rows of P sum to 1
    np.testing.assert_allclose(ones, 1.0, rtol=0, atol=1e-14)
    o_nc = O.attention_head(np.zeros_like(q), k, v, causal=False)
    np.testing.assert_allclose(o_nc, np.broadcast_to(v.mean(axis=0), v.shape), atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_attention_vs_library_sdpa(causal):
    rng = np.random.default_rng(8)
    T, dh = 33, 32
    q, k, v = rng.standard_normal((3, T, dh)) * 2.0
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], is_causal=causal)[0, 0].numpy()
    np.testing.assert_allclose(O.attention_head(q, k, v, causal=causal), ref, rtol=0, atol=1e-12)
    rows = np.array([0, 5, 17, 32])
    np.testing.assert_allclose(O.attention_head(q, k, v, causal=causal, rows=rows), ref[rows],
                               rtol=0, atol=1e-12)


def test_attention_brute_force():
    rng = np.random.default_rng(12)
    q, k, v = rng.standard_normal((3, 5, 3))
    ref = _brute.attention(q.tolist(), k.tolist(), v.tolist(), causal=True)
    np.testing.assert_allclose(O.attention_head(q, k, v), np.array(ref), rtol=0, atol=1e-14)


@pytest.mark.parametrize("n_heads,n_kv", [(4, 4), (8, 2)])
def test_head_sharded_attention_equals_full_multihead(n_heads, n_kv):
    """Concatenating every rank's O(t) gives the unsharded multi-head output; the
    sum of the row-sharded projections gives the full O . Wo."""
    rng = np.random.default_rng(15)
    T, d, dh = 7, 12, 4
    x = rng.standard_normal((T, d))
    wq = rng.standard_normal((d, n_heads * dh)) / math.sqrt(d)
    wk = rng.standard_normal((d, n_kv * dh)) / math.sqrt(d)
    wv = rng.standard_normal((d, n_kv * dh)) / math.sqrt(d)
    wo = rng.standard_normal((n_heads * dh, d)) / math.sqrt(n_heads * dh)
    heads = []
    g = n_heads // n_kv
    for j in range(n_heads):
        kv = j // g
        heads.append(_brute.attention((x @ wq[:, j * dh:(j + 1) * dh]).tolist(),
                                      (x @ wk[:, kv * dh:(kv + 1) * dh]).tolist(),
                                      (x @ wv[:, kv * dh:(kv + 1) * dh]).tolist()))
    o_full = np.concatenate([np.array(h) for h in heads], axis=1)
    for T_p in (1, 2):
        if n_kv % T_p:
            continue
        o_parts = [O.attn_heads_shard(x, wq, wk, wv, n_heads, n_kv, dh, T_p, t) for t in range(T_p)]
        np.testing.assert_allclose(np.concatenate(o_parts, axis=1), o_full, atol=1e-13)
        a = O.partial_sum([O.attn_outproj_shard(o_parts[t], wo, n_heads, n_kv, dh, T_p, t)
                           for t in range(T_p)])
        np.testing.assert_allclose(a, o_full @ wo, atol=1e-13)


def test_block_sharded_equals_unsharded_and_rows():
    rng = np.random.default_rng(19)
    T, d, dh, H, d_ff = 6, 16, 4, 4, 32
    w = {"wq": rng.standard_normal((d, H * dh)) * 0.3, "wk": rng.standard_normal((d, H * dh)) * 0.3,
         "wv": rng.standard_normal((d, H * dh)) * 0.3, "wo": rng.standard_normal((H * dh, d)) * 0.3,
         "w1": rng.standard_normal((d, d_ff)) * 0.3, "w2": rng.standard_normal((d_ff, d)) * 0.3}
    x = rng.standard_normal((T, d))
    x1_ref, y_ref = O.block_sequence(x, w, H, H, dh, 1)
    # unsharded, written out directly: attention over all heads, then FFN, with residuals
    att = np.concatenate([np.array(_brute.attention((x @ w["wq"][:, j * dh:(j + 1) * dh]).tolist(),
                                                    (x @ w["wk"][:, j * dh:(j + 1) * dh]).tolist(),
                                                    (x @ w["wv"][:, j * dh:(j + 1) * dh]).tolist()))
                          for j in range(H)], axis=1)
    x1 = x + att @ w["wo"]
    u = x1 @ w["w1"]
    y = x1 + (0.5 * u * (1 + special.erf(u / math.sqrt(2)))) @ w["w2"]
    np.testing.assert_allclose(x1_ref, x1, atol=1e-12)
    np.testing.assert_allclose(y_ref, y, atol=1e-12)
    for T_p in (2, 4):
        x1_t, y_t = O.block_sequence(x, w, H, H, dh, T_p)
        np.testing.assert_allclose(y_t, y, atol=1e-12)
    rows = np.array([0, 3, 5])
    x1_r, y_r = O.block_sequence(x, w, H, H, dh, 2, rows=rows)
    np.testing.assert_allclose(y_r, y[rows], atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_heads_shard_rows_equal_the_full_result_rows(causal):
    """Restricting the computed query rows changes nothing but which rows come back: a
    causal row i still sees keys 0..i, and a row without the mask sees every key, so rows
    taken from the start, the middle and the end equal those rows of the full O(t)."""
    rng = np.random.default_rng(29)
    T, d, dh, H = 9, 12, 4, 4
    x = rng.standard_normal((T, d))
    wq, wk, wv = (rng.standard_normal((d, H * dh)) / math.sqrt(d) for _ in range(3))
    for T_p in (1, 2):
        for t in range(T_p):
            full = O.attn_heads_shard(x, wq, wk, wv, H, H, dh, T_p, t, causal=causal)
            for rows in ([0, 3], [2, 5, 8], [4], [0]):
                got = O.attn_heads_shard(x, wq, wk, wv, H, H, dh, T_p, t, causal=causal,
                                         rows=np.array(rows))
                np.testing.assert_allclose(got, full[rows], rtol=0, atol=1e-13)


@pytest.mark.parametrize("n_heads,n_kv,T_p", [(16, 2, 4), (16, 2, 8), (8, 1, 8), (16, 4, 2)])
def test_kv_replicated_shards_equal_full_gqa(n_heads, n_kv, T_p):
    """With T_p above the KV heads (each KV head replicated on T_p / n_kv ranks), the ranks'
    O(t) concatenate to the unsharded grouped-query output written out by brute force; with
    T_p dividing n_kv the replicated reading is the plain head shard."""
    rng = np.random.default_rng(23)
    T, d, dh = 6, 10, 4
    x = rng.standard_normal((T, d))
    wq = rng.standard_normal((d, n_heads * dh)) / math.sqrt(d)
    wk = rng.standard_normal((d, n_kv * dh)) / math.sqrt(d)
    wv = rng.standard_normal((d, n_kv * dh)) / math.sqrt(d)
    g = n_heads // n_kv
    heads = [np.array(_brute.attention((x @ wq[:, j * dh:(j + 1) * dh]).tolist(),
                                       (x @ wk[:, (j // g) * dh:(j // g + 1) * dh]).tolist(),
                                       (x @ wv[:, (j // g) * dh:(j // g + 1) * dh]).tolist()))
             for j in range(n_heads)]
    o_full = np.concatenate(heads, axis=1)
    parts = [O.attn_heads_shard(x, wq, wk, wv, n_heads, n_kv, dh, T_p, t, kv_replicate=True)
             for t in range(T_p)]
    np.testing.assert_allclose(np.concatenate(parts, axis=1), o_full, atol=1e-13)
    if n_kv % T_p == 0:
        assert O.head_shard_kv_replicated(n_heads, n_kv, dh, T_p, 1) == O.head_shard(n_heads, n_kv, dh, T_p, 1)
    else:
        hs = O.head_shard_kv_replicated(n_heads, n_kv, dh, T_p, T_p - 1)
        assert hs["kv_t"] == 1 and hs["kv_cols"] == ((n_kv - 1) * dh, n_kv * dh)


def test_kv_replication_needs_an_even_multiple():
    """Llama-3-70B-shaped 64 query / 8 KV heads: TP16 works by replicating each KV head on 2
    ranks; 6 KV heads cannot be spread evenly over 16 ranks."""
    hs = O.head_shard_kv_replicated(64, 8, 128, 16, 5)
    assert hs["h_t"] == 4 and hs["kv_cols"] == (2 * 128, 3 * 128) and hs["q_cols"] == (5 * 512, 6 * 512)
    with pytest.raises(ValueError, match="replicate"):
        O.head_shard_kv_replicated(48, 6, 128, 16, 0)


def test_gqa_divisibility():
    with pytest.raises(ValueError, match="n_kv_heads"):
        O.head_shard(64, 8, 128, 16, 0)
    with pytest.raises(ValueError, match="n_heads="):
        O.head_shard(48, 48, 128, 5, 0)
    hs = O.head_shard(64, 8, 128, 8, 3)
    assert hs["q_cols"] == (3 * 1024, 4 * 1024) and hs["kv_cols"] == (384, 512)
    assert hs["o_rows"] == (3072, 4096)


# ----------------------------------------------------------------------------- printed values
def _golden_rows():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "pages_printed_values.txt")
    rows = []
    with open(path) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            parts = [p.strip() for p in line.split(" | ")]
            rows.append(parts)
    return rows


def _eval_golden(fn, args):
    if fn == "tp_decode_comm_mib":
        layers, batch, d, n = args
        return float(analytic.tp_decode_comm_bytes_per_step(layers, batch, d, n)) / 2 ** 20
    if fn == "weight_gib_per_device":
        p_billion, b, tp = args
        return analytic.weight_bytes_per_device(p_billion * 1e9, b, tp) / 2 ** 30
    if fn == "weight_gb_per_device":
        p_billion, b, tp = args
        return analytic.weight_bytes_per_device(p_billion * 1e9, b, tp) / 1e9
    return getattr(analytic, fn)(*args)


@pytest.mark.parametrize("row", _golden_rows(), ids=lambda r: r[0])
def test_pages_printed_values(row):
    name, fn, args, printed, tol, _cite = row
    args = [int(a) for a in args.split()]
    got = _eval_golden(fn, args)
    if tol == "exact":
        if "/" in printed:
            assert got == Fraction(printed), name
        else:
            assert got == int(printed), name
    else:
        assert abs(float(got) - float(printed)) <= float(tol) + 1e-12, (name, float(got))


def test_bubble_four_stages_eight_micro_batches():
    assert analytic.bubble_fraction(4, 8) == Fraction(3, 11)
    # the two normalisations describe the same idle time
    assert analytic.bubble_vs_useful(4, 8) * 8 == analytic.bubble_fraction(4, 8) * 11


def test_interleaved_bubble_forms_agree():
    """The two pages print the interleaved bubble in two normalisations: per whole step,
    (1/v) (P-1)/(M+P-1) ("7.9 ...", section 3.4), and per useful work, (p-1)/(v m)
    ("Parallelism II: model", "Pipeline parallelism", whose 18.8 % and 9.4 % pin the
    latter through the printed-value table).  The step form is the useful form times the
    share M/(M+P-1) of a plain schedule's slots that do useful work, i.e. times
    1 - bubble_fraction; with v = 1 it is the plain bubble, 3/11 for 4 stages and 8
    micro-batches, about 18 % for P = 8, M = 32 and about 47 % for P = 8, M = 8 (3.2)."""
    for P in range(1, 10):
        for M in range(1, 40):
            for v in (1, 2, 3, 4, 8):
                step = analytic.bubble_interleaved_step(P, M, v)
                useful = analytic.bubble_interleaved_useful(P, M, v)
                assert step == useful * (1 - analytic.bubble_fraction(P, M)), (P, M, v)
                assert step <= analytic.bubble_fraction(P, M)
    assert analytic.bubble_interleaved_step(4, 8, 1) == Fraction(3, 11)
    assert abs(float(analytic.bubble_interleaved_step(8, 32, 1)) - 0.18) <= 0.005
    assert abs(float(analytic.bubble_interleaved_step(8, 8, 1)) - 0.47) <= 0.005
    # p5's printed interleaved values, carried over to the step form
    assert analytic.bubble_interleaved_step(4, 8, 2) == Fraction(3, 22)
    assert analytic.bubble_interleaved_step(4, 8, 4) == Fraction(3, 44)


@pytest.mark.parametrize("T_p", [1, 2, 4, 8])
def test_reduce_scatter_rows_gather_to_the_all_reduce(T_p):
    """The ranks' reduce-scatter rows, gathered in rank order, are the all-reduce's sum
    (the same bytes split in two steps, "Parallelism II: model"); T_p must divide T."""
    r = np.random.default_rng(17)
    T, d = 24, 5
    parts = [r.standard_normal((T, d)) for _ in range(T_p)]
    res = r.standard_normal((T, d))
    full = O.partial_sum(parts, res)
    m = T // T_p
    got = np.concatenate([O.reduce_scatter_rows(parts, T_p, t, res[t * m:(t + 1) * m]) for t in range(T_p)])
    assert np.max(np.abs(got - full)) <= 1e-13
    if T_p > 1:
        with pytest.raises(ValueError):
            O.reduce_scatter_rows([p[:T - 1] for p in parts], T_p, 0)


@pytest.mark.parametrize("n", [2, 3, 4, 8])
def test_ring_allreduce_bytes_by_simulation(n):
    """S17 "Mechanics": a ring all-reduce over N GPUs moves 2(N-1)/N times the payload per
    GPU.  Pinned by running one: a reduce-scatter (at step s GPU g passes its partial of
    chunk g-s to GPU g+1, which adds it) then an all-gather (GPU g passes its finished chunk
    g+1-s on), on integer vectors.  Every GPU must end with the exact sum, and each must
    have sent exactly the bytes the formula gives."""
    rng = np.random.default_rng(100 + n)
    data = [rng.integers(-9, 10, 6 * n).astype(np.int64) for _ in range(n)]
    chunks = [np.array_split(v.copy(), n) for v in data]
    sent = [0] * n
    for s in range(n - 1):     # reduce-scatter; messages of one step leave together
        msgs = [(g, (g - s) % n, chunks[g][(g - s) % n].copy()) for g in range(n)]
        for g, c, m in msgs:
            chunks[(g + 1) % n][c] = chunks[(g + 1) % n][c] + m
            sent[g] += m.nbytes
    for s in range(n - 1):     # all-gather of the finished chunks
        msgs = [(g, (g + 1 - s) % n, chunks[g][(g + 1 - s) % n].copy()) for g in range(n)]
        for g, c, m in msgs:
            chunks[(g + 1) % n][c] = m
            sent[g] += m.nbytes
    total = np.sum(data, axis=0)
    for g in range(n):
        assert np.array_equal(np.concatenate(chunks[g]), total)
        assert sent[g] == analytic.ring_allreduce_bytes_per_gpu(n, data[0].nbytes)
