"""The entry points allocate, free, synchronise and clear nothing themselves (every
output is written by a kernel), so a caller can capture them in a HIP graph.  A forward
step (two ranks' FFN shards and the partial sum with a residual), an attention sublayer
(two ranks' heads and out-projection shards, the sum with the residual) and a
ring-attention pass (set-up, two chunk folds, finish) are captured once and replayed
several times, with
eager work and synchronisation between the replays; every replay must match the eager
result bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from _gpu_util import dev, log, requires_gpu
from megatron_tensor_transformer_gemm_amd import inputs as I
from megatron_tensor_transformer_gemm_amd import tpshard as S

pytestmark = [pytest.mark.gpu, requires_gpu]
BF = S.TP_BF16


def _capture(fn):
    """Run fn once on a side stream (warm-up), then capture it into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("case", [(1000, 328, 1600, 2, "swiglu"), (2000, 5376, 6144, 2, "gelu"),
                                  (4100, 4104, 8208, 2, "swiglu")],
                         ids=["swiglu-small", "gelu-192-column-tiles", "swiglu-persistent"])
def test_forward_step_graph_replays_match_eager(case):
    """The second case runs the column GEMM split over k (fp32 partials in the workspace,
    then the reduce kernel with GELU) on 256 x 192 tiles, and the row GEMM on 256 x 192
    tiles with the LDS-staged bf16 epilogue.  The third has more 256 x 256 tiles than the
    GPU has CUs in both products (561 and 289): both run one workgroup per CU over several
    tiles each."""
    T, d, d_ff, T_p, act = case
    log(f"[graph] forward step T={T} d={d} d_ff={d_ff} T_p={T_p} {act}")
    c = I.small_ffn_case(41, T, d, d_ff, act, I.BF16)
    x, w1, w2 = (dev(c[k], I.BF16) for k in ("x", "w1", "w2"))
    w3 = dev(c["w3"], I.BF16) if "w3" in c else None
    res = dev(I.bf16_bits(np.random.default_rng(3).standard_normal((T, d)).astype(np.float32)), I.BF16)
    parts = torch.empty((T_p, T, d), dtype=torch.bfloat16, device="cuda:0")
    nb = S.tp_ffn_workspace_bytes(T, d_ff, T_p, BF)
    ws = [torch.empty(nb, dtype=torch.uint8, device="cuda:0") for _ in range(T_p)]
    y = torch.empty((T, d), dtype=torch.bfloat16, device="cuda:0")

    def step():
        for t in range(T_p):
            S.tp_ffn_shard_fwd(x, w1, w3, w2, parts[t], ws[t], nb, T, d, d_ff, T_p, t, act, BF, BF)
        S.tp_partial_sum(parts, T * d, T_p, res, y, T * d, BF, BF)

    step()
    torch.cuda.synchronize()
    ref_y, ref_parts = y.clone(), parts.clone()
    g = _capture(step)
    for i in range(3):
        y.fill_(float("nan"))
        parts.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(ref_y)), f"replay {i}: y differs"
        assert torch.equal(_bits(parts), _bits(ref_parts)), f"replay {i}: partials differ"


def test_ring_attention_graph_replays_match_eager():
    L, C, h_t, dh = 512, 2, 2, 128
    c = L // C
    log(f"[graph] ring attention L={L} C={C} h_t={h_t} dh={dh}")
    g0 = np.random.default_rng(8)
    q, k, v = (dev(I.bf16_bits(g0.standard_normal((L, h_t * dh)).astype(np.float32)), I.BF16)
               for _ in range(3))
    st = torch.empty((c, h_t * dh), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((c, h_t), dtype=torch.float32, device="cuda:0")
    o = torch.empty((c, h_t * dh), dtype=torch.bfloat16, device="cuda:0")
    kd = h_t * dh

    def ring():     # the last rank: its own chunk, then the one before
        S.tp_attn_ring_init(st, lse, c, h_t, dh, kd, h_t)
        for src in (1, 0):
            S.tp_attn_ring_step(q[c:], k[src * c:], v[src * c:], st, lse, 1, c, h_t, h_t, dh, kd, kd, kd,
                                h_t, c, src * c, True)
        S.tp_attn_ring_finish(st, o, c, h_t, dh, kd, kd)

    ring()
    torch.cuda.synchronize()
    ref = (o.clone(), st.clone(), lse.clone())
    g = _capture(ring)
    for i in range(3):
        for t in (o, st, lse):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((o, st, lse), ref):
            assert torch.equal(_bits(got), _bits(want)), f"replay {i} differs"


def test_attention_sublayer_graph_replays_match_eager():
    """Two ranks' tp_attn_heads_shard_fwd (the Q, K, V projection split over k: fp32
    partials in the workspace, then the reduce kernel; then the causal core) and
    tp_attn_outproj_shard_fwd, and the sum of their partials with the residual."""
    L, d, H, dh, T_p, ranks = 2048, 2048, 16, 128, 8, (0, 5)
    kd = H // T_p * dh
    log(f"[graph] attention sublayer L={L} d={d} H={H} T_p={T_p} ranks={ranks}")
    g0 = np.random.default_rng(21)
    x = dev(I.bf16_bits(g0.standard_normal((L, d)).astype(np.float32)), I.BF16)
    wq, wk, wv = (dev(I.bf16_bits((g0.standard_normal((d, H * dh)) * 0.02).astype(np.float32)), I.BF16)
                  for _ in range(3))
    wo = dev(I.bf16_bits((g0.standard_normal((H * dh, d)) * 0.02).astype(np.float32)), I.BF16)
    nb = S.tp_attn_heads_workspace_bytes(1, L, H, H, dh, T_p)
    assert nb > L * 3 * kd * 2, "this shape should get split-K scratch"
    ws = [torch.empty(nb, dtype=torch.uint8, device="cuda:0") for _ in ranks]
    o = [torch.empty((L, kd), dtype=torch.bfloat16, device="cuda:0") for _ in ranks]
    parts = torch.empty((len(ranks), L, d), dtype=torch.bfloat16, device="cuda:0")
    y = torch.empty((L, d), dtype=torch.bfloat16, device="cuda:0")

    def sub():
        for i, t in enumerate(ranks):
            S.tp_attn_heads_shard_fwd(x, wq, wk, wv, o[i], ws[i], nb, 1, L, d, H, H, dh, T_p, t, True)
            S.tp_attn_outproj_shard_fwd(o[i], wo, parts[i], L, d, H, H, dh, T_p, t, BF, BF)
        S.tp_partial_sum(parts, L * d, len(ranks), x, y, L * d, BF, BF)

    sub()
    torch.cuda.synchronize()
    ref = [y.clone(), parts.clone()] + [t.clone() for t in o]
    g = _capture(sub)
    for i in range(3):
        for t in [y, parts] + o:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip([y, parts] + o, ref):
            assert torch.equal(_bits(got), _bits(want)), f"replay {i} differs"
