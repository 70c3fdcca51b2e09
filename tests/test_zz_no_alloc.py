"""The allocation-free FFN entry point against the one that takes a workspace.

tp_ffn_shard_fwd_noalloc runs the same two kernels as tp_ffn_shard_fwd with H(t) in the
library's own per-GPU scratch, so its y(t) must equal tp_ffn_shard_fwd's bit for bit.
Two calls in a row, the second smaller (the scratch keeps the first call's H(t), which
the second overwrites in part), then the oracle on sampled rows of both.
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

CALLS = [
    # T, d, d_ff, T_p, t, act, out dtype
    (3000, 1024, 4096, 4, 1, "swiglu", S.TP_BF16),
    (700, 512, 2048, 2, 1, "gelu", S.TP_F32),
]


def _inputs(T, d, d_ff, act, seed):
    c = I.small_ffn_case(seed, T, d, d_ff, act, I.BF16)
    gated = act == "swiglu"
    devs = {k: dev(v, I.BF16) for k, v in c.items() if k != "dy" and (gated or k != "w3")}
    return c, devs


def test_noalloc_equals_workspace_entry_point_twice():
    outs = []
    for i, (T, d, d_ff, T_p, t, act, odt) in enumerate(CALLS):
        log(f"[noalloc] call {i}: T={T} d={d} d_ff={d_ff} T_p={T_p} t={t} act={act}")
        c, dv = _inputs(T, d, d_ff, act, 900 + i)
        tdt = torch.float32 if odt == S.TP_F32 else torch.bfloat16
        y_ref = torch.full((T, d), float("nan"), dtype=tdt, device="cuda:0")
        nb = S.tp_ffn_workspace_bytes(T, d_ff, T_p, S.TP_BF16)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
        S.tp_ffn_shard_fwd(dv["x"], dv["w1"], dv.get("w3"), dv["w2"], y_ref, ws, nb, T, d, d_ff, T_p,
                           t, act, S.TP_BF16, odt)
        y = torch.full((T, d), float("nan"), dtype=tdt, device="cuda:0")
        S.tp_ffn_shard_fwd_noalloc(dv["x"], dv["w1"], dv.get("w3"), dv["w2"], y, T, d, d_ff, T_p, t,
                                   act, S.TP_BF16, odt)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"call {i}: differs from tp_ffn_shard_fwd"
        outs.append((c, y))
    for i, ((T, d, d_ff, T_p, t, act, _), (c, y)) in enumerate(zip(CALLS, outs)):
        rows = sample_rows(T, 256, seed=i)
        x = f64(c["x"][rows], I.BF16)
        w1, w2 = f64(c["w1"], I.BF16), f64(c["w2"], I.BF16)
        w3 = f64(c["w3"], I.BF16) if act == "swiglu" else None
        _, y_o = O.ffn_shard(x, w1, w3, w2, T_p, t, act)
        e = nerr(host64(y[rows]), y_o)
        log(f"   call {i}: err(y) vs oracle {e:.3e}")
        assert e <= BF16_TOL


def test_noalloc_rejects_oversized_hidden_state():
    """H(t) above the scratch size is refused before anything is launched."""
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda:0")
    y = torch.full((8, 64), 3.0, dtype=torch.bfloat16, device="cuda:0")
    T, d_ff, T_p = 1 << 20, 512, 4     # H(t): 2^20 x 128 bf16 = 256 MiB
    with pytest.raises(S.TPError) as e:
        S.tp_ffn_shard_fwd_noalloc(x, x, None, x, y, T, 64, d_ff, T_p, 0, "gelu", S.TP_BF16, S.TP_BF16)
    assert e.value.code == S.TP_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)
