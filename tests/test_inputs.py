"""The seeded input generator: determinism, bf16 encoding, workload shapes."""
from __future__ import annotations

import numpy as np
import torch

from megatron_tensor_transformer_gemm_amd import inputs as I


def test_bf16_rne_matches_torch_conversion():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * s for s in (1e-3, 1, 1e3)])
    # exact ties: mantissa low half == 0x8000, both parities of the kept bit
    ties = (np.arange(0, 4000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    a = np.concatenate([a, ties, -ties, np.array([0.0, -0.0, 1.0, 65504.0], np.float32)])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(I.bf16_bits(a), ref)
    back = I.bf16_to_f32(ref)
    np.testing.assert_array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_draw_is_deterministic_and_seeded_per_tensor():
    a = I.draw(3, 1, (64, 32), 0.5)
    b = I.draw(3, 1, (64, 32), 0.5)
    c = I.draw(3, 2, (64, 32), 0.5)
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, c)
    assert a.dtype == np.float32
    g = np.random.Generator(np.random.PCG64(3001)).standard_normal((64, 32), dtype=np.float32)
    np.testing.assert_array_equal(a, g * np.float32(0.5))


def test_rms_normalised_rows_have_unit_rms():
    x = I.rms_normalise_rows(I.draw(9, 0, (16, 4096), 3.0))
    np.testing.assert_allclose(np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=1)), 1.0, rtol=1e-5)


def test_workload_table():
    w = I.WORKLOADS
    assert (w[1].T, w[1].d, w[1].d_ff, w[1].T_p, w[1].n) == (64, 256, 1024, 2, 512)
    assert (w[2].T, w[2].n) == (4096, 1024)
    assert (w[3].T, w[3].d, w[3].n, w[3].act) == (8192, 4096, 1792, "swiglu")
    assert (w[4].T, w[4].d, w[4].n, w[4].n_heads, w[4].n_kv_heads, w[4].head_dim) == \
        (16384, 8192, 3584, 64, 8, 128)
    assert (w[5].T, w[5].seq_len, w[5].n_seq, w[5].n, w[5].n_heads // w[5].T_p) == \
        (8192, 2048, 4, 3072, 6)


def test_make_tensor_small_workload():
    w = I.WORKLOADS[1]
    x = I.make_tensor(w, "x")
    w1 = I.make_tensor(w, "w1")
    assert x.shape == (64, 256) and x.dtype == np.float32
    assert w1.shape == (256, 1024)
    assert abs(float(np.std(w1)) - 1 / 16) < 0.01
    w2 = I.WORKLOADS[2]
    xb = I.make_tensor(w2, "x")
    assert xb.dtype == np.uint16 and xb.shape == (4096, 1024)


def test_integer_case_is_exact():
    c = I.integer_offset_case(T=5, d=16, d_ff=32)
    x = I.bf16_to_f32(c["x"])
    assert np.all(x == np.round(x)) and np.max(np.abs(x)) <= 8
    w1 = I.bf16_to_f32(c["w1"])
    assert np.all(np.sum(np.abs(w1), axis=0) == 1)


def test_integer_backward_case_is_exact_in_the_kernels_formats():
    """The integer backward case keeps dU, dV within +-32 and H within +-64 (bf16-exact
    integers) and every gradient an integer below 2^24 (fp32-exact)."""
    from oracle import tp_oracle as O
    c = I.integer_backward_case(300, 264, 544)
    x, w1, w3, w2, dy = (I.as_f64(c[k], I.BF16) for k in ("x", "w1", "w3", "w2", "dy"))
    for act in ("none", "bilinear"):
        for t in range(4):
            r = O.ffn_shard_bwd(x, w1, w3, w2, dy, 4, t, act)
            for k in ("du", "dv", "h", "dx_t", "dw1", "dw2", "dw3"):
                a = r[k]
                if a is None:
                    continue
                assert np.all(a == np.round(a)) and np.max(np.abs(a)) < 2 ** 24, k
            assert np.max(np.abs(r["du"])) <= 32 and np.max(np.abs(r["h"])) <= 64
            if r["dv"] is not None:
                assert np.max(np.abs(r["dv"])) <= 32
