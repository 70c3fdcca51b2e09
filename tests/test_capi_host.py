"""Host side of the C ABI, without a GPU: the library loads, exports every function
the header declares, and rejects invalid calls before launching anything.

Every call below is invalid in at least one argument that is checked before any
kernel launch, so the fake device addresses are never dereferenced.
"""
from __future__ import annotations

import pytest

from megatron_tensor_transformer_gemm_amd import tpshard as S
from oracle import tp_oracle as O

P = 0x100000          # fake, 16-byte aligned "device" address (never dereferenced)
MIS = 0x100008        # misaligned


@pytest.fixture(scope="module")
def L():
    return S.lib()


def test_library_exports_every_declared_function(L):
    names = S.header_functions()
    assert len(names) == 23
    for n in names:
        assert hasattr(L, n), n
    assert S.tp_abi_version() == 3


@pytest.mark.parametrize("extent,T_p", [(14336, 8), (28672, 8), (4096, 4), (27720, 11), (0, 3),
                                        (1024, 2), (6144, 8)])
def test_shard_range_matches_oracle(extent, T_p):
    for t in range(T_p):
        assert S.tp_shard_range(extent, T_p, t) == O.shard_range(extent, T_p, t)


@pytest.mark.parametrize("args,code", [((10, 3, 0), S.TP_ERR_NOT_DIVISIBLE), ((8, 0, 0), S.TP_ERR_INVALID_ARG),
                                       ((8, 2, 2), S.TP_ERR_INVALID_ARG), ((8, 2, -1), S.TP_ERR_INVALID_ARG),
                                       ((-8, 2, 0), S.TP_ERR_INVALID_ARG)])
def test_shard_range_errors(args, code):
    with pytest.raises(S.TPError) as e:
        S.tp_shard_range(*args)
    assert e.value.code == code
    assert S.tp_last_error()


def test_workspace_queries():
    assert S.tp_ffn_workspace_bytes(8192, 14336, 8, S.TP_BF16) == 8192 * 1792 * 2
    assert S.tp_ffn_workspace_bytes(3, 24, 8, S.TP_BF16) == 256          # rounded up
    assert S.tp_ffn_workspace_bytes(64, 1024, 2, S.TP_F32) == 64 * 512 * 4
    assert S.tp_ffn_workspace_bytes(64, 1000, 3, S.TP_BF16) == 0
    # the Llama-shaped ranks fill the GPU without splitting; the GPT block's 2048-token FFN
    # column product (128 tiles of 256 x 192) splits k two ways: 2 fp32 copies of [2048, 3072]
    assert S.tp_ffn_workspace_bytes(16384, 28672, 8, S.TP_BF16) == 16384 * 3584 * 2
    assert S.tp_ffn_workspace_bytes(2048, 24576, 8, S.TP_BF16) == 2048 * 3072 * 2 + 2 * 2048 * 3072 * 4
    assert S.tp_ffn_workspace_bytes(2048, 24576, 8, S.TP_F32) == 2048 * 3072 * 4
    assert S.tp_ffn_workspace_bytes(64, 1024, 2, 7) == 0
    # the GPT block's 2048-token rank: Q, K, V (18 heads of 128), then split-K scratch for the
    # fused projection (72 tiles of 256 x 256 over 3 k-splits: 3 fp32 copies of [2048, 2304])
    assert S.tp_attn_heads_workspace_bytes(1, 2048, 48, 48, 128, 8) == 2048 * 18 * 128 * 2 + 3 * 2048 * 2304 * 4
    assert S.tp_attn_heads_workspace_bytes(1, 2048, 64, 8, 128, 16) == 0
    # TP16 over 8 KV heads: 4 query heads and one replicated KV head per rank; the projection
    # (32 tiles) splits 4 ways
    assert S.tp_attn_heads_kvrep_workspace_bytes(1, 2048, 64, 8, 128, 16) == 2048 * 6 * 128 * 2 + 4 * 2048 * 768 * 4
    # short sequences are not split
    assert S.tp_attn_heads_workspace_bytes(2, 200, 8, 4, 64, 2) == 400 * 8 * 64 * 2
    assert S.tp_attn_heads_kvrep_workspace_bytes(1, 2048, 64, 8, 128, 8) == \
        S.tp_attn_heads_workspace_bytes(1, 2048, 64, 8, 128, 8)
    assert S.tp_attn_heads_kvrep_workspace_bytes(1, 2048, 48, 6, 128, 16) == 0


def _ffn(**kw):
    a = dict(x=P, w1=P, w3=None, w2=P, y_t=P, workspace=P, workspace_bytes=1 << 30, T=64, d=256,
             d_ff=1024, T_p=2, t=0, act=S.TP_ACT_GELU, in_dtype=S.TP_BF16, out_dtype=S.TP_BF16,
             hip_stream=0)
    a.update(kw)
    return S.tp_ffn_shard_fwd(**a)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), S.TP_ERR_INVALID_ARG),
    (dict(w2=MIS), S.TP_ERR_INVALID_ARG),
    (dict(d_ff=1000, T_p=3), S.TP_ERR_NOT_DIVISIBLE),
    (dict(T_p=0), S.TP_ERR_INVALID_ARG),
    (dict(t=2), S.TP_ERR_INVALID_ARG),
    (dict(T=-1), S.TP_ERR_INVALID_ARG),
    (dict(d=0), S.TP_ERR_INVALID_ARG),
    (dict(act=S.TP_ACT_SWIGLU), S.TP_ERR_INVALID_ARG),          # SwiGLU without W3
    (dict(w3=P), S.TP_ERR_INVALID_ARG),                          # W3 with GELU
    (dict(act=9), S.TP_ERR_UNSUPPORTED),
    (dict(in_dtype=S.TP_F32, out_dtype=S.TP_BF16), S.TP_ERR_UNSUPPORTED),
    (dict(d=260), S.TP_ERR_UNSUPPORTED),                         # not a multiple of 8 (bf16)
    (dict(d_ff=1020, T_p=5), S.TP_ERR_UNSUPPORTED),              # n = 204: not a multiple of 8
    (dict(workspace_bytes=100), S.TP_ERR_WORKSPACE),
    (dict(workspace=None), S.TP_ERR_WORKSPACE),
    (dict(d=(1 << 20) + 8), S.TP_ERR_UNSUPPORTED),               # beyond the supported extent
])
def test_ffn_rejects_before_launch(kw, code):
    with pytest.raises(S.TPError) as e:
        _ffn(**kw)
    assert e.value.code == code, S.tp_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(n_kv_heads=8, T_p=16), S.TP_ERR_NOT_DIVISIBLE),         # GQA: 8 KV heads cap TP at 8
    (dict(n_heads=48, n_kv_heads=48, T_p=5), S.TP_ERR_NOT_DIVISIBLE),
    (dict(t=8), S.TP_ERR_INVALID_ARG),
    (dict(o_t=None), S.TP_ERR_INVALID_ARG),
    (dict(n_heads=64, n_kv_heads=24, T_p=8), S.TP_ERR_INVALID_ARG),
    (dict(in_dtype=S.TP_F32, out_dtype=S.TP_BF16), S.TP_ERR_UNSUPPORTED),
])
def test_outproj_rejects_before_launch(kw, code):
    a = dict(o_t=P, wo=P, y_t=P, T=16, d=8192, n_heads=64, n_kv_heads=8, head_dim=128, T_p=8, t=0,
             in_dtype=S.TP_BF16, out_dtype=S.TP_BF16, hip_stream=0)
    a.update(kw)
    with pytest.raises(S.TPError) as e:
        S.tp_attn_outproj_shard_fwd(**a)
    assert e.value.code == code, S.tp_last_error()
    if "n_kv_heads" in kw and kw.get("T_p") == 16:
        assert "n_kv_heads" in S.tp_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(T_p=0), S.TP_ERR_INVALID_ARG),
    (dict(partial_stride=10), S.TP_ERR_INVALID_ARG),
    (dict(partial_stride=1001), S.TP_ERR_UNSUPPORTED),
    (dict(y=P + 16), S.TP_ERR_INVALID_ARG),                      # overlaps the partials
    (dict(part_dtype=5), S.TP_ERR_UNSUPPORTED),
    (dict(n_elems=-1), S.TP_ERR_INVALID_ARG),
    (dict(residual=MIS), S.TP_ERR_INVALID_ARG),
])
def test_partial_sum_rejects_before_launch(kw, code):
    a = dict(partials=P, partial_stride=1000, T_p=4, residual=None, y=P + (1 << 24), n_elems=1000,
             part_dtype=S.TP_BF16, out_dtype=S.TP_BF16, hip_stream=0)
    a.update(kw)
    with pytest.raises(S.TPError) as e:
        S.tp_partial_sum(**a)
    assert e.value.code == code, S.tp_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(h_t=6, kv_t=4), S.TP_ERR_INVALID_ARG),
    (dict(head_dim=96), S.TP_ERR_UNSUPPORTED),
    (dict(ldq=100), S.TP_ERR_INVALID_ARG),
    (dict(ldkv=772), S.TP_ERR_UNSUPPORTED),
    (dict(causal=2), S.TP_ERR_INVALID_ARG),
    (dict(q=None), S.TP_ERR_INVALID_ARG),
    (dict(n_seq=-1), S.TP_ERR_INVALID_ARG),
])
def test_attn_core_rejects_before_launch(kw, code):
    a = dict(q=P, k=P, v=P, o=P, n_seq=1, seq_len=2048, h_t=6, kv_t=6, head_dim=128, ldq=768,
             ldkv=768, ldo=768, causal=True, hip_stream=0)
    a.update(kw)
    with pytest.raises(S.TPError) as e:
        S.tp_attn_core_fwd(**a)
    assert e.value.code == code, S.tp_last_error()


def test_backward_workspace_query():
    assert S.tp_ffn_bwd_workspace_bytes(8192, 14336, 8, "swiglu") == 2 * 8192 * 1792 * 2
    assert S.tp_ffn_bwd_workspace_bytes(8192, 14336, 8, "gelu") == 8192 * 1792 * 2
    assert S.tp_ffn_bwd_workspace_bytes(3, 24, 8, "swiglu") == 2 * 256      # each plane rounded up
    assert S.tp_ffn_bwd_workspace_bytes(64, 1000, 3, "gelu") == 0
    assert S.tp_ffn_bwd_workspace_bytes(64, 1024, 2, 9) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(act=S.TP_ACT_NONE), S.TP_ERR_UNSUPPORTED),             # U would be H
    (dict(u_t=None), S.TP_ERR_INVALID_ARG),
    (dict(v_t=P), S.TP_ERR_INVALID_ARG),                          # V with GELU
    (dict(act=S.TP_ACT_SWIGLU, w3=P), S.TP_ERR_INVALID_ARG),      # SwiGLU without v_t
    (dict(h_t=None), S.TP_ERR_INVALID_ARG),
    (dict(out_dtype=7), S.TP_ERR_UNSUPPORTED),
    (dict(d_ff=1000, T_p=3), S.TP_ERR_NOT_DIVISIBLE),
])
def test_train_forward_rejects_before_launch(kw, code):
    a = dict(x=P, w1=P, w3=None, w2=P, y_t=P, h_t=P, u_t=P, v_t=None, T=64, d=256, d_ff=1024, T_p=2,
             t=0, act=S.TP_ACT_GELU, out_dtype=S.TP_BF16, hip_stream=0)
    a.update(kw)
    with pytest.raises(S.TPError) as e:
        S.tp_ffn_shard_fwd_train(**a)
    assert e.value.code == code, S.tp_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(dy=None), S.TP_ERR_INVALID_ARG),
    (dict(dx_t=None), S.TP_ERR_INVALID_ARG),
    (dict(dw2=MIS), S.TP_ERR_INVALID_ARG),
    (dict(u_t=None), S.TP_ERR_INVALID_ARG),                       # GELU needs U
    (dict(dw3=P), S.TP_ERR_INVALID_ARG),                          # dW3 with GELU
    (dict(act=S.TP_ACT_SWIGLU, w3=P, dw3=P), S.TP_ERR_INVALID_ARG),   # SwiGLU without v_t
    (dict(act=S.TP_ACT_SWIGLU, w3=P, v_t=P), S.TP_ERR_INVALID_ARG),   # SwiGLU without dw3
    (dict(grad_dtype=3), S.TP_ERR_UNSUPPORTED),
    (dict(dx_dtype=3), S.TP_ERR_UNSUPPORTED),
    (dict(d=260), S.TP_ERR_UNSUPPORTED),
    (dict(workspace_bytes=100), S.TP_ERR_WORKSPACE),
    (dict(workspace=None), S.TP_ERR_WORKSPACE),
    (dict(t=2), S.TP_ERR_INVALID_ARG),
])
def test_backward_rejects_before_launch(kw, code):
    a = dict(x=P, w1=P, w3=None, w2=P, dy=P, h_t=P, u_t=P, v_t=None, dx_t=P, dw1=P, dw3=None, dw2=P,
             workspace=P, workspace_bytes=1 << 30, T=64, d=256, d_ff=1024, T_p=2, t=0,
             act=S.TP_ACT_GELU, dx_dtype=S.TP_BF16, grad_dtype=S.TP_F32, hip_stream=0)
    a.update(kw)
    with pytest.raises(S.TPError) as e:
        S.tp_ffn_shard_bwd(**a)
    assert e.value.code == code, S.tp_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(T=1000, T_p=3), S.TP_ERR_NOT_DIVISIBLE),               # sequence not divisible by T_p
    (dict(t=4), S.TP_ERR_INVALID_ARG),
    (dict(d=100), S.TP_ERR_UNSUPPORTED),
    (dict(partial_stride=100), S.TP_ERR_INVALID_ARG),
    (dict(partials=MIS), S.TP_ERR_INVALID_ARG),
    (dict(part_dtype=5), S.TP_ERR_UNSUPPORTED),
])
def test_reduce_scatter_rejects_before_launch(kw, code):
    a = dict(partials=P, partial_stride=1024 * 64, T_p=4, t=1, residual=None, y_rows=P + (1 << 24),
             T=1024, d=64, part_dtype=S.TP_BF16, out_dtype=S.TP_BF16, hip_stream=0)
    a.update(kw)
    with pytest.raises(S.TPError) as e:
        S.tp_reduce_scatter_rows(**a)
    assert e.value.code == code, S.tp_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(n_kv_heads=8, T_p=16), S.TP_ERR_NOT_DIVISIBLE),
    (dict(t=8), S.TP_ERR_INVALID_ARG),
    (dict(dy=None), S.TP_ERR_INVALID_ARG),
    (dict(dwo=MIS), S.TP_ERR_INVALID_ARG),
    (dict(grad_dtype=4), S.TP_ERR_UNSUPPORTED),
    (dict(d=8196), S.TP_ERR_UNSUPPORTED),
])
def test_outproj_backward_rejects_before_launch(kw, code):
    a = dict(o_t=P, wo=P, dy=P, do_t=P, dwo=P, T=16, d=8192, n_heads=64, n_kv_heads=8, head_dim=128,
             T_p=8, t=0, grad_dtype=S.TP_F32, hip_stream=0)
    a.update(kw)
    with pytest.raises(S.TPError) as e:
        S.tp_attn_outproj_shard_bwd(**a)
    assert e.value.code == code, S.tp_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(n_heads=48, n_kv_heads=6, T_p=16), S.TP_ERR_NOT_DIVISIBLE),   # 6 KV heads over 16 ranks
    (dict(n_heads=60, T_p=16), S.TP_ERR_NOT_DIVISIBLE),                 # query heads not divisible
    (dict(t=16), S.TP_ERR_INVALID_ARG),
    (dict(workspace_bytes=1000), S.TP_ERR_WORKSPACE),
])
def test_kvrep_rejects_before_launch(kw, code):
    a = dict(x=P, wq=P, wk=P, wv=P, o_t=P, workspace=P, workspace_bytes=1 << 30, n_seq=1, seq_len=256,
             d=512, n_heads=64, n_kv_heads=8, head_dim=128, T_p=16, t=0, causal=True, hip_stream=0)
    a.update(kw)
    with pytest.raises(S.TPError) as e:
        S.tp_attn_heads_shard_fwd_kvrep(**a)
    assert e.value.code == code, S.tp_last_error()


_RING = dict(q=P, k=P + (1 << 24), v=P + (2 << 24), o_state=P + (3 << 24), lse_state=P + (5 << 24),
             n_seq=1, seq_len=256, h_t=4, kv_t=2, head_dim=128, ldq=512, ldkv=256, ld_state=512,
             ld_lse=4, q_pos0=256, k_pos0=0, causal=True, hip_stream=0)


@pytest.mark.parametrize("kw,code", [
    (dict(ld_state=510), S.TP_ERR_INVALID_ARG),        # not a multiple of 4
    (dict(ld_state=256), S.TP_ERR_INVALID_ARG),        # narrower than h_t*head_dim
    (dict(ld_lse=3), S.TP_ERR_INVALID_ARG),            # narrower than h_t
    (dict(q_pos0=-1), S.TP_ERR_INVALID_ARG),
    (dict(q_pos0=1 << 30, k_pos0=0), S.TP_ERR_INVALID_ARG),
    (dict(head_dim=96, ldq=384, ldkv=192, ld_state=384), S.TP_ERR_UNSUPPORTED),
    (dict(lse_state=None), S.TP_ERR_INVALID_ARG),
    (dict(o_state=MIS), S.TP_ERR_INVALID_ARG),
    (dict(o_state=P), S.TP_ERR_INVALID_ARG),           # the state overlaps q
    (dict(lse_state=P + (3 << 24)), S.TP_ERR_INVALID_ARG),   # lse overlaps o_state
    (dict(h_t=3), S.TP_ERR_INVALID_ARG),               # not a multiple of kv_t
    (dict(causal=2), S.TP_ERR_INVALID_ARG),
])
def test_ring_step_rejects_before_launch(kw, code):
    a = dict(_RING)
    a.update(kw)
    with pytest.raises(S.TPError) as e:
        S.tp_attn_ring_step(**a)
    assert e.value.code == code, S.tp_last_error()


def test_ring_step_without_work_launches_nothing():
    """A key chunk wholly after the query chunk (causal), or an empty chunk, returns before
    any launch, so fake device addresses are fine."""
    S.tp_attn_ring_step(**dict(_RING, q_pos0=0, k_pos0=256))
    S.tp_attn_ring_step(**dict(_RING, q_pos0=0, k_pos0=10_000))
    S.tp_attn_ring_step(**dict(_RING, seq_len=0))


@pytest.mark.parametrize("kw,code", [
    (dict(ld_state=510), S.TP_ERR_INVALID_ARG),
    (dict(ld_lse=3), S.TP_ERR_INVALID_ARG),
    (dict(rows=-1), S.TP_ERR_INVALID_ARG),
    (dict(head_dim=32), S.TP_ERR_UNSUPPORTED),
    (dict(lse_state=P + 64), S.TP_ERR_INVALID_ARG),    # overlaps o_state
])
def test_ring_init_rejects_before_launch(kw, code):
    a = dict(o_state=P, lse_state=P + (1 << 24), rows=256, h_t=4, head_dim=128, ld_state=512, ld_lse=4,
             hip_stream=0)
    a.update(kw)
    with pytest.raises(S.TPError) as e:
        S.tp_attn_ring_init(**a)
    assert e.value.code == code, S.tp_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(ldo=510), S.TP_ERR_INVALID_ARG),
    (dict(ldo=256), S.TP_ERR_INVALID_ARG),
    (dict(o=P + 1024), S.TP_ERR_INVALID_ARG),          # overlaps the state
    (dict(o=MIS), S.TP_ERR_INVALID_ARG),
    (dict(h_t=0), S.TP_ERR_INVALID_ARG),
])
def test_ring_finish_rejects_before_launch(kw, code):
    a = dict(o_state=P, o=P + (1 << 24), rows=256, h_t=4, head_dim=128, ld_state=512, ldo=512,
             hip_stream=0)
    a.update(kw)
    with pytest.raises(S.TPError) as e:
        S.tp_attn_ring_finish(**a)
    assert e.value.code == code, S.tp_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(T=16384, d_ff=28672 * 2, T_p=8), S.TP_ERR_WORKSPACE),    # H(t) of 224 MiB > 128 MiB
    (dict(T=1 << 20, d_ff=512, T_p=4), S.TP_ERR_WORKSPACE),        # 256 MiB
    (dict(d_ff=1000, T_p=3), S.TP_ERR_NOT_DIVISIBLE),
    (dict(w3=P), S.TP_ERR_INVALID_ARG),                             # W3 with GELU
    (dict(y_t=MIS), S.TP_ERR_INVALID_ARG),
    (dict(in_dtype=S.TP_F32, out_dtype=S.TP_BF16), S.TP_ERR_UNSUPPORTED),
])
def test_noalloc_rejects_before_launch(kw, code):
    """The allocation-free FFN entry point checks its arguments, and that H(t) fits the
    library's per-GPU scratch, before it touches the device."""
    a = dict(x=P, w1=P, w3=None, w2=P, y_t=P, T=64, d=256, d_ff=1024, T_p=2, t=0, act="gelu",
             in_dtype=S.TP_BF16, out_dtype=S.TP_BF16, hip_stream=0)
    a.update(kw)
    with pytest.raises(S.TPError) as e:
        S.tp_ffn_shard_fwd_noalloc(**a)
    assert e.value.code == code, S.tp_last_error()


def test_noalloc_limit_fits_the_70b_shard():
    """128 MiB of scratch holds H(t) of the Llama-3-70B-shaped rank (16,384 x 3,584 bf16)."""
    assert S.tp_ffn_workspace_bytes(16384, 28672, 8, S.TP_BF16) <= S.TP_NOALLOC_SCRATCH_BYTES
    assert S.TP_NOALLOC_SCRATCH_BYTES == 128 << 20
