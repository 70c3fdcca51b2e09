"""Python binding of the C ABI in include/tpshard.h (argument marshalling only).

Each ``tp_*`` function here has the same name and argument order as the C
entry point; device buffers may be given as torch tensors (their data pointer
is passed) or as integer addresses, and ``hip_stream=None`` means torch's
current stream on the current device.  Every computation runs in the HIP
kernels of ``libtpshard.so``; there is no fallback: if the library is not
built, or a call returns a non-zero status, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtpshard.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "tpshard.h")

TP_OK, TP_ERR_INVALID_ARG, TP_ERR_NOT_DIVISIBLE, TP_ERR_WORKSPACE, TP_ERR_UNSUPPORTED, TP_ERR_HIP = \
    0, -1, -2, -3, -4, -5
TP_ACT_NONE, TP_ACT_GELU, TP_ACT_SWIGLU, TP_ACT_BILINEAR = 0, 1, 2, 3
TP_F32, TP_BF16 = 0, 1
TP_NOALLOC_SCRATCH_BYTES = 128 << 20
ACT = {"none": TP_ACT_NONE, "gelu": TP_ACT_GELU, "swiglu": TP_ACT_SWIGLU, "bilinear": TP_ACT_BILINEAR}
STATUS_NAMES = {0: "TP_OK", -1: "TP_ERR_INVALID_ARG", -2: "TP_ERR_NOT_DIVISIBLE",
                -3: "TP_ERR_WORKSPACE", -4: "TP_ERR_UNSUPPORTED", -5: "TP_ERR_HIP"}


class TPError(RuntimeError):
    def __init__(self, func: str, code: int, msg: str):
        super().__init__(f"{func} -> {STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code
        self.func = func


_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
_SIGS = {
    "tp_abi_version": (_i32, []),
    "tp_last_error": (ctypes.c_char_p, []),
    "tp_shard_range": (_i32, [_i64, _i32, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "tp_ffn_workspace_bytes": (_sz, [_i64, _i64, _i32, _i32]),
    "tp_ffn_shard_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64, _i64, _i32, _i32,
                                _i32, _i32, _i32, _vp]),
    "tp_ffn_shard_fwd_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32,
                                        _i32, _i32, _vp]),
    "tp_ffn_column_fwd": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _vp]),
    "tp_ffn_row_fwd": (_i32, [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _vp]),
    "tp_attn_outproj_shard_fwd": (_i32, [_vp, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _i32, _i32,
                                         _i32, _i32, _vp]),
    "tp_attn_heads_workspace_bytes": (_sz, [_i64, _i64, _i32, _i32, _i32, _i32]),
    "tp_attn_heads_shard_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64, _i64, _i32,
                                       _i32, _i32, _i32, _i32, _i32, _vp]),
    "tp_attn_heads_shard_fwd_kvrep": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64, _i64, _i32,
                                             _i32, _i32, _i32, _i32, _i32, _vp]),
    "tp_attn_heads_kvrep_workspace_bytes": (_sz, [_i64, _i64, _i32, _i32, _i32, _i32]),
    "tp_attn_core_fwd": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _i64, _i64, _i64,
                                _i32, _vp]),
    "tp_partial_sum": (_i32, [_vp, _i64, _i32, _vp, _vp, _i64, _i32, _i32, _vp]),
    "tp_ffn_shard_fwd_train": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32,
                                      _i32, _i32, _i32, _vp]),
    "tp_ffn_bwd_workspace_bytes": (_sz, [_i64, _i64, _i32, _i32]),
    "tp_attn_outproj_shard_bwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _i32,
                                         _i32, _i32, _vp]),
    "tp_reduce_scatter_rows": (_i32, [_vp, _i64, _i32, _i32, _vp, _vp, _i64, _i64, _i32, _i32, _vp]),
    "tp_ffn_shard_bwd": (_i32, [_vp] * 12 + [_vp, _sz, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _i32,
                                             _vp]),
    "tp_attn_ring_init": (_i32, [_vp, _vp, _i64, _i32, _i32, _i64, _i64, _vp]),
    "tp_attn_ring_step": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _i64, _i64,
                                 _i64, _i64, _i64, _i64, _i32, _vp]),
    "tp_attn_ring_finish": (_i32, [_vp, _vp, _i64, _i32, _i32, _i64, _i64, _vp]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libtpshard.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m megatron_tensor_transformer_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/tpshard.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z0-9_]+)\s*\(", text)))


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(func: str, rc: int):
    if rc != TP_OK:
        raise TPError(func, rc, lib().tp_last_error().decode())


def dtype_code(dtype) -> int:
    import torch
    if dtype == torch.bfloat16:
        return TP_BF16
    if dtype == torch.float32:
        return TP_F32
    raise ValueError(f"unsupported dtype {dtype}")


# ----------------------------------------------------------------------------- C entry points
def tp_abi_version() -> int:
    return lib().tp_abi_version()


def tp_last_error() -> str:
    return lib().tp_last_error().decode()


def tp_shard_range(extent: int, T_p: int, t: int) -> tuple[int, int]:
    b, n = _i64(), _i64()
    _check("tp_shard_range", lib().tp_shard_range(extent, T_p, t, ctypes.byref(b), ctypes.byref(n)))
    return b.value, n.value


def tp_ffn_workspace_bytes(T: int, d_ff: int, T_p: int, in_dtype: int) -> int:
    return lib().tp_ffn_workspace_bytes(T, d_ff, T_p, in_dtype)


def tp_ffn_shard_fwd(x, w1, w3, w2, y_t, workspace, workspace_bytes, T, d, d_ff, T_p, t, act,
                     in_dtype, out_dtype, hip_stream=None):
    if isinstance(act, str):
        act = ACT[act]
    _check("tp_ffn_shard_fwd", lib().tp_ffn_shard_fwd(
        _ptr(x), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(y_t), _ptr(workspace), workspace_bytes,
        T, d, d_ff, T_p, t, act, in_dtype, out_dtype, _stream(hip_stream)))


def tp_ffn_shard_fwd_noalloc(x, w1, w3, w2, y_t, T, d, d_ff, T_p, t, act, in_dtype, out_dtype,
                             hip_stream=None):
    if isinstance(act, str):
        act = ACT[act]
    _check("tp_ffn_shard_fwd_noalloc", lib().tp_ffn_shard_fwd_noalloc(
        _ptr(x), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(y_t), T, d, d_ff, T_p, t, act, in_dtype,
        out_dtype, _stream(hip_stream)))


def tp_ffn_column_fwd(x, w1, w3, h_t, T, d, d_ff, T_p, t, act, in_dtype, hip_stream=None):
    if isinstance(act, str):
        act = ACT[act]
    _check("tp_ffn_column_fwd", lib().tp_ffn_column_fwd(
        _ptr(x), _ptr(w1), _ptr(w3), _ptr(h_t), T, d, d_ff, T_p, t, act, in_dtype,
        _stream(hip_stream)))


def tp_ffn_row_fwd(h_t, w2, y_t, T, d, d_ff, T_p, t, in_dtype, out_dtype, hip_stream=None):
    _check("tp_ffn_row_fwd", lib().tp_ffn_row_fwd(
        _ptr(h_t), _ptr(w2), _ptr(y_t), T, d, d_ff, T_p, t, in_dtype, out_dtype,
        _stream(hip_stream)))


def tp_attn_outproj_shard_fwd(o_t, wo, y_t, T, d, n_heads, n_kv_heads, head_dim, T_p, t,
                              in_dtype, out_dtype, hip_stream=None):
    _check("tp_attn_outproj_shard_fwd", lib().tp_attn_outproj_shard_fwd(
        _ptr(o_t), _ptr(wo), _ptr(y_t), T, d, n_heads, n_kv_heads, head_dim, T_p, t, in_dtype,
        out_dtype, _stream(hip_stream)))


def tp_attn_heads_workspace_bytes(n_seq, seq_len, n_heads, n_kv_heads, head_dim, T_p) -> int:
    return lib().tp_attn_heads_workspace_bytes(n_seq, seq_len, n_heads, n_kv_heads, head_dim, T_p)


def tp_attn_heads_shard_fwd(x, wq, wk, wv, o_t, workspace, workspace_bytes, n_seq, seq_len, d,
                            n_heads, n_kv_heads, head_dim, T_p, t, causal, hip_stream=None):
    _check("tp_attn_heads_shard_fwd", lib().tp_attn_heads_shard_fwd(
        _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(o_t), _ptr(workspace), workspace_bytes,
        n_seq, seq_len, d, n_heads, n_kv_heads, head_dim, T_p, t, int(causal),
        _stream(hip_stream)))


def tp_attn_heads_kvrep_workspace_bytes(n_seq, seq_len, n_heads, n_kv_heads, head_dim, T_p) -> int:
    return lib().tp_attn_heads_kvrep_workspace_bytes(n_seq, seq_len, n_heads, n_kv_heads, head_dim, T_p)


def tp_attn_heads_shard_fwd_kvrep(x, wq, wk, wv, o_t, workspace, workspace_bytes, n_seq, seq_len, d,
                                  n_heads, n_kv_heads, head_dim, T_p, t, causal, hip_stream=None):
    _check("tp_attn_heads_shard_fwd_kvrep", lib().tp_attn_heads_shard_fwd_kvrep(
        _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(o_t), _ptr(workspace), workspace_bytes,
        n_seq, seq_len, d, n_heads, n_kv_heads, head_dim, T_p, t, int(causal),
        _stream(hip_stream)))


def tp_attn_core_fwd(q, k, v, o, n_seq, seq_len, h_t, kv_t, head_dim, ldq, ldkv, ldo, causal,
                     hip_stream=None):
    _check("tp_attn_core_fwd", lib().tp_attn_core_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), n_seq, seq_len, h_t, kv_t, head_dim, ldq, ldkv, ldo,
        int(causal), _stream(hip_stream)))


def tp_attn_ring_init(o_state, lse_state, rows, h_t, head_dim, ld_state, ld_lse, hip_stream=None):
    _check("tp_attn_ring_init", lib().tp_attn_ring_init(
        _ptr(o_state), _ptr(lse_state), rows, h_t, head_dim, ld_state, ld_lse, _stream(hip_stream)))


def tp_attn_ring_step(q, k, v, o_state, lse_state, n_seq, seq_len, h_t, kv_t, head_dim, ldq, ldkv,
                      ld_state, ld_lse, q_pos0, k_pos0, causal, hip_stream=None):
    _check("tp_attn_ring_step", lib().tp_attn_ring_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o_state), _ptr(lse_state), n_seq, seq_len, h_t, kv_t,
        head_dim, ldq, ldkv, ld_state, ld_lse, q_pos0, k_pos0, int(causal), _stream(hip_stream)))


def tp_attn_ring_finish(o_state, o, rows, h_t, head_dim, ld_state, ldo, hip_stream=None):
    _check("tp_attn_ring_finish", lib().tp_attn_ring_finish(
        _ptr(o_state), _ptr(o), rows, h_t, head_dim, ld_state, ldo, _stream(hip_stream)))


def tp_partial_sum(partials, partial_stride, T_p, residual, y, n_elems, part_dtype, out_dtype,
                   hip_stream=None):
    _check("tp_partial_sum", lib().tp_partial_sum(
        _ptr(partials), partial_stride, T_p, _ptr(residual), _ptr(y), n_elems, part_dtype,
        out_dtype, _stream(hip_stream)))


def tp_ffn_shard_fwd_train(x, w1, w3, w2, y_t, h_t, u_t, v_t, T, d, d_ff, T_p, t, act, out_dtype,
                           hip_stream=None):
    if isinstance(act, str):
        act = ACT[act]
    _check("tp_ffn_shard_fwd_train", lib().tp_ffn_shard_fwd_train(
        _ptr(x), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(y_t), _ptr(h_t), _ptr(u_t), _ptr(v_t), T, d, d_ff,
        T_p, t, act, out_dtype, _stream(hip_stream)))


def tp_ffn_bwd_workspace_bytes(T: int, d_ff: int, T_p: int, act) -> int:
    if isinstance(act, str):
        act = ACT[act]
    return lib().tp_ffn_bwd_workspace_bytes(T, d_ff, T_p, act)


def tp_ffn_shard_bwd(x, w1, w3, w2, dy, h_t, u_t, v_t, dx_t, dw1, dw3, dw2, workspace,
                     workspace_bytes, T, d, d_ff, T_p, t, act, dx_dtype, grad_dtype, hip_stream=None):
    if isinstance(act, str):
        act = ACT[act]
    _check("tp_ffn_shard_bwd", lib().tp_ffn_shard_bwd(
        _ptr(x), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(dy), _ptr(h_t), _ptr(u_t), _ptr(v_t), _ptr(dx_t),
        _ptr(dw1), _ptr(dw3), _ptr(dw2), _ptr(workspace), workspace_bytes, T, d, d_ff, T_p, t, act,
        dx_dtype, grad_dtype, _stream(hip_stream)))


def tp_attn_outproj_shard_bwd(o_t, wo, dy, do_t, dwo, T, d, n_heads, n_kv_heads, head_dim, T_p, t,
                              grad_dtype, hip_stream=None):
    _check("tp_attn_outproj_shard_bwd", lib().tp_attn_outproj_shard_bwd(
        _ptr(o_t), _ptr(wo), _ptr(dy), _ptr(do_t), _ptr(dwo), T, d, n_heads, n_kv_heads, head_dim, T_p,
        t, grad_dtype, _stream(hip_stream)))


def tp_reduce_scatter_rows(partials, partial_stride, T_p, t, residual, y_rows, T, d, part_dtype,
                           out_dtype, hip_stream=None):
    _check("tp_reduce_scatter_rows", lib().tp_reduce_scatter_rows(
        _ptr(partials), partial_stride, T_p, t, _ptr(residual), _ptr(y_rows), T, d, part_dtype,
        out_dtype, _stream(hip_stream)))


# ----------------------------------------------------------------------------- tensor helpers
def ffn_shard_fwd(x, w1, w3, w2, T_p: int, t: int, act: str, out_dtype=None, y_t=None,
                  workspace=None, hip_stream=None):
    """Allocate-and-call wrapper: returns (y_t, H(t) view of the workspace)."""
    import torch
    T, d = x.shape
    d_ff = w1.shape[1]
    ind = dtype_code(x.dtype)
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if y_t is None:
        y_t = torch.empty((T, d), dtype=out_dtype, device=x.device)
    nbytes = tp_ffn_workspace_bytes(T, d_ff, T_p, ind)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=x.device)
    tp_ffn_shard_fwd(x, w1, w3, w2, y_t, workspace, workspace.numel() * workspace.element_size(),
                     T, d, d_ff, T_p, t, ACT[act], ind, dtype_code(out_dtype), hip_stream)
    n = d_ff // T_p
    h = workspace.view(torch.uint8)[: T * n * x.element_size()].view(x.dtype).view(T, n)
    return y_t, h
