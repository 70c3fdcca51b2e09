"""GPU parity of the FFN shard (column GEMM + activation epilogue, row GEMM) and
the local partial sum, against the CPU oracle, through the C ABI."""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

from _gpu_util import BF16_TOL, F32_TOL, dev, f64, host64, log, nerr, requires_gpu, sample_rows
from megatron_tensor_transformer_gemm_amd import inputs as I
from megatron_tensor_transformer_gemm_amd import tpshard as S
from oracle import tp_oracle as O

pytestmark = [pytest.mark.gpu, requires_gpu]


def _run_shard(xd, w1d, w3d, w2d, T, d, d_ff, T_p, t, act, in_code, out_code, y=None):
    n = d_ff // T_p
    out_dt = torch.float32 if out_code == S.TP_F32 else torch.bfloat16
    in_elt = 2 if in_code == S.TP_BF16 else 4
    if y is None:
        y = torch.full((T, d), float("nan"), dtype=out_dt, device="cuda:0")
    nbytes = S.tp_ffn_workspace_bytes(T, d_ff, T_p, in_code)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda:0")
    S.tp_ffn_shard_fwd(xd, w1d, w3d, w2d, y, ws, ws.numel(), T, d, d_ff, T_p, t, act, in_code,
                       out_code)
    torch.cuda.synchronize()
    h = ws[: T * n * in_elt].view(torch.bfloat16 if in_code == S.TP_BF16 else torch.float32)
    return y, h.view(T, n)


# ----------------------------------------------------------------------------- bit-exact offsets
@pytest.mark.parametrize("act", ["none", "bilinear"])
@pytest.mark.parametrize("shape", [(300, 264, 4, 136), (8200, 2056, 2, 1032), (2000, 264, 1, 2304),
                                   (2000, 5376, 2, 3072)],
                         ids=["small-tiles", "large-tiles", "192-row-tiles", "192-col-tiles"])
def test_integer_offsets_bit_exact(act, shape):
    """Integer inputs: H(t) and y(t) (fp32 out) must equal the oracle bit for bit."""
    T, d, T_p, n = shape
    d_ff = T_p * n
    log(f"[integer] act={act} T={T} d={d} d_ff={d_ff} T_p={T_p}")
    c = I.integer_offset_case(T, d, d_ff)
    xd, w1d, w3d, w2d = (dev(c[k], I.BF16) for k in ("x", "w1", "w3", "w2"))
    x, w1, w3, w2 = (f64(c[k], I.BF16) for k in ("x", "w1", "w3", "w2"))
    for t in range(T_p):
        y, h = _run_shard(xd, w1d, w3d if act == "bilinear" else None, w2d, T, d, d_ff, T_p, t,
                          act, S.TP_BF16, S.TP_F32)
        h_ref, y_ref = O.ffn_shard(x, w1, w3, w2, T_p, t, act)
        assert np.array_equal(host64(h), h_ref), f"H({t}) differs"
        assert np.array_equal(host64(y), y_ref), f"y({t}) differs"


@pytest.mark.parametrize("act,shape", [("none", (4100, 4104, 2, 4104)), ("bilinear", (4100, 4104, 2, 2200)),
                                       ("none", (16384, 64, 2, 1280)), ("bilinear", (16384, 8, 2, 640)),
                                       ("none", (65792, 256, 1, 8))],
                         ids=["none-289-tiles", "bilinear-306-tiles", "k64-two-stage-loop",
                              "k8-one-ragged-k-tile", "257-tiles"])
def test_integer_persistent_bit_exact(act, shape):
    """More 256 x 256 tiles than the GPU has CUs: the products run one workgroup per CU over
    several tiles each.  289 and 306 tiles with ragged M, N and K; column products whose
    k-loop is two stages long (k 64), so the copies move on to the next tile at the first
    stage, or one ragged k-tile (k 8); and 257 tiles in both products, one workgroup taking
    a second.  Integer inputs, bf16 outputs: H(t) equals the oracle bit for bit, and y(t)
    equals the oracle's exact integer sum rounded once to bf16 (round to nearest, ties to
    even)."""
    T, d, T_p, n = shape
    d_ff = T_p * n
    t = min(1, T_p - 1)
    log(f"[integer persistent] act={act} T={T} d={d} d_ff={d_ff} T_p={T_p} t={t}")
    c = I.integer_offset_case(T, d, d_ff, seed=11)
    xd, w1d, w3d, w2d = (dev(c[k], I.BF16) for k in ("x", "w1", "w3", "w2"))
    x, w1, w3, w2 = (f64(c[k], I.BF16) for k in ("x", "w1", "w3", "w2"))
    y, h = _run_shard(xd, w1d, w3d if act == "bilinear" else None, w2d, T, d, d_ff, T_p, t,
                      act, S.TP_BF16, S.TP_BF16)
    h_ref, y_ref = O.ffn_shard(x, w1, w3, w2, T_p, t, act)
    assert np.abs(y_ref).max() < 2 ** 24
    assert np.array_equal(host64(h), h_ref), "H(t) differs"
    y_ref_bf16 = f64(I.bf16_bits(y_ref.astype(np.float32)), I.BF16)
    assert np.array_equal(host64(y), y_ref_bf16), "y(t) differs"


# ----------------------------------------------------------------------------- float parity
CASES = [
    # T, d, d_ff, T_p, act, in, out
    (64, 256, 1024, 2, "gelu", I.F32, I.F32),
    (77, 136, 264, 2, "swiglu", I.F32, I.F32),
    (1000, 328, 800, 4, "gelu", I.BF16, I.BF16),
    (1000, 328, 800, 4, "swiglu", I.BF16, I.F32),
    (513, 1032, 4112, 2, "swiglu", I.BF16, I.BF16),
    (3000, 2048, 8192, 4, "gelu", I.BF16, I.BF16),
    (2000, 1032, 2304, 1, "gelu", I.BF16, I.BF16),     # 198 tiles of 192 x 128
    # sub-wave products on 192-column tiles: column 128 x 192 (32-k), row 256 x 192 (32-k,
    # ragged last tile row); column 128 x 192 (64-k); row 256 x 192 (64-k, bf16 and fp32 out)
    (2000, 5376, 6144, 2, "gelu", I.BF16, I.BF16),
    (2000, 2048, 6144, 2, "gelu", I.BF16, I.F32),
    (2048, 6144, 1536, 2, "gelu", I.BF16, I.BF16),
    (2048, 6144, 1536, 2, "gelu", I.BF16, I.F32),
    # row GEMM of 33 x 33 256 x 256 tiles, ragged in both M and N
    (8200, 8200, 512, 2, "gelu", I.BF16, I.BF16),
    (1, 64, 64, 1, "gelu", I.BF16, I.BF16),
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}-d{c[1]}-dff{c[2]}-tp{c[3]}-{c[4]}-{c[5]}-{c[6]}"
                                             for c in CASES])
def test_ffn_shard_parity_small(case):
    T, d, d_ff, T_p, act, dt, odt = case
    log(f"[ffn] {case}")
    c = I.small_ffn_case(zlib.crc32(repr(case).encode()) % 1000, T, d, d_ff, act, dt)
    code = S.TP_BF16 if dt == I.BF16 else S.TP_F32
    ocode = S.TP_BF16 if odt == I.BF16 else S.TP_F32
    xd, w1d, w2d = dev(c["x"], dt), dev(c["w1"], dt), dev(c["w2"], dt)
    w3d = dev(c["w3"], dt) if act == "swiglu" else None
    x, w1, w2 = f64(c["x"], dt), f64(c["w1"], dt), f64(c["w2"], dt)
    w3 = f64(c["w3"], dt) if act == "swiglu" else None
    tol = F32_TOL if dt == I.F32 else BF16_TOL
    parts = []
    for t in range(T_p):
        y, h = _run_shard(xd, w1d, w3d, w2d, T, d, d_ff, T_p, t, act, code, ocode)
        h_ref, y_ref = O.ffn_shard(x, w1, w3, w2, T_p, t, act)
        eh, ey = nerr(host64(h), h_ref), nerr(host64(y), y_ref)
        log(f"   t={t} err(H)={eh:.3e} err(y)={ey:.3e}")
        assert eh <= tol and ey <= tol
        parts.append(y)
    # local all-reduce stand-in over all ranks vs the unsharded sublayer
    P = torch.stack(parts)
    out = torch.empty((T, d), dtype=P.dtype, device="cuda:0")
    S.tp_partial_sum(P, T * d, T_p, None, out, T * d, ocode, ocode)
    torch.cuda.synchronize()
    e = nerr(host64(out), O.ffn_unsharded(x, w1, w3, w2, act))
    log(f"   sum err={e:.3e}")
    assert e <= tol


# ----------------------------------------------------------------------------- largest extents
def _extent_case(T, d, d_ff, T_p, act, seed):
    log(f"[extent] T={T} d={d} d_ff={d_ff} T_p={T_p} act={act}")
    c = I.small_ffn_case(seed, T, d, d_ff, act, I.BF16)
    gated = act == "swiglu"
    xd, w1d, w2d = dev(c["x"], I.BF16), dev(c["w1"], I.BF16), dev(c["w2"], I.BF16)
    w3d = dev(c["w3"], I.BF16) if gated else None
    x, w1, w2 = f64(c["x"], I.BF16), f64(c["w1"], I.BF16), f64(c["w2"], I.BF16)
    w3 = f64(c["w3"], I.BF16) if gated else None
    for t in range(T_p):
        y, h = _run_shard(xd, w1d, w3d, w2d, T, d, d_ff, T_p, t, act, S.TP_BF16, S.TP_BF16)
        h_ref, y_ref = O.ffn_shard(x, w1, w3, w2, T_p, t, act)
        eh, ey = nerr(host64(h), h_ref), nerr(host64(y), y_ref)
        log(f"   t={t} err(H)={eh:.3e} err(y)={ey:.3e}")
        assert eh <= BF16_TOL and ey <= BF16_TOL


def test_largest_feature_extent():
    """d = 2^20, the largest feature extent the library accepts (one more multiple of 8 is
    rejected): a 256-row activation tile then spans 512 MB of per-lane byte offsets, the
    column GEMM runs a 2^20-deep k-loop and the row GEMM 4,096 tiles of y(t)."""
    _extent_case(24, 1 << 20, 64, 1, "gelu", 41)


def test_largest_hidden_extent():
    """d_ff = 2^20 with SwiGLU over 2 ranks: each rank's W1/W3 column blocks start 2^19
    columns apart in rows of 2^20 elements, and its row GEMM runs a 2^19-deep k-loop."""
    _extent_case(40, 64, 1 << 20, 2, "swiglu", 42)


def _workload_tensors(w):
    names = ["x", "w1", "w2"] + (["w3"] if w.act == "swiglu" else [])
    return {k: I.make_tensor(w, k) for k in names}


@pytest.mark.parametrize("cid", [1, 2])
def test_workload_full_parity(cid):
    """Workloads the oracle finishes in seconds: every element of every rank and the sum."""
    w = I.WORKLOADS[cid]
    log(f"[workload {cid}] {w.name}")
    c = _workload_tensors(w)
    dt = w.dtype
    code = S.TP_BF16 if dt == I.BF16 else S.TP_F32
    d_ = {k: dev(v, dt) for k, v in c.items()}
    h_ = {k: f64(v, dt) for k, v in c.items()}
    tol = F32_TOL if dt == I.F32 else BF16_TOL
    P = torch.empty((w.T_p, w.T, w.d), dtype=torch.float32 if dt == I.F32 else torch.bfloat16,
                    device="cuda:0")
    for t in range(w.T_p):
        _, h = _run_shard(d_["x"], d_["w1"], d_.get("w3"), d_["w2"], w.T, w.d, w.d_ff, w.T_p, t,
                          w.act, code, code, y=P[t])
        h_ref, y_ref = O.ffn_shard(h_["x"], h_["w1"], h_.get("w3"), h_["w2"], w.T_p, t, w.act)
        eh, ey = nerr(host64(h), h_ref), nerr(host64(P[t]), y_ref)
        log(f"   t={t} err(H)={eh:.3e} err(y)={ey:.3e}")
        assert eh <= tol and ey <= tol
    y = torch.empty((w.T, w.d), dtype=P.dtype, device="cuda:0")
    S.tp_partial_sum(P, w.T * w.d, w.T_p, None, y, w.T * w.d, code, code)
    torch.cuda.synchronize()
    e = nerr(host64(y), O.ffn_unsharded(h_["x"], h_["w1"], h_.get("w3"), h_["w2"], w.act))
    log(f"   sum err={e:.3e}")
    assert e <= tol


@pytest.mark.slow
@pytest.mark.parametrize("cid", [3, 4])
def test_workload_sampled_parity(cid):
    """Full-size Llama-shaped shards in the benchmark's launch configuration.  The oracle
    checks every token row of the 8B-shaped workload, and a seeded sample of 1,024 token
    rows plus the first and last of the 70B-shaped one (FFN rows are independent), of
    every rank's H(t), y(t) and of the 8-way partial sum."""
    w = I.WORKLOADS[cid]
    log(f"[workload {cid}] {w.name} generating inputs")
    c = _workload_tensors(w)
    d_ = {k: dev(v, w.dtype) for k, v in c.items()}
    rows = np.arange(w.T) if cid == 3 else sample_rows(w.T, 1024, seed=cid)
    log(f"   comparing {len(rows)} of {w.T} token rows")
    xs = f64(c["x"][rows], w.dtype)
    P = torch.empty((w.T_p, w.T, w.d), dtype=torch.bfloat16, device="cuda:0")
    ref_parts = []
    for t in range(w.T_p):
        _, h = _run_shard(d_["x"], d_["w1"], d_.get("w3"), d_["w2"], w.T, w.d, w.d_ff, w.T_p, t,
                          w.act, S.TP_BF16, S.TP_BF16, y=P[t])
        b, n = O.shard_range(w.d_ff, w.T_p, t)
        w1s = f64(c["w1"][:, b:b + n], w.dtype)
        w3s = f64(c["w3"][:, b:b + n], w.dtype) if "w3" in c else None
        w2s = f64(c["w2"][b:b + n], w.dtype)
        h_ref, y_ref = O.ffn_shard(xs, w1s, w3s, w2s, 1, 0, w.act)
        eh = nerr(host64(h[rows]), h_ref)
        ey = nerr(host64(P[t][rows]), y_ref)
        log(f"   t={t} err(H)={eh:.3e} err(y)={ey:.3e}")
        assert eh <= BF16_TOL and ey <= BF16_TOL
        ref_parts.append(y_ref)
    y = torch.empty((w.T, w.d), dtype=torch.bfloat16, device="cuda:0")
    S.tp_partial_sum(P, w.T * w.d, w.T_p, None, y, w.T * w.d, S.TP_BF16, S.TP_BF16)
    torch.cuda.synchronize()
    e = nerr(host64(y[rows]), O.partial_sum(ref_parts))
    log(f"   sum err={e:.3e}")
    assert e <= BF16_TOL


# ----------------------------------------------------------------------------- partial sum
@pytest.mark.parametrize("T_p", [1, 2, 3, 8, 11])
@pytest.mark.parametrize("pd,od", [(S.TP_BF16, S.TP_BF16), (S.TP_BF16, S.TP_F32),
                                   (S.TP_F32, S.TP_F32), (S.TP_F32, S.TP_BF16)])
@pytest.mark.parametrize("residual", [False, True])
def test_partial_sum_parity(T_p, pd, od, residual):
    n = 100003                                      # ragged: n % 8 == 3
    stride = n + 5                                  # padded slices, multiple of 8
    g = np.random.default_rng(T_p * 7 + pd)
    pdt = torch.bfloat16 if pd == S.TP_BF16 else torch.float32
    odt = torch.bfloat16 if od == S.TP_BF16 else torch.float32
    P = torch.from_numpy(g.standard_normal((T_p, stride)).astype(np.float32)).to(pdt).cuda()
    res = torch.from_numpy(g.standard_normal(n).astype(np.float32)).to(odt).cuda() if residual else None
    y = torch.full((n,), float("nan"), dtype=odt, device="cuda:0")
    S.tp_partial_sum(P, stride, T_p, res, y, n, pd, od)
    torch.cuda.synchronize()
    Ph = host64(P)[:, :n]
    ref = O.partial_sum(list(Ph), residual=host64(res) if residual else None)
    # one fp32 accumulation then one rounding: within a few ulps of the output type
    tol = 2 ** -8 if od == S.TP_BF16 else 4e-6
    assert nerr(host64(y), ref) <= tol
    y2 = torch.empty_like(y)
    S.tp_partial_sum(P, stride, T_p, res, y2, n, pd, od)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().view(torch.int16 if od == S.TP_BF16 else torch.int32).numpy(),
                          y2.cpu().view(torch.int16 if od == S.TP_BF16 else torch.int32).numpy())


def test_partial_sum_integers_exact_and_in_place():
    T_p, n = 8, 4099
    g = np.random.default_rng(3)
    P = torch.from_numpy(g.integers(-1000, 1000, (T_p, n + 5)).astype(np.float32)).cuda()
    r = torch.from_numpy(g.integers(-1000, 1000, n).astype(np.float32)).cuda()
    y = r.clone()
    S.tp_partial_sum(P, n + 5, T_p, y, y, n, S.TP_F32, S.TP_F32)   # residual aliased with y
    torch.cuda.synchronize()
    ref = host64(P)[:, :n].sum(axis=0) + host64(r)
    assert np.array_equal(host64(y), ref)


def test_partial_sum_past_one_grid_pass():
    """An array longer than one pass of the partial sum's grid (2^28 vectors of 8, the largest
    grid it launches): 2^31 + 13 bf16 elements over 2 slices, so one vector is summed on a
    second pass and 5 elements by the scalar tail.  Small integer partials make every sum
    exact in bf16: the sampled outputs (every pass and tail boundary, and 4,096 seeded
    positions) equal the oracle's sum exactly, and no output is left unwritten."""
    T_p, n = 2, (1 << 31) + 13
    stride = n + 3                                  # a multiple of 8
    log(f"[partial sum past one grid pass] T_p={T_p} n={n} stride={stride}")
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(31)
    P = torch.randint(-64, 65, (T_p, stride), dtype=torch.int16, device="cuda:0", generator=gen)
    P = P.to(torch.bfloat16)
    y = torch.full((n,), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    S.tp_partial_sum(P, stride, T_p, None, y, n, S.TP_BF16, S.TP_BF16)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(y).any())
    edge = 8 << 28                                  # first element of the second pass
    idx = np.concatenate([np.arange(0, 16), np.arange(edge - 16, n),
                          np.random.default_rng(31).integers(0, n, 4096)])
    it = torch.from_numpy(idx).cuda()
    parts = [host64(P[t].index_select(0, it)) for t in range(T_p)]
    assert np.array_equal(host64(y.index_select(0, it)), O.partial_sum(parts))
    del P, y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T_p,pd,od", [(8, S.TP_BF16, S.TP_BF16), (4, S.TP_F32, S.TP_BF16),
                                        (2, S.TP_BF16, S.TP_F32)])
def test_reduce_scatter_rows_are_the_sum_rows(T_p, pd, od):
    """Sequence-parallel reduce-scatter: each rank's rows equal the same rows of the full
    partial sum bit for bit, the oracle within rounding, and the ranks' rows gathered in
    place form the full sum."""
    T, d = 1032, 520
    stride = T * d + 2048
    g = np.random.default_rng(T_p + 10 * pd + 100 * od)
    pdt = torch.bfloat16 if pd == S.TP_BF16 else torch.float32
    odt = torch.bfloat16 if od == S.TP_BF16 else torch.float32
    P = torch.from_numpy(g.standard_normal((T_p, stride)).astype(np.float32)).to(pdt).cuda()
    res = torch.from_numpy(g.standard_normal((T, d)).astype(np.float32)).to(odt).cuda()
    full = torch.empty((T, d), dtype=odt, device="cuda:0")
    S.tp_partial_sum(P, stride, T_p, res, full, T * d, pd, od)
    gathered = torch.full((T, d), float("nan"), dtype=odt, device="cuda:0")
    m = T // T_p
    for t in range(T_p):
        S.tp_reduce_scatter_rows(P, stride, T_p, t, res[t * m:(t + 1) * m], gathered[t * m:(t + 1) * m],
                                 T, d, pd, od)
    torch.cuda.synchronize()
    assert torch.equal(gathered, full)
    Ph = host64(P)[:, :T * d].reshape(T_p, T, d)
    rh = host64(res)
    tol = 2 ** -8 if od == S.TP_BF16 else 4e-6
    for t in (0, T_p - 1):
        ref = O.reduce_scatter_rows(list(Ph), T_p, t, rh[t * m:(t + 1) * m])
        assert nerr(host64(gathered[t * m:(t + 1) * m]), ref) <= tol


def test_empty_inputs_are_noops():
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda:0")
    w = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda:0")
    y = torch.full((8, 64), 7.0, dtype=torch.bfloat16, device="cuda:0")
    S.tp_ffn_shard_fwd(x, w, None, w, y, None, 0, 0, 64, 64, 1, 0, "gelu", S.TP_BF16, S.TP_BF16)
    S.tp_partial_sum(x, 0, 1, None, y, 0, S.TP_BF16, S.TP_BF16)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


def test_errors_leave_outputs_untouched():
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda:0")
    w = torch.zeros((64, 96), dtype=torch.bfloat16, device="cuda:0")
    y = torch.full((8, 64), 7.0, dtype=torch.bfloat16, device="cuda:0")
    ws = torch.empty(4096, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(S.TPError) as e:
        S.tp_ffn_shard_fwd(x, w, None, w, y, ws, 4096, 8, 64, 96, 5, 0, "gelu", S.TP_BF16, S.TP_BF16)
    assert e.value.code == S.TP_ERR_NOT_DIVISIBLE
    with pytest.raises(S.TPError) as e:
        S.tp_ffn_shard_fwd(x, w, None, w, y, ws, 8, 8, 64, 96, 2, 0, "gelu", S.TP_BF16, S.TP_BF16)
    assert e.value.code == S.TP_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
