"""Q4_K dequant and dequant-GEMM on the GPU against the oracle (fp64)."""
import numpy as np
import pytest

import synth
from oracle import formats as OF
from oracle import ops as OO
from tests.gpu_util import assert_rel, sync, ws

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qd():
    import quantized_decode_amd as m
    m.load_library()
    return m


def _dev(a):
    from quantized_decode_amd.tensors import dev
    return dev(a)


def _x16(x):
    import torch
    return _dev(x.view(np.uint16)).view(torch.float16)


def test_dequant_bit_exact(qd):
    import torch
    rng = np.random.default_rng(11)
    n = 6000
    blocks = rng.integers(0, 256, (n, 144), dtype=np.uint8)
    blocks[:1000, 1] &= 0x03    # subnormal d
    blocks[:1000, 3] &= 0x03    # subnormal dmin
    blocks[1000:1100, 0:4] = 0
    out = torch.empty(n * 256, dtype=torch.float32, device="cuda")
    qd.qkdec_dequant_q4k(_dev(blocks.reshape(-1)), n, out)
    sync()
    with np.errstate(invalid="ignore"):   # raw random bytes include inf/NaN d, dmin: NaN in, NaN out
        ref = OF.q4k_dequant_blocks(blocks).astype(np.float32).reshape(-1)
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def _run_gemm(qd, mat, n, k, x, residual=None, b=None):
    import torch
    b = x.shape[0] if b is None else b
    y = torch.empty((b, n), dtype=torch.float32, device="cuda")
    res = None if residual is None else _dev(residual)
    w = ws(qd.qkdec_gemm_q4k_workspace_size(n, k, b))
    qd.qkdec_gemm_q4k(_dev(mat.reshape(-1)), n, k, _x16(x), b, y, residual=res, workspace=w)
    sync()
    return y.cpu().numpy()


@pytest.mark.parametrize("n,k", [(768, 512), (512, 1536), (3072, 512), (96, 256), (208, 768)])
@pytest.mark.parametrize("b", [1, 2, 3, 8, 13, 16])
def test_gemm_toy_shapes(qd, n, k, b):
    st = synth.Streams(100 + n + k + b)
    mat = synth.q4k_matrix(st.next(), n, k)
    x = synth.f16_normal(st.next(), (b, k))
    got = _run_gemm(qd, mat, n, k, x)
    ref = OO.q4k_gemm(mat, n, k, x)
    assert_rel(got, ref, what=f"gemm {n}x{k} B={b}")


@pytest.mark.parametrize("n,k", [(6144, 4096), (4096, 4096), (4096, 12288)])
@pytest.mark.parametrize("b", [1, 8, 16])
def test_gemm_full_shapes_sampled_rows(qd, n, k, b):
    st = synth.Streams(7000 + n // 16 + k // 256 + b)
    mat = synth.q4k_matrix(st.next(), n, k)
    x = synth.f16_normal(st.next(), (b, k))
    got = _run_gemm(qd, mat, n, k, x)
    rows = np.unique(np.concatenate([np.arange(0, 16), np.arange(n - 16, n),
                                     np.random.default_rng(b).integers(0, n, 96)]))
    w = OF.q4k_dequant_rows(mat, n, k, rows=rows)
    ref = x.astype(np.float64) @ w.T
    assert_rel(got[:, rows], ref, what=f"gemm {n}x{k} B={b}")


def test_gemm_residual_in_place(qd):
    import torch
    n, k, b = 4096, 4096, 8
    st = synth.Streams(31)
    mat = synth.q4k_matrix(st.next(), n, k)
    x = synth.f16_normal(st.next(), (b, k))
    r = (st.next().standard_normal((b, n)) * 1e4).astype(np.float32)
    y = _dev(r)
    w = ws(qd.qkdec_gemm_q4k_workspace_size(n, k, b))
    qd.qkdec_gemm_q4k(_dev(mat.reshape(-1)), n, k, _x16(x), b, y, residual=y, workspace=w)
    sync()
    ref = r.astype(np.float64) + OO.q4k_gemm(mat, n, k, x)
    assert_rel(y.cpu().numpy(), ref, what="residual")


def test_gemm_strided_operands(qd):
    import torch
    n, k, b = 512, 1536, 5
    st = synth.Streams(32)
    mat = synth.q4k_matrix(st.next(), n, k)
    xfull = synth.f16_normal(st.next(), (b, k + 64))
    xs = _x16(xfull)[:, :k]
    y = torch.full((b, n + 32), float("nan"), dtype=torch.float32, device="cuda")
    w = ws(qd.qkdec_gemm_q4k_workspace_size(n, k, b))
    qd.qkdec_gemm_q4k(_dev(mat.reshape(-1)), n, k, xs, b, y, workspace=w)
    sync()
    got = y.cpu().numpy()
    assert np.isnan(got[:, n:]).all()
    assert_rel(got[:, :n], OO.q4k_gemm(mat, n, k, xfull[:, :k]), what="strided")


@pytest.mark.parametrize("b", [3, 16])
def test_gemm_wide_range_fp16_activations(qd, b):
    # fp16 activations from 1e-4 up to the format's maximum, per 256-value block: the
    # sums of 32 of them leave fp16's range in the large blocks and must still be exact
    n, k = 512, 2048
    st = synth.Streams(70 + b)
    mat = synth.q4k_matrix(st.next(), n, k)
    rng = st.next()
    mag = 10.0 ** rng.uniform(-4, np.log10(65504.0), (b, k // 256)).repeat(256, axis=1)
    x = np.clip(rng.uniform(-1, 1, (b, k)) * mag, -65504, 65504).astype(np.float16)
    x[0, :256] = np.float16(65504.0)
    x[-1, 256:512] = np.float16(-65504.0)
    got = _run_gemm(qd, mat, n, k, x)
    ref = OO.q4k_gemm(mat, n, k, x.astype(np.float64))
    assert_rel(got, ref, what=f"wide-range fp16 activations, B={b}")


def test_gemm_deterministic_and_batch_invariant(qd):
    n, k = 4096, 12288
    st = synth.Streams(33)
    mat = synth.q4k_matrix(st.next(), n, k)
    x = synth.f16_normal(st.next(), (8, k))
    y1 = _run_gemm(qd, mat, n, k, x)
    y2 = _run_gemm(qd, mat, n, k, x)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    # each sequence's row does not depend on the others (same K chunking for
    # B <= 8, and the same engine: one row alone would otherwise take the
    # matvec, whose sums are rounded in another order)
    import torch
    w = ws(qd.qkdec_gemm_q4k_workspace_size(n, k, 1))
    for b in (0, 5):
        yb = torch.empty((1, n), dtype=torch.float32, device="cuda")
        qd.qkdec_gemm_q4k_engine(_dev(mat.reshape(-1)), n, k, _x16(x[b:b + 1]), 1, yb, qd.GEMM_MFMA, workspace=w)
        sync()
        assert np.array_equal(yb.cpu().numpy()[0].view(np.uint32), y1[b].view(np.uint32))


def test_gemm_workspace_shared_across_shapes(qd):
    # one workspace, used in turn by launches of different shapes (as inside a decode
    # step): every launch's split-K bookkeeping must survive the others' partial sums
    import torch
    b = 8
    st = synth.Streams(44)
    shapes = [(6144, 4096), (4096, 4096), (4096, 12288)]
    mats = [synth.q4k_matrix(st.next(), n, k) for n, k in shapes]
    xs = [synth.f16_normal(st.next(), (b, k)) for _, k in shapes]
    f = 12288
    gmat = synth.q4k_matrix(st.next(), 2 * f, 4096)
    gx = synth.f16_normal(st.next(), (b, 4096))
    need = max([qd.qkdec_gemm_q4k_workspace_size(n, k, b) for n, k in shapes] +
               [qd.qkdec_gemm_q4k_swiglu_workspace_size(f, 4096, b)])
    w = ws(need)
    ga = torch.empty((b, f), dtype=torch.float32, device="cuda")
    for rep in range(2):
        for (n, k), mat, x in zip(shapes, mats, xs):
            y = torch.empty((b, n), dtype=torch.float32, device="cuda")
            qd.qkdec_gemm_q4k(_dev(mat.reshape(-1)), n, k, _x16(x), b, y, workspace=w)
            sync()
            rows = np.unique(np.concatenate([np.arange(64), np.arange(n - 64, n),
                                             np.random.default_rng(n + k).integers(0, n, 128)]))
            ref = x.astype(np.float64) @ OF.q4k_dequant_rows(mat, n, k, rows=rows).T
            assert_rel(y.cpu().numpy()[:, rows], ref, what=f"shared workspace {n}x{k}, pass {rep}")
        qd.qkdec_gemm_q4k_swiglu(_dev(gmat.reshape(-1)), f, 4096, _x16(gx), b, ga, workspace=w)
        sync()
        cols = np.unique(np.concatenate([np.arange(32), np.arange(f - 32, f),
                                         np.random.default_rng(f).integers(0, f, 96)]))
        wd = OF.q4k_dequant_rows(gmat, 2 * f, 4096, rows=np.concatenate([cols, f + cols]))
        gu = gx.astype(np.float64) @ wd.T
        ref = OO.swiglu(gu[:, :cols.size], gu[:, cols.size:])
        assert_rel(ga.cpu().numpy()[:, cols], ref, what=f"shared workspace SwiGLU, pass {rep}")


@pytest.mark.parametrize("f,k,b", [(1536, 512, 2), (1536, 512, 16), (12288, 4096, 8), (12288, 4096, 1),
                                   (48, 256, 3)])
def test_gemm_swiglu(qd, f, k, b):
    import torch
    st = synth.Streams(900 + f + b)
    mat = synth.q4k_matrix(st.next(), 2 * f, k)
    x = synth.f16_normal(st.next(), (b, k))
    a = torch.empty((b, f), dtype=torch.float32, device="cuda")
    w = ws(qd.qkdec_gemm_q4k_swiglu_workspace_size(f, k, b))
    qd.qkdec_gemm_q4k_swiglu(_dev(mat.reshape(-1)), f, k, _x16(x), b, a, workspace=w)
    sync()
    got = a.cpu().numpy().astype(np.float64)
    if f > 2048:
        cols = np.unique(np.concatenate([np.arange(16), np.random.default_rng(f).integers(0, f, 200)]))
    else:
        cols = np.arange(f)
    wg = OF.q4k_dequant_rows(mat, 2 * f, k, rows=cols)
    wu = OF.q4k_dequant_rows(mat, 2 * f, k, rows=cols + f)
    xd = x.astype(np.float64)
    ref = OO.swiglu(xd @ wg.T, xd @ wu.T)
    assert_rel(got[:, cols], ref, what=f"swiglu F={f} B={b}")


@pytest.mark.parametrize("n,k,b", [(512, 1536, 2), (4096, 12288, 8), (4096, 12288, 16), (96, 768, 5)])
def test_gemm_fp32_activations_blocked_rounding(qd, n, k, b):
    import torch
    st = synth.Streams(950 + n + b)
    mat = synth.q4k_matrix(st.next(), n, k)
    rng = st.next()
    # magnitudes from 1e-3 to 1e7 per 256-block: some blocks fit fp16, others need an offset
    x = (rng.standard_normal((b, k)) * 10.0 ** rng.integers(-3, 8, (b, k // 256)).repeat(256, axis=1))
    x[0, :256] = 65504.0      # exactly at the limit: no offset
    x[0, 256] = 65520.0       # would round to inf in plain fp16
    x = x.astype(np.float32)
    y = torch.empty((b, n), dtype=torch.float32, device="cuda")
    w = ws(qd.qkdec_gemm_q4k_workspace_size(n, k, b))
    qd.qkdec_gemm_q4k_xf32(_dev(mat.reshape(-1)), n, k, _dev(x), b, y, workspace=w)
    sync()
    got = y.cpu().numpy()
    xr = OF.round_f16_blocked(x.astype(np.float64))
    rows = np.arange(n) if n <= 512 else np.unique(np.concatenate([np.arange(16),
                                                                   np.random.default_rng(n).integers(0, n, 100)]))
    ref = xr @ OF.q4k_dequant_rows(mat, n, k, rows=rows).T
    assert np.isfinite(got).all()
    assert_rel(got[:, rows], ref, what=f"xf32 {n}x{k} B={b}")
    # in-range activations: the blocked rounding is plain fp16 rounding, so the
    # result is the product with fp16(x) (oracle), and it agrees with the
    # fp16-input entry point (another kernel: the same exact products, added
    # in fp32 in another order) to a few fp32 ulps of the sums
    xs = (rng.standard_normal((b, k)) * 100).astype(np.float32)
    y2 = torch.empty((b, n), dtype=torch.float32, device="cuda")
    qd.qkdec_gemm_q4k_xf32(_dev(mat.reshape(-1)), n, k, _dev(xs), b, y2, workspace=w)
    y3 = torch.empty((b, n), dtype=torch.float32, device="cuda")
    qd.qkdec_gemm_q4k(_dev(mat.reshape(-1)), n, k, _x16(xs.astype(np.float16)), b, y3, workspace=w)
    sync()
    got2, got3 = y2.cpu().numpy(), y3.cpu().numpy()
    ref2 = OF.round_f16(xs.astype(np.float64)) @ OF.q4k_dequant_rows(mat, n, k, rows=rows).T
    assert_rel(got2[:, rows], ref2, what=f"xf32 in-range {n}x{k} B={b}")
    rms = float(np.sqrt(np.mean(got3.astype(np.float64) ** 2)))
    assert float(np.abs(got2.astype(np.float64) - got3).max()) <= 1e-5 * rms, f"xf32 vs fp16 entry {n}x{k} B={b}"


FULL_SHAPES = [(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)]


@pytest.mark.parametrize("n,k", FULL_SHAPES)
@pytest.mark.parametrize("b", [1, 2])
@pytest.mark.parametrize("residual", [False, True])
def test_gemm_matvec_engine_full_shapes(qd, n, k, b, residual):
    # the vector-ALU matvec (no batch padding) on the projection shapes of the
    # Qwen-shaped model, with and without a residual, against the oracle; and
    # the MFMA engine on the same inputs within the same bound
    import torch
    rng = np.random.default_rng(n + k + b)
    mat = synth.q4k_matrix(rng, n, k)
    x = synth.f16_normal(rng, (b, k))
    res = rng.standard_normal((b, n)).astype(np.float32) * 50 if residual else None
    ref = OO.q4k_gemm(mat, n, k, x.astype(np.float64)) + (0 if res is None else res.astype(np.float64))
    w = ws(qd.qkdec_gemm_q4k_workspace_size(n, k, b))
    qd.qkdec_workspace_init(w)
    for engine in (qd.GEMM_MATVEC, qd.GEMM_MFMA):
        y = torch.empty((b, n), dtype=torch.float32, device="cuda")
        qd.qkdec_gemm_q4k_engine(_dev(mat.reshape(-1)), n, k, _x16(x), b, y, engine,
                                 residual=None if res is None else _dev(res), workspace=w)
        sync()
        assert_rel(y.cpu().numpy(), ref, what=f"engine {engine} {n}x{k} B={b}")


def test_gemm_matvec_engine_limits(qd):
    import torch
    rng = np.random.default_rng(5)
    mat = synth.q4k_matrix(rng, 64, 4096)
    x = synth.f16_normal(rng, (3, 4096))
    y = torch.empty((3, 64), dtype=torch.float32, device="cuda")
    w = ws(qd.qkdec_gemm_q4k_workspace_size(64, 4096, 3))
    with pytest.raises(qd.QkdecError) as e:
        qd.qkdec_gemm_q4k_engine(_dev(mat.reshape(-1)), 64, 4096, _x16(x), 3, y, qd.GEMM_MATVEC, workspace=w)
    assert e.value.status == -2
    with pytest.raises(qd.QkdecError) as e:
        qd.qkdec_gemm_q4k_engine(_dev(mat.reshape(-1)), 64, 4096, _x16(x), 3, y, 7, workspace=w)
    assert e.value.status == -1
