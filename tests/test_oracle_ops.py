"""Pins for the oracle's per-layer operations (CPU only): exact special cases,
closed forms, invariants and brute force on tiny inputs."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import ops
from tests.test_oracle_formats import pack_q4k


def _tiled(blocks_rowmajor: np.ndarray) -> np.ndarray:
    """Row-major blocks [N, K/256, 144] -> row-tiled storage [N/16, K/256, 16, 144]."""
    n, kb, _ = blocks_rowmajor.shape
    return np.ascontiguousarray(blocks_rowmajor.reshape(n // 16, 16, kb, 144).transpose(0, 2, 1, 3))


def _rand_fields(rng, n, kb, d_bits, dmin_bits):
    blocks = np.zeros((n, kb, 144), np.uint8)
    fields = []
    for r in range(n):
        row = []
        for c in range(kb):
            sc, m, q = rng.integers(0, 64, 8), rng.integers(0, 64, 8), rng.integers(0, 16, 256)
            blocks[r, c] = np.frombuffer(pack_q4k(d_bits, dmin_bits, sc, m, q), np.uint8)
            row.append((sc, m, q))
        fields.append(row)
    return blocks, fields


def test_q4k_gemm_exact_integer_case():
    # d = 2^-4, dmin = 2^-6, integer activations: every result is a dyadic rational
    # that fp64 holds exactly, so the oracle must equal exact rational arithmetic.
    rng = np.random.default_rng(1)
    n, k, bsz = 32, 512, 3
    d_bits, dmin_bits = 0x2C00, 0x2400  # 2^-4, 2^-6
    blocks, fields = _rand_fields(rng, n, k // 256, d_bits, dmin_bits)
    x = rng.integers(-8, 9, (bsz, k)).astype(np.float16)
    y = ops.q4k_gemm(_tiled(blocks), n, k, x)
    d, dmin = Fraction(1, 16), Fraction(1, 64)
    for b in range(bsz):
        xs = [int(v) for v in x[b]]
        for r in range(n):
            acc = Fraction(0)
            for c in range(k // 256):
                sc, m, q = fields[r][c]
                for i in range(256):
                    w = d * int(sc[i // 32]) * int(q[i]) - dmin * int(m[i // 32])
                    acc += w * xs[256 * c + i]
            assert Fraction(y[b, r]) == acc


def test_q4k_gemm_rows_match_fsum():
    rng = np.random.default_rng(4)
    n, k, bsz = 48, 768, 2
    mat = rng.integers(0, 256, (n // 16, k // 256, 16, 144), dtype=np.uint8)
    mat[..., 1] &= 0x17
    mat[..., 3] &= 0x17
    x = rng.standard_normal((bsz, k)).astype(np.float16)
    y = ops.q4k_gemm(mat, n, k, x)
    w = F.q4k_dequant_rows(mat, n, k)
    for b in range(bsz):
        for r in range(n):
            # products of an exact weight and an fp16 value are exact in fp64
            ref = math.fsum(float(w[r, i]) * float(x[b, i]) for i in range(k))
            assert abs(y[b, r] - ref) <= 1e-13 * (abs(ref) + math.fsum(abs(float(w[r, i]) * float(x[b, i])) for i in range(k)))


def test_q4k_gemm_orientation():
    # a single nonzero weight at (row r, column c) picks out x[:, c] into y[:, r]
    n, k = 32, 512
    for r, c in [(0, 0), (5, 300), (31, 511), (17, 256)]:
        blocks = np.zeros((n, k // 256, 144), np.uint8)
        q = np.zeros(256, int)
        q[c % 256] = 1
        sc = np.zeros(8, int)
        sc[(c % 256) // 32] = 1
        blocks[r, c // 256] = np.frombuffer(pack_q4k(0x3C00, 0, sc, np.zeros(8, int), q), np.uint8)
        x = np.arange(2 * k, dtype=np.float64).reshape(2, k)
        y = ops.q4k_gemm(_tiled(blocks), n, k, x)
        want = np.zeros((2, n))
        want[:, r] = x[:, c]
        assert (y == want).all()


def test_dense_gemm_brute_force():
    rng = np.random.default_rng(6)
    w = rng.standard_normal((37, 16)).astype(np.float16)
    x = rng.standard_normal((3, 16)).astype(np.float16)
    y = ops.dense_gemm(w, x, row_chunk=10)
    for b in range(3):
        for r in range(37):
            assert abs(y[b, r] - math.fsum(float(w[r, i]) * float(x[b, i]) for i in range(16))) < 1e-14


# ---------------------------------------------------------------- attention
def _brute_attention(q, k, v, scale):
    hq, d = q.shape
    hkv, n, _ = k.shape
    out = np.zeros((hq, d))
    for h in range(hq):
        g = h * hkv // hq
        s = [scale * math.fsum(q[h, i] * k[g, t, i] for i in range(d)) for t in range(n)]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        tot = math.fsum(e)
        for i in range(d):
            out[h, i] = math.fsum(e[t] * v[g, t, i] for t in range(n)) / tot
    return out


def test_attention_brute_force_gqa():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((8, 16))
    k = rng.standard_normal((2, 11, 16))
    v = rng.standard_normal((2, 11, 16))
    o = ops.attention(q, k, v, 0.25)
    assert np.allclose(o, _brute_attention(q, k, v, 0.25), rtol=1e-12, atol=1e-14)


def test_attention_invariants():
    rng = np.random.default_rng(10)
    hq, hkv, n, d = 8, 2, 40, 32
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((hkv, n, d))
    v = rng.standard_normal((hkv, n, d))
    s = 1 / math.sqrt(d)
    o = ops.attention(q, k, v, s)
    # n = 1: output is the only value
    assert np.allclose(ops.attention(q, k[:, :1], v[:, :1], s), np.repeat(v[:, 0], hq // hkv, axis=0))
    # all keys equal: output is the mean value
    ke = np.repeat(k[:, :1], n, axis=1)
    assert np.allclose(ops.attention(q, ke, v, s), np.repeat(v.mean(axis=1), hq // hkv, axis=0))
    # permutation of tokens does not matter
    perm = rng.permutation(n)
    assert np.allclose(ops.attention(q, k[:, perm], v[:, perm], s), o, rtol=1e-12, atol=1e-13)
    # GQA equals MHA with duplicated KV heads
    kk = np.repeat(k, hq // hkv, axis=0)
    vv = np.repeat(v, hq // hkv, axis=0)
    assert np.allclose(ops.attention(q, kk, vv, s), o, rtol=1e-12, atol=1e-13)
    # one dominant key: output tends to its value
    kd = k.copy()
    kd[:, 7] = 1e3 * q[:: hq // hkv]
    od = ops.attention(q[:: hq // hkv], kd, v, s)
    assert np.allclose(od, v[:, 7], atol=1e-9)
    # outputs are convex combinations of the values
    for h in range(hq):
        g = h // (hq // hkv)
        assert (o[h] <= v[g].max(axis=0) + 1e-12).all() and (o[h] >= v[g].min(axis=0) - 1e-12).all()


def test_lse_split_merge_identity():
    # The split-K combine: O = sum_j e^{m_j-M} o_j / sum_j e^{m_j-M} l_j with per-split
    # (m_j, l_j, o_j = sum_t e^{s_t-m_j} v_t) equals attention over the whole range.
    rng = np.random.default_rng(12)
    hq, hkv, n, d = 4, 1, 300, 64
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((hkv, n, d)) * 3
    v = rng.standard_normal((hkv, n, d))
    s = 1 / 8
    full = ops.attention(q, k, v, s)
    bounds = [0, 1, 77, 128, 129, 256, 300]
    for h in range(hq):
        parts = []
        for a, b in zip(bounds[:-1], bounds[1:]):
            sc = s * (k[0, a:b] @ q[h])
            m = sc.max()
            e = np.exp(sc - m)
            parts.append((m, e.sum(), e @ v[0, a:b]))
        big = max(p[0] for p in parts)
        num = sum(np.exp(p[0] - big) * p[2] for p in parts)
        den = sum(np.exp(p[0] - big) * p[1] for p in parts)
        assert np.allclose(num / den, full[h], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- small ops
def test_rmsnorm_closed_forms():
    g = np.linspace(0.5, 1.5, 64)
    c = 3.0
    assert np.allclose(ops.rmsnorm(np.full(64, c), g, 1e-6), g * c / math.sqrt(c * c + 1e-6), rtol=1e-15)
    x = np.random.default_rng(0).standard_normal((3, 64))
    assert np.allclose(ops.rmsnorm(1e6 * x, g, 0.0), ops.rmsnorm(x, g, 0.0), rtol=1e-13)
    y = ops.rmsnorm(x, np.ones(64), 0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0)
    for row in range(3):
        ms = math.fsum(v * v for v in x[row]) / 64
        assert np.allclose(ops.rmsnorm(x[row], g, 1e-6), g * x[row] / math.sqrt(ms + 1e-6), rtol=1e-14)


def test_rope_closed_forms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 64))
    base = 1e6
    assert np.array_equal(ops.rope(x, 0, base), x)
    r = ops.rope(x, 1234, base)
    half = 32
    # pair norms are preserved
    assert np.allclose(x[:, :half] ** 2 + x[:, half:] ** 2, r[:, :half] ** 2 + r[:, half:] ** 2)
    # pair 0 turns by exactly pos radians; the last pair by pos * base^(-(D-2)/D)
    for pos in (1, 7, 19000):
        rr = ops.rope(x, pos, base)
        a0 = pos * 1.0
        assert np.allclose(rr[:, 0], x[:, 0] * math.cos(a0) - x[:, half] * math.sin(a0))
        assert np.allclose(rr[:, half], x[:, half] * math.cos(a0) + x[:, 0] * math.sin(a0))
        al = pos * base ** (-(64 - 2) / 64)
        assert np.allclose(rr[:, half - 1], x[:, half - 1] * math.cos(al) - x[:, -1] * math.sin(al))
    # relative position: <R_m q, R_n k> = <R_{m-n} q, k>
    q, k = rng.standard_normal((1, 64)), rng.standard_normal((1, 64))
    for m, n in [(10, 3), (5000, 4990), (19000, 0)]:
        lhs = float((ops.rope(q, m, base) @ ops.rope(k, n, base).T)[0, 0])
        rhs = float((ops.rope(q, m - n, base) @ k.T)[0, 0])
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(rhs))


def test_silu_swiglu_closed_forms():
    z = np.array([-1e4, -800.0, -50.0, -1.0, 0.0, 1.0, 50.0, 800.0])
    with np.errstate(over="raise", invalid="raise", divide="raise"):
        s = ops.silu(z)
    assert s[4] == 0.0
    assert np.allclose(s[[0, 1]], 0.0) and np.allclose(s[[6, 7]], z[[6, 7]])
    zz = np.random.default_rng(2).standard_normal(100) * 5
    assert np.allclose(ops.silu(-zz), ops.silu(zz) - zz, rtol=1e-13, atol=1e-13)
    for v in zz[:10]:
        assert abs(ops.silu(np.array([v]))[0] - v / (1 + math.exp(-v))) < 1e-13
    g, u = zz[:50], zz[50:]
    assert np.allclose(ops.swiglu(g, u), ops.silu(g) * u)


def test_argmax_lowest_index_on_ties():
    a = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0], [-1.0, -2.0, -1.0, -3.0]])
    assert list(ops.argmax_lowest(a)) == [1, 0, 0]
