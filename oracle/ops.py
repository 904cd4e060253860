"""The per-layer operations of a decode step in plain fp64 (oracle; test
infrastructure only).
(P1, P2, P3: the three pages listed, with their titles, in oracle/__init__.py.)

Each function is the textbook definition; none is blocked, fused or reordered.
"""
from __future__ import annotations

import numpy as np

from .formats import q4k_dequant_rows

GEMM_ROW_CHUNK = 1024


def q4k_gemm(mat: np.ndarray, n_rows: int, n_cols: int, x: np.ndarray) -> np.ndarray:
    """Y[b, n] = sum_k W[n, k] * X[b, k] with W the dequantized Q4_K matrix.

    P1 "The weight read is the only term that does not scale": a step reads the
    weights once and multiplies every sequence's hidden state against them.
    The dequantized weights are exact (see formats.q4k_dequant_blocks); each
    sequence's row is a separate matrix-vector product on the same fp64
    weights, so a sequence's result does not depend on the rest of the batch.

    x: [B, n_cols] (fp16 values given as any float dtype).  Returns fp64 [B, n_rows].
    """
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] == n_cols
    y = np.empty((x.shape[0], n_rows), dtype=np.float64)
    for r0 in range(0, n_rows, GEMM_ROW_CHUNK):
        r1 = min(n_rows, r0 + GEMM_ROW_CHUNK)
        w = q4k_dequant_rows(mat, n_rows, n_cols, rows=slice(r0, r1))
        for b in range(x.shape[0]):
            y[b, r0:r1] = w @ x[b]
    return y


def dense_gemm(w: np.ndarray, x: np.ndarray, row_chunk: int = 8192) -> np.ndarray:
    """Y[b, n] = sum_k W[n, k] * X[b, k] for a dense (fp16) weight matrix."""
    x = np.asarray(x, dtype=np.float64)
    y = np.empty((x.shape[0], w.shape[0]), dtype=np.float64)
    for r0 in range(0, w.shape[0], row_chunk):
        wc = np.asarray(w[r0:r0 + row_chunk], dtype=np.float64)
        for b in range(x.shape[0]):
            y[b, r0:r0 + wc.shape[0]] = wc @ x[b]
    return y


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """gamma * x / sqrt(mean(x^2) + eps) over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(gamma, dtype=np.float64) * x / np.sqrt(ms + eps)


def rope(x: np.ndarray, pos: int, base: float) -> np.ndarray:
    """Rotate-half rotary embedding of x [heads, D] at position pos.

    For i < D/2 the pair (x_i, x_{i+D/2}) is rotated by a = pos * base^(-2i/D).
    """
    x = np.asarray(x, dtype=np.float64)
    dim = x.shape[-1]
    half = dim // 2
    i = np.arange(half, dtype=np.float64)
    theta = base ** (-2.0 * i / dim)
    a = float(pos) * theta
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Grouped-query attention of one sequence over its whole private cache.

    P2 "The two halves of a decode-step memory bill": every sequence reads all
    of its own keys and values each step; several query heads share one KV
    head (grouped-query attention).

    q: [Hq, D]; k, v: [Hkv, n, D].  Query head h reads KV head h // (Hq/Hkv).
    Returns O [Hq, D] = softmax_t(scale * q_h . k_t) . v_t.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq, hkv = q.shape[0], k.shape[0]
    group = hq // hkv
    out = np.empty_like(q)
    for h in range(hq):
        g = h // group
        s = scale * (k[g] @ q[h])
        p = np.exp(s - np.max(s))
        p /= np.sum(p)
        out[h] = p @ v[g]
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z), in the form that does not overflow for z << 0."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """silu(gate) * up."""
    return silu(gate) * np.asarray(up, dtype=np.float64)


def argmax_lowest(logits: np.ndarray) -> np.ndarray:
    """Index of the maximum along the last axis; the lowest index wins ties."""
    return np.argmax(np.asarray(logits), axis=-1)
