"""Storage formats decoded in plain fp64 (oracle; test infrastructure only).
(P1, P2, P3: the three pages listed, with their titles, in oracle/__init__.py.)

Q4_K super-block (144 bytes, 256 weights), as fixed by the synthetic weight
workload of the batched-decode pages (P1 names the weights "Q4_K"; the field
semantics are d, dmin, eight 6-bit scales, eight 6-bit mins, 4-bit quants and
w = d*sc*q - dmin*m).  The byte layout below is this library's own:

* bytes 0-1   fp16 d      (little-endian)
* bytes 2-3   fp16 dmin   (little-endian)
* bytes 4-15  four 24-bit little-endian groups; group p (bytes 4+3p..6+3p)
  holds, from its least significant bit: sc[2p], sc[2p+1], m[2p], m[2p+1],
  6 bits each.  Sub-block s covers weights 32s..32s+31.
* bytes 16-143 32 little-endian 32-bit words; word j covers weights 8j..8j+7:
  its low half-word holds weights 8j, 8j+2, 8j+4, 8j+6 and its high half-word
  weights 8j+1, 8j+3, 8j+5, 8j+7, each in increasing nibble order.  So weight
  8j + 2i + par sits at bits 16*par + 4*i of word j.

A Q4_K matrix of N rows (outputs) and K columns (inputs) is stored in row
tiles of 16 rows: [N/16][K/256][16][144] (tile, super-block column, row within
the tile, block bytes).

Q8_0 (P3, "Why Q8 is close to free and where the sharp edges are": one byte per
KV element plus a per-block scale): 32 int8 values and one fp16 scale per
block; value = d*q.  Blocks run along head_dim within one token and head.

FP8 E4M3 (P2 "What a long-running swarm should actually tune" and P3 "Why Q8
is close to free and where the sharp edges are": an 8-bit float KV cache that
halves the fp16 footprint).  The pages name no variant; this library reads it
as the OCP E4M3 format with no scale: one byte per element, sign bit, 4-bit
exponent with bias 7, 3-bit mantissa; exponent field 0 is subnormal
(m/8 * 2^-6); there is no infinity and S.1111.111 is NaN, so the largest finite
magnitude is 1.75 * 2^8 = 448.  Stores round to nearest (ties to even) and
saturate at +-448.
"""
from __future__ import annotations

import numpy as np

Q4K_BLOCK_BYTES = 144
QK_K = 256
ROW_TILE = 16
Q8_BLOCK = 32

# weight index held by (word j, half-word par, nibble i): 8j + 2i + par
_Q_INDEX = np.empty((32, 2, 4), dtype=np.int64)
for _j in range(32):
    for _par in range(2):
        for _i in range(4):
            _Q_INDEX[_j, _par, _i] = 8 * _j + 2 * _i + _par


def f16_bits_to_f64(bits) -> np.ndarray:
    """fp16 bit patterns (any unsigned int dtype) -> exact fp64 values."""
    return np.asarray(bits).astype(np.uint16).view(np.float16).astype(np.float64)


def round_f16(x) -> np.ndarray:
    """Round-to-nearest-even to fp16, returned as fp64 (one rounding)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def round_f16_blocked(x, block: int = 256) -> np.ndarray:
    """fp16 rounding with one power-of-two exponent offset per block of values.

    Along the last axis, each run of `block` consecutive values gets the
    smallest integer s >= 0 with max|x| * 2^-s <= 65504, and each value
    becomes 2^s * RN_fp16(x * 2^-s).  A block already inside fp16's range has
    s = 0, so this equals round_f16 wherever plain fp16 does not overflow.
    Used for the SwiGLU activation handed to the down projection, whose
    magnitude the pages leave open and which exceeds fp16's range on the
    synthetic weights (their mean is about 0.16, not 0).
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    assert n % block == 0
    xb = x.reshape(x.shape[:-1] + (n // block, block))
    amax = np.max(np.abs(xb), axis=-1, keepdims=True)
    s = np.zeros_like(amax)
    while True:
        over = amax * np.exp2(-s) > 65504.0
        if not over.any():
            break
        s = s + over
    scale = np.exp2(s)
    return (round_f16(xb / scale) * scale).reshape(x.shape)


def q4k_fields(blocks: np.ndarray):
    """Decode the fields of Q4_K blocks.

    blocks: uint8 [..., 144].  Returns (d, dmin, sc, m, q) with d, dmin fp64
    [...], sc, m int64 [..., 8] and q int64 [..., 256].
    """
    b = np.asarray(blocks, dtype=np.uint8)
    assert b.shape[-1] == Q4K_BLOCK_BYTES
    bw = b.astype(np.uint32)
    d = f16_bits_to_f64(bw[..., 0] | (bw[..., 1] << 8))
    dmin = f16_bits_to_f64(bw[..., 2] | (bw[..., 3] << 8))
    sc = np.empty(b.shape[:-1] + (8,), dtype=np.int64)
    m = np.empty(b.shape[:-1] + (8,), dtype=np.int64)
    for p in range(4):
        g = bw[..., 4 + 3 * p] | (bw[..., 5 + 3 * p] << 8) | (bw[..., 6 + 3 * p] << 16)
        sc[..., 2 * p] = g & 63
        sc[..., 2 * p + 1] = (g >> 6) & 63
        m[..., 2 * p] = (g >> 12) & 63
        m[..., 2 * p + 1] = (g >> 18) & 63
    words = bw[..., 16:].reshape(b.shape[:-1] + (32, 4))
    w = words[..., 0] | (words[..., 1] << 8) | (words[..., 2] << 16) | (words[..., 3] << 24)
    q = np.empty(b.shape[:-1] + (QK_K,), dtype=np.int64)
    for par in range(2):
        for i in range(4):
            q[..., _Q_INDEX[:, par, i]] = (w >> (16 * par + 4 * i)) & 15
    return d, dmin, sc, m, q


def q4k_dequant_blocks(blocks: np.ndarray) -> np.ndarray:
    """w = d*sc*q - dmin*m for every weight, exact in fp64.

    Both products are integer multiples of 2^-24 below 2^26 in magnitude (an
    fp16 value times an integer <= 945 or <= 63), so each product and their
    difference fit in 53 bits: no rounding happens.
    """
    d, dmin, sc, m, q = q4k_fields(blocks)
    sc_w = np.repeat(sc, 32, axis=-1).astype(np.float64)
    m_w = np.repeat(m, 32, axis=-1).astype(np.float64)
    return d[..., None] * (sc_w * q) - dmin[..., None] * m_w


def q4k_matrix_blocks(mat: np.ndarray, n_rows: int, n_cols: int) -> np.ndarray:
    """Row-major view of a row-tiled Q4_K matrix: uint8 [n_rows, n_cols/256, 144]."""
    t = np.asarray(mat, dtype=np.uint8).reshape(n_rows // ROW_TILE, n_cols // QK_K, ROW_TILE,
                                                 Q4K_BLOCK_BYTES)
    return t.transpose(0, 2, 1, 3).reshape(n_rows, n_cols // QK_K, Q4K_BLOCK_BYTES)


def q4k_dequant_rows(mat: np.ndarray, n_rows: int, n_cols: int, rows=None) -> np.ndarray:
    """Dequantized rows of a row-tiled Q4_K matrix as fp64 [len(rows), n_cols]."""
    blocks = q4k_matrix_blocks(mat, n_rows, n_cols)
    if rows is not None:
        blocks = blocks[rows]
    return q4k_dequant_blocks(blocks).reshape(blocks.shape[0], n_cols)


def q8_0_dequant(q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """q int8 [..., n], d fp16 [..., n/32] -> fp64 d*q (exact)."""
    q = np.asarray(q)
    dd = np.asarray(d, dtype=np.float16).astype(np.float64)
    qq = q.astype(np.float64).reshape(q.shape[:-1] + (q.shape[-1] // Q8_BLOCK, Q8_BLOCK))
    return (qq * dd[..., None]).reshape(q.shape)


def q8_0_quantize(x: np.ndarray):
    """Quantize values to Q8_0 along the last axis (blocks of 32), in fp64.

    Per block: amax = max |x|; d = amax/127 rounded to fp16 (nearest-even);
    q = x/d rounded half away from zero and clamped to [-127, 127]; a block whose
    fp16 scale is zero stores q = 0.  Returns (q int8 [..., n], d fp16 [..., n/32]).
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    assert n % Q8_BLOCK == 0
    xb = x.reshape(x.shape[:-1] + (n // Q8_BLOCK, Q8_BLOCK))
    amax = np.max(np.abs(xb), axis=-1)
    d16 = (amax / 127.0).astype(np.float16)
    d = d16.astype(np.float64)[..., None]
    safe = np.where(d == 0.0, 1.0, d)
    y = xb / safe
    t = np.trunc(y)
    frac = np.abs(y - t)
    r = t + np.sign(y) * (frac >= 0.5)
    r = np.clip(r, -127, 127)
    r = np.where(d == 0.0, 0.0, r)
    return r.astype(np.int8).reshape(x.shape), d16


FP8_MAX = 448.0


def fp8_e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 E4M3 codes -> fp64 values (exact; NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def fp8_e4m3_encode(x: np.ndarray) -> np.ndarray:
    """fp64 values -> uint8 E4M3 codes: round to nearest, ties to even,
    magnitudes above 448 saturate to 448 (NaN -> 0x7F, sign kept).

    Below 2^-6 the grid is the subnormal step 2^-9; from 2^e (e >= -6) to
    2^(e+1) it is 2^(e-3).  A magnitude that rounds up to the next power of
    two lands on that binade's first code (code arithmetic carries into the
    exponent field)."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), FP8_MAX)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, a)
    _, ex = np.frexp(a)                      # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)               # binade floor(log2 a), at least -6
    step = np.exp2((e - 3).astype(np.float64))
    q = np.rint(a / step).astype(np.int64)   # rint: ties to even
    sub = a < 2.0 ** -6
    code = np.where(sub, q, ((e + 7) << 3) + q - 8)
    code = np.where(nan, 0x7F, code)
    return (code | (neg.astype(np.int64) << 7)).astype(np.uint8)
