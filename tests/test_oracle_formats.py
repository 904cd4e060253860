"""Pins for the oracle's storage-format decoding (CPU only).

The Q4_K byte layout is this library's own (documented in include/qkdec.h and
oracle/formats.py).  The packer below is written independently of the
decoder, bit by bit with Python integers, from that written description.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F


# ---------------------------------------------------------------- helpers written for the tests
def pack_q4k(d_bits: int, dmin_bits: int, sc, m, q) -> bytes:
    """Independent Q4_K packer: build the 1152-bit block as one Python integer."""
    acc = d_bits | (dmin_bits << 16)
    bit = 32
    for p in range(4):
        for val in (sc[2 * p], sc[2 * p + 1], m[2 * p], m[2 * p + 1]):
            assert 0 <= val < 64
            acc |= int(val) << bit
            bit += 6
    assert bit == 128
    for k in range(256):
        word, r = divmod(k, 8)
        half, nib = r % 2, r // 2
        acc |= int(q[k]) << (128 + 32 * word + 16 * half + 4 * nib)
    return acc.to_bytes(144, "little")


def f16_value(bits: int) -> Fraction:
    """Exact value of an fp16 bit pattern (finite only)."""
    s = -1 if bits >> 15 else 1
    e = (bits >> 10) & 31
    f = bits & 1023
    assert e != 31
    if e == 0:
        return s * Fraction(f, 1 << 24)
    return s * Fraction(1024 + f, 1 << 10) * Fraction(2) ** (e - 15)


def rne_f16_bits(x: Fraction) -> int:
    """Round-to-nearest-even of an exact rational to fp16 bits (by enumeration of neighbours)."""
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    if a >= Fraction(65520):
        return sign | 0x7C00
    # find the largest finite magnitude pattern with value <= a
    lo, hi = 0, 0x7BFF
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if f16_value(mid) <= a:
            lo = mid
        else:
            hi = mid - 1
    below = lo
    if f16_value(below) == a:
        return sign | below
    above = below + 1
    vb, va = f16_value(below), (f16_value(above) if above <= 0x7BFF else Fraction(65536))
    if a - vb < va - a:
        return sign | below
    if a - vb > va - a:
        return sign | (above if above <= 0x7BFF else 0x7C00)
    return sign | (below if below % 2 == 0 else above)


# ---------------------------------------------------------------- fp16 rounding
def test_f64_to_f16_is_one_correct_rounding():
    rng = np.random.default_rng(7)
    vals = list(rng.standard_normal(300) * 10.0 ** rng.integers(-9, 5, 300))
    # exact midpoints between neighbouring fp16 values and their double neighbours
    for bits in list(rng.integers(1, 0x7BFE, 200)) + [0, 1, 2, 0x3FF, 0x400, 0x3C00, 0x7BFE]:
        mid = (f16_value(int(bits)) + f16_value(int(bits) + 1)) / 2
        m = float(mid)
        vals += [m, np.nextafter(m, 0.0), np.nextafter(m, np.inf), -m]
    vals += [65504.0, 65519.99, 65520.0, 1e-9, 2.0 ** -25, 2.0 ** -25 * 1.0000001]
    with np.errstate(over="ignore"):
        for v in vals:
            got = int(np.float64(v).astype(np.float16).view(np.uint16))
            assert got == rne_f16_bits(Fraction(float(v))), v
            assert F.round_f16(v) == float(np.float16(np.float64(v)))


# ---------------------------------------------------------------- Q4_K layout
def test_q4k_hand_built_positions():
    z = bytearray(144)

    def decode(buf):
        d, dmin, sc, m, q = F.q4k_fields(np.frombuffer(bytes(buf), np.uint8))
        return d, dmin, list(sc), list(m), list(q)

    cases = [  # (byte index, byte value, field, index, value)
        (16, 0x01, "q", 0, 1), (16, 0x10, "q", 2, 1), (17, 0x01, "q", 4, 1), (17, 0x80, "q", 6, 8),
        (18, 0x01, "q", 1, 1), (18, 0x10, "q", 3, 1), (19, 0x10, "q", 7, 1), (19, 0x0F, "q", 5, 15),
        (20, 0x03, "q", 8, 3), (143, 0xF0, "q", 255, 15), (142, 0x0F, "q", 249, 15), (143, 0x05, "q", 253, 5),
        (141, 0x10, "q", 254, 1), (140, 0x01, "q", 248, 1),
        (4, 0x3F, "sc", 0, 63), (4, 0x40, "sc", 1, 1), (5, 0x0F, "sc", 1, 60), (5, 0x10, "m", 0, 1),
        (6, 0x03, "m", 0, 48), (6, 0x04, "m", 1, 1), (6, 0xFC, "m", 1, 63),
        (7, 0x01, "sc", 2, 1), (13, 0x01, "sc", 6, 1), (15, 0x80, "m", 7, 32), (12, 0xC0, "m", 5, 48),
    ]
    for bidx, bval, field, idx, val in cases:
        buf = bytearray(z)
        buf[bidx] = bval
        d, dmin, sc, m, q = decode(buf)
        got = {"q": q, "sc": sc, "m": m}
        for name, arr in got.items():
            for i, x in enumerate(arr):
                want = val if (name == field and i == idx) else 0
                assert x == want, (bidx, bval, name, i, x, want)
        assert d == 0 and dmin == 0


def test_q4k_one_hot_every_bit():
    # every one of the 1120 field bits changes exactly one field by a power of two
    seen = set()
    for bit in range(32, 1152):
        acc = 1 << bit
        buf = np.frombuffer(acc.to_bytes(144, "little"), np.uint8)
        _, _, sc, m, q = F.q4k_fields(buf)
        nz = [(n, i, int(v)) for n, arr in (("sc", sc), ("m", m), ("q", q)) for i, v in enumerate(arr) if v]
        assert len(nz) == 1, bit
        n, i, v = nz[0]
        assert v & (v - 1) == 0
        seen.add((n, i, v))
    assert len(seen) == 1120


def test_q4k_packer_decoder_bijection():
    rng = np.random.default_rng(11)
    for _ in range(50):
        sc = rng.integers(0, 64, 8)
        m = rng.integers(0, 64, 8)
        q = rng.integers(0, 16, 256)
        db, mb = (int(x) for x in rng.integers(0, 0x7C00, 2))
        blk = np.frombuffer(pack_q4k(db, mb, sc, m, q), np.uint8)
        d, dmin, sc2, m2, q2 = F.q4k_fields(blk)
        assert (sc2 == sc).all() and (m2 == m).all() and (q2 == q).all()
        assert d == float(f16_value(db)) and dmin == float(f16_value(mb))
    raw = rng.integers(0, 256, (20, 144), dtype=np.uint8)
    for row in raw:
        d, dmin, sc, m, q = F.q4k_fields(row)
        db = int(row[0]) | int(row[1]) << 8
        mb = int(row[2]) | int(row[3]) << 8
        assert pack_q4k(db, mb, sc, m, q) == row.tobytes()


def test_q4k_closed_forms():
    rng = np.random.default_rng(3)
    q = rng.integers(0, 16, 256)
    one = 0x3C00
    sc = rng.integers(0, 64, 8)
    w = F.q4k_dequant_blocks(np.frombuffer(pack_q4k(one, 0, sc, [0] * 8, q), np.uint8))
    assert (w == np.repeat(sc, 32) * q).all()
    sc = np.arange(1, 9)
    m = np.arange(0, 8)
    w = F.q4k_dequant_blocks(np.frombuffer(pack_q4k(one, one, sc, m, q), np.uint8))
    assert (w == np.repeat(sc, 32) * q - np.repeat(m, 32)).all()


def test_q4k_dequant_is_exact():
    rng = np.random.default_rng(5)
    blocks = rng.integers(0, 256, (40, 144), dtype=np.uint8)
    # include subnormal and large scales
    blocks[:10, 1] &= 0x03
    blocks[:10, 3] &= 0x03
    blocks[10:20, 1] = (blocks[10:20, 1] & 0x83) | 0x78
    blocks[10:20, 3] = (blocks[10:20, 3] & 0x83) | 0x78
    w = F.q4k_dequant_blocks(blocks)
    for bi, blk in enumerate(blocks):
        acc = int.from_bytes(blk.tobytes(), "little")
        d = f16_value(acc & 0xFFFF)
        dmin = f16_value((acc >> 16) & 0xFFFF)
        fields = [(acc >> (32 + 6 * i)) & 63 for i in range(16)]
        for k in range(0, 256, 7):
            s = k // 32
            p, r = divmod(s, 2)
            sc = fields[4 * p + r]
            mm = fields[4 * p + 2 + r]
            word, rr = divmod(k, 8)
            qq = (acc >> (128 + 32 * word + 16 * (rr % 2) + 4 * (rr // 2))) & 15
            assert Fraction(w[bi, k]) == d * sc * qq - dmin * mm


def test_q4k_matrix_row_tiling():
    n_rows, n_cols = 48, 768
    tiles = np.zeros((3, 3, 16, 144), np.uint8)
    for t in range(3):
        for c in range(3):
            for r in range(16):
                row = 16 * t + r
                tiles[t, c, r, 0:2] = np.array([row * 8 + c], np.float16).view(np.uint8)
                tiles[t, c, r, 4] = 1  # sc[0] = 1
                tiles[t, c, r, 16] = 1  # q[0] = 1
    w = F.q4k_dequant_rows(tiles, n_rows, n_cols)
    for row in range(n_rows):
        for c in range(3):
            assert w[row, 256 * c] == row * 8 + c
            assert not w[row, 256 * c + 1:256 * (c + 1)].any()
    sub = F.q4k_dequant_rows(tiles, n_rows, n_cols, rows=slice(17, 19))
    assert (sub == w[17:19]).all()


# ---------------------------------------------------------------- Q8_0
def test_q8_0_hand_cases():
    # amax = 127 * 2^e: scale is exactly 2^e and every multiple of 2^e is kept exactly
    x = np.zeros(32)
    x[:5] = [127 * 0.25, -3 * 0.25, 0.0, 100 * 0.25, -127 * 0.25]
    q, d = F.q8_0_quantize(x)
    assert float(d[0]) == 0.25
    assert list(q[:5]) == [127, -3, 0, 100, -127]
    # halves round away from zero
    x = np.zeros(32)
    x[:5] = [127.0, 2.5, -2.5, 0.5, -0.5]
    q, d = F.q8_0_quantize(x)
    assert float(d[0]) == 1.0 and list(q[:5]) == [127, 3, -3, 1, -1]
    # all-zero block
    q, d = F.q8_0_quantize(np.zeros(64))
    assert not q.any() and not d.astype(np.float64).any()
    # subnormal scale that rounds down forces the clamp at 127
    x = np.zeros(32)
    x[0] = 127 * 1.4 * 2.0 ** -24
    x[1] = -x[0]
    q, d = F.q8_0_quantize(x)
    assert float(d[0]) == 2.0 ** -24
    assert q[0] == 127 and q[1] == -127
    # scale rounding to zero stores zeros
    x = np.zeros(32)
    x[0] = 1e-12
    q, d = F.q8_0_quantize(x)
    assert float(d[0]) == 0.0 and not q.any()


def test_q8_0_roundtrip_bound_and_dequant_exact():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((50, 128)) * 10.0 ** rng.integers(-3, 3, (50, 1))
    q, d = F.q8_0_quantize(x)
    y = F.q8_0_dequant(q, d)
    dd = np.repeat(d.astype(np.float64), 32, axis=-1)
    assert (np.abs(y - x) <= 0.5 * dd + np.abs(x) * 2 ** -10).all()
    for i in range(0, 50, 7):
        for j in range(0, 128, 5):
            assert Fraction(y[i, j]) == Fraction(int(q[i, j])) * Fraction(float(d[i, j // 32]))


def test_q8_0_scale_is_rounded_amax_over_127():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((200, 32))
    q, d = F.q8_0_quantize(x)
    for i in range(200):
        amax = Fraction(float(np.max(np.abs(x[i]))))
        assert int(d[i, 0].view(np.uint16)) == rne_f16_bits(amax / 127) or \
            rne_f16_bits(Fraction(float(amax / 127))) == int(d[i, 0].view(np.uint16))
    assert np.abs(q).max() == 127


@pytest.mark.parametrize("shape", [(4, 64), (2, 3, 128)])
def test_q8_0_shapes(shape):
    x = np.random.default_rng(0).standard_normal(shape)
    q, d = F.q8_0_quantize(x)
    assert q.shape == shape and d.shape == shape[:-1] + (shape[-1] // 32,)
    assert q.dtype == np.int8 and d.dtype == np.float16


# ---------------------------------------------------------------- blocked fp16 rounding
def test_blocked_f16_equals_plain_f16_in_range():
    x = np.random.default_rng(3).standard_normal((3, 512)) * 1000
    assert np.array_equal(F.round_f16_blocked(x), F.round_f16(x))


def test_blocked_f16_exponent_offsets():
    x = np.zeros((1, 768))
    x[0, 5] = 1e6          # block 0: 1e6 / 16 = 62500 <= 65504, 1e6 / 8 > 65504 -> s = 4
    x[0, 6] = 3.0          # small value in the same block keeps 11 bits at 2^4 granularity
    x[0, 256] = 65504.0    # block 1: exactly at the limit -> s = 0
    x[0, 512] = 65505.0    # block 2: just above -> s = 1
    x[0, 513] = -1e-3
    y = F.round_f16_blocked(x)
    assert y[0, 5] == 16 * float(np.float16(1e6 / 16))
    assert y[0, 6] == 3.0
    assert y[0, 256] == 65504.0
    assert y[0, 512] == 2 * float(np.float16(65505.0 / 2))
    assert y[0, 513] == 2 * float(np.float16(-1e-3 / 2))
    # every result is an fp16 value times its block's power of two
    for blk, s in ((0, 4), (1, 0), (2, 1)):
        part = y[0, 256 * blk:256 * (blk + 1)] / 2.0 ** s
        assert np.array_equal(part, part.astype(np.float16).astype(np.float64))
    assert np.isfinite(F.round_f16_blocked(np.full((1, 256), 1e30))).all()
    with pytest.raises(AssertionError):
        F.round_f16_blocked(np.zeros(100))


def test_blocked_f16_relative_precision():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((4, 1024)) * 10.0 ** rng.integers(3, 9, (4, 1))
    y = F.round_f16_blocked(x)
    amax = np.abs(x).reshape(4, 4, 256).max(-1, keepdims=True)
    err = np.abs(y - x).reshape(4, 4, 256)
    # normal-range values keep fp16's half-ulp relative error
    big = np.abs(x).reshape(4, 4, 256) > amax * 2.0 ** -10
    assert (err[big] <= np.abs(x.reshape(4, 4, 256))[big] * 2.0 ** -11).all()


# ---- FP8 E4M3 (OCP variant: bias 7, no infinity, S.1111.111 NaN, max 448)

def _finite_codes():
    c = np.arange(256, dtype=np.uint8)
    return c[(c & 0x7F) != 0x7F]


def test_fp8_decode_hand_values():
    d = F.fp8_e4m3_decode(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x39, 0x3F, 0x40, 0x7E, 0xB8, 0xFE],
                                   dtype=np.uint8))
    expect = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.125, 1.875, 2.0, 448.0, -1.0, -448.0]
    assert d.tolist() == expect
    assert np.isnan(F.fp8_e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))).all()
    z = F.fp8_e4m3_decode(np.array([0x80], dtype=np.uint8))
    assert z[0] == 0.0 and np.signbit(z[0])


def test_fp8_decode_matches_torch_float8_e4m3fn():
    torch = pytest.importorskip("torch")
    c = _finite_codes()
    ref = torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(F.fp8_e4m3_decode(c), ref)


def test_fp8_decode_is_monotone_and_distinct():
    c = np.arange(0x7F, dtype=np.uint8)          # non-negative finite codes in order
    v = F.fp8_e4m3_decode(c)
    assert (np.diff(v) > 0).all()


def test_fp8_roundtrip_every_finite_code():
    c = _finite_codes()
    np.testing.assert_array_equal(F.fp8_e4m3_encode(F.fp8_e4m3_decode(c)), c)


def test_fp8_encode_ties_to_even_and_saturation():
    x = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 5 * 2.0 ** -10, 15 * 2.0 ** -10, 1.9375,
                  464.0, 1e9, -1e9, -1.0625, 447.9])
    expect = [0x38, 0x3A, 0x00, 0x02, 0x02, 0x08, 0x40, 0x7E, 0x7E, 0xFE, 0xB8, 0x7E]
    assert F.fp8_e4m3_encode(x).tolist() == expect
    assert F.fp8_e4m3_encode(np.array([np.nan]))[0] == 0x7F


def test_fp8_encode_is_nearest_by_brute_force():
    # every value goes to the nearest finite code (ties: even mantissa), and
    # magnitudes past 448 to +-448
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(4000) * 3, rng.standard_normal(2000) * 100,
                        rng.standard_normal(2000) * 2.0 ** -8, rng.uniform(-600, 600, 500)])
    got = F.fp8_e4m3_encode(x)
    codes = _finite_codes()
    vals = F.fp8_e4m3_decode(codes)
    for xi, gi in zip(x, got):
        a = min(abs(xi), 448.0)
        cand = np.abs(vals - np.copysign(a, xi))
        best = cand.min()
        ties = codes[cand == best]
        if len(ties) > 1:   # +0/-0, or a tie between two neighbours: the even mantissa
            ties = [t for t in ties if (t & 1) == 0 and (np.signbit(xi) == bool(t & 0x80) or a != 0.0)]
        assert gi in ties, (xi, gi, ties)


def test_fp8_encode_matches_torch_in_range():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(20000) * np.exp2(rng.uniform(-12, 8, 20000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(F.fp8_e4m3_encode(x.astype(np.float64)), ref)
