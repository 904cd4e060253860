"""Pins for the oracle's decode step (CPU only).

* batch invariance, bitwise: a batched step equals B single-sequence steps;
* an identity network (zero output projections) reduces the step to
  embedding -> final RMSNorm -> LM head -> argmax, checked directly;
* a pure-Python brute force of a micro model built from Q4_K *fields* (not
  bytes), fp16 rounding via ``struct``'s half format, Q8_0 via exact rationals.
"""
import copy
import math
import struct
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import step as S
from tests.test_oracle_formats import pack_q4k


def f16(x: float) -> float:
    return struct.unpack("<e", struct.pack("<e", x))[0]


def _toy(seed=1000, kind="f16", n_layers=None, batch=2, length=128):
    dims = synth.TOY
    model = synth.make_model(dims, seed, n_layers=n_layers)
    st = synth.Streams(seed + 7)
    cap = length + 8
    filled = [length] * batch
    caches = []
    for _ in model.layers:
        caches.append(synth.kv_cache(kind, st.next(), st.next(), batch, dims.n_kv_heads, cap, dims.head_dim,
                                     filled))
    tok = synth.tokens(st.next(), batch, dims.vocab)
    return model, caches, tok


@pytest.mark.parametrize("kind", ["f16", "q8_0", "fp8"])
def test_batch_invariance_bitwise(kind):
    model, caches, tok = _toy(kind=kind)
    slots = np.array([0, 1])
    pos = np.array([128, 128])
    c_batch = copy.deepcopy(caches)
    lg, nt = S.decode_step(model, c_batch, kind, slots, pos, tok)
    for b in range(2):
        c_one = copy.deepcopy(caches)
        lg1, nt1 = S.decode_step(model, c_one, kind, slots[b:b + 1], pos[b:b + 1], tok[b:b + 1])
        assert np.array_equal(lg1[0], lg[b])
        assert nt1[0] == nt[b]
        for ca, cb in zip(c_one, c_batch):
            for name in vars(ca):
                assert np.array_equal(getattr(ca, name)[b], getattr(cb, name)[b])


def test_identity_network_reduces_to_lm_head():
    model, caches, tok = _toy()
    for ly in model.layers:
        ly.w_o = np.zeros_like(ly.w_o)
        ly.w_down = np.zeros_like(ly.w_down)
    lg, nt = S.decode_step(model, caches, "f16", np.array([0, 1]), np.array([128, 128]), tok)
    dims = model.dims
    for b in range(2):
        x = model.embed[tok[b]].astype(np.float64)
        ms = math.fsum(float(v) * float(v) for v in x) / dims.hidden
        hf = [f16(float(model.norm_final[i]) * float(x[i]) / math.sqrt(ms + dims.rms_eps))
              for i in range(dims.hidden)]
        want = np.array([math.fsum(hf[i] * float(model.lm_head[v, i]) for i in range(dims.hidden))
                         for v in range(0, dims.vocab, 97)])
        assert np.allclose(lg[b, ::97], want, rtol=1e-12, atol=1e-12)
        assert nt[b] == int(np.argmax(lg[b]))


# ---------------------------------------------------------------- micro-model brute force
MICRO = synth.ModelDims(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                        ffn=256, vocab=64)


class FieldMatrix:
    """A Q4_K matrix kept as fields, plus its packed row-tiled bytes for the oracle."""

    def __init__(self, rng, n, k):
        self.n, self.k = n, k
        kb = k // 256
        self.d = rng.integers(0, 0x1C00, (n, kb))       # fp16 bit patterns, positive, small
        self.dmin = rng.integers(0, 0x1C00, (n, kb))
        self.sc = rng.integers(0, 64, (n, kb, 8))
        self.m = rng.integers(0, 64, (n, kb, 8))
        self.q = rng.integers(0, 16, (n, kb, 256))
        rows = np.zeros((n, kb, 144), np.uint8)
        for r in range(n):
            for c in range(kb):
                rows[r, c] = np.frombuffer(pack_q4k(int(self.d[r, c]), int(self.dmin[r, c]), self.sc[r, c],
                                                    self.m[r, c], self.q[r, c]), np.uint8)
        self.bytes = np.ascontiguousarray(rows.reshape(n // 16, 16, kb, 144).transpose(0, 2, 1, 3))
        hb = lambda b: struct.unpack("<e", struct.pack("<H", int(b)))[0]
        self.w = [[hb(self.d[r, c // 256]) * int(self.sc[r, c // 256, (c % 256) // 32]) * int(self.q[r, c // 256, c % 256])
                   - hb(self.dmin[r, c // 256]) * int(self.m[r, c // 256, (c % 256) // 32])
                   for c in range(k)] for r in range(n)]

    def matvec(self, x):
        return [math.fsum(wi * xi for wi, xi in zip(row, x)) for row in self.w]


def _q8_brute(vals):
    amax = max(abs(v) for v in vals)
    d = f16(amax / 127.0)
    if d == 0.0:
        return [0] * len(vals), 0.0
    out = []
    for v in vals:
        y = Fraction(v / d)
        r = math.floor(abs(y) + Fraction(1, 2))
        out.append(int(math.copysign(min(r, 127), v)) if r else 0)
    return out, d


def _fp8_values():
    """(code, value) of every finite E4M3 code, from the format's definition:
    bias 7, subnormal at exponent field 0, S.1111.111 NaN."""
    out = []
    for code in range(256):
        sgn, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            continue
        mag = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        out.append((code, -mag if sgn else mag))
    return out


_FP8 = _fp8_values()


def _fp8_brute(x: float) -> float:
    """Nearest finite E4M3 value (ties: the even code), magnitudes past 448 to +-448."""
    a = min(abs(x), 448.0)
    t = math.copysign(a, x)
    best = min(abs(v - t) for _, v in _FP8)
    cands = [(c, v) for c, v in _FP8 if abs(v - t) == best]
    if len(cands) > 1:
        cands = [(c, v) for c, v in cands if c % 2 == 0]
    return cands[0][1]


def _fp8_code_value(c: int) -> float:
    return dict(_FP8)[int(c)]


def _brute_step(mdl, cache, kind, slots, pos, tok):
    dm = MICRO
    hq, hkv, hd, f = dm.n_q_heads, dm.n_kv_heads, dm.head_dim, dm.ffn
    logits, toks = [], []
    for b in range(len(tok)):
        x = [float(v) for v in mdl["embed"][tok[b]]]
        p = int(pos[b])
        slot = int(slots[b])
        for li, ly in enumerate(mdl["layers"]):
            def norm(vec, g):
                ms = math.fsum(v * v for v in vec) / len(vec)
                return [f16(float(g[i]) * vec[i] / math.sqrt(ms + dm.rms_eps)) for i in range(len(vec))]
            h = norm(x, ly["norm_attn"])
            qkv = ly["w_qkv"].matvec(h)

            def rot(vec):
                out = list(vec)
                for i in range(hd // 2):
                    a = p * dm.rope_base ** (-2.0 * i / hd)
                    c, s = math.cos(a), math.sin(a)
                    out[i] = vec[i] * c - vec[i + hd // 2] * s
                    out[i + hd // 2] = vec[i + hd // 2] * c + vec[i] * s
                return out
            qs = [rot(qkv[hh * hd:(hh + 1) * hd]) for hh in range(hq)]
            ks = [rot(qkv[(hq + g) * hd:(hq + g + 1) * hd]) for g in range(hkv)]
            vs = [qkv[(hq + hkv + g) * hd:(hq + hkv + g + 1) * hd] for g in range(hkv)]
            for g in range(hkv):   # append, then read back as the attention sees it
                if kind == "f16":
                    cache[li]["k"][slot][g][p] = [f16(v) for v in ks[g]]
                    cache[li]["v"][slot][g][p] = [f16(v) for v in vs[g]]
                elif kind == "fp8":
                    cache[li]["k"][slot][g][p] = [_fp8_brute(v) for v in ks[g]]
                    cache[li]["v"][slot][g][p] = [_fp8_brute(v) for v in vs[g]]
                else:
                    for name, src in (("k", ks[g]), ("v", vs[g])):
                        row = []
                        for blk in range(hd // 32):
                            qv, dd = _q8_brute(src[32 * blk:32 * blk + 32])
                            row += [dd * qq for qq in qv]
                        cache[li][name][slot][g][p] = row
            o = []
            for hh in range(hq):
                g = hh // (hq // hkv)
                qv = [f16(v) for v in qs[hh]]
                sc = [math.fsum(qv[i] * cache[li]["k"][slot][g][t][i] for i in range(hd)) / math.sqrt(hd)
                      for t in range(p + 1)]
                mx = max(sc)
                e = [math.exp(s - mx) for s in sc]
                tot = math.fsum(e)
                o += [f16(math.fsum(e[t] * cache[li]["v"][slot][g][t][i] for t in range(p + 1)) / tot)
                      for i in range(hd)]
            x = [a + c for a, c in zip(x, ly["w_o"].matvec(o))]
            h2 = norm(x, ly["norm_ffn"])
            gu = ly["w_gate_up"].matvec(h2)
            act = []
            for i in range(f):
                z = gu[i]
                sil = z / (1.0 + math.exp(-z)) if z >= 0 else z * math.exp(z) / (1.0 + math.exp(z))
                act.append(f16(sil * gu[f + i]))
            x = [a + c for a, c in zip(x, ly["w_down"].matvec(act))]
        ms = math.fsum(v * v for v in x) / len(x)
        hf = [f16(float(mdl["norm_final"][i]) * x[i] / math.sqrt(ms + dm.rms_eps)) for i in range(len(x))]
        lg = [math.fsum(hf[i] * float(mdl["lm_head"][v, i]) for i in range(len(x))) for v in range(dm.vocab)]
        logits.append(lg)
        toks.append(max(range(dm.vocab), key=lambda v: (lg[v], -v)))
    return np.array(logits), np.array(toks)


@pytest.mark.parametrize("kind", ["f16", "q8_0", "fp8"])
def test_micro_model_brute_force(kind):
    rng = np.random.default_rng(77)
    dm = MICRO
    hq, hkv, hd = dm.n_q_heads, dm.n_kv_heads, dm.head_dim
    mdl = {"embed": rng.standard_normal((dm.vocab, dm.hidden)).astype(np.float16),
           "lm_head": (rng.standard_normal((dm.vocab, dm.hidden)) / 16).astype(np.float16),
           "norm_final": (1 + 0.1 * rng.standard_normal(dm.hidden)).astype(np.float32), "layers": []}
    for _ in range(dm.n_layers):
        mdl["layers"].append({
            "w_qkv": FieldMatrix(rng, (hq + 2 * hkv) * hd, dm.hidden),
            "w_o": FieldMatrix(rng, dm.hidden, hq * hd),
            "w_gate_up": FieldMatrix(rng, 2 * dm.ffn, dm.hidden),
            "w_down": FieldMatrix(rng, dm.hidden, dm.ffn),
            "norm_attn": (1 + 0.1 * rng.standard_normal(dm.hidden)).astype(np.float32),
            "norm_ffn": (1 + 0.1 * rng.standard_normal(dm.hidden)).astype(np.float32)})
    model = synth.ModelWeights(dims=dm, embed=mdl["embed"], lm_head=mdl["lm_head"], norm_final=mdl["norm_final"],
                               layers=[synth.LayerWeights(w_qkv=ly["w_qkv"].bytes, w_o=ly["w_o"].bytes,
                                                          w_gate_up=ly["w_gate_up"].bytes, w_down=ly["w_down"].bytes,
                                                          norm_attn=ly["norm_attn"], norm_ffn=ly["norm_ffn"])
                                       for ly in mdl["layers"]])
    n_slots, cap, length = 3, 8, 3
    st = synth.Streams(5)
    caches, bf_cache = [], []
    for _ in range(dm.n_layers):
        if kind == "f16":
            c = synth.kv_cache_f16(st.next(), st.next(), n_slots, hkv, cap, hd, [length] * n_slots)
            kk, vv = c.k.astype(np.float64), c.v.astype(np.float64)
        elif kind == "fp8":
            c = synth.kv_cache_fp8(st.next(), st.next(), n_slots, hkv, cap, hd, [length] * n_slots)
            kk = np.vectorize(_fp8_code_value, otypes=[np.float64])(c.kf8)
            vv = np.vectorize(_fp8_code_value, otypes=[np.float64])(c.vf8)
        else:
            c = synth.kv_cache_q8(st.next(), st.next(), n_slots, hkv, cap, hd, [length] * n_slots)
            kk = c.kq.astype(np.float64) * np.repeat(c.ks.astype(np.float64), 32, axis=-1)
            vv = c.vq.astype(np.float64) * np.repeat(c.vs.astype(np.float64), 32, axis=-1)
        caches.append(c)
        bf_cache.append({"k": kk.tolist(), "v": vv.tolist()})
    slots, pos = np.array([2, 0]), np.array([3, 3])
    tok = np.array([5, 17])
    for stepno in range(2):
        lg, nt = S.decode_step(model, caches, kind, slots, pos, tok)
        lb, tb = _brute_step(mdl, bf_cache, kind, slots, pos, tok)
        assert np.allclose(lg, lb, rtol=1e-9, atol=1e-9), np.abs(lg - lb).max()
        assert (nt == tb).all()
        for li in range(dm.n_layers):   # the appended entries agree exactly
            for b, s in enumerate(slots):
                p = int(pos[b])
                if kind == "f16":
                    got_k = caches[li].k[s, :, p].astype(np.float64)
                elif kind == "fp8":
                    got_k = np.vectorize(_fp8_code_value, otypes=[np.float64])(caches[li].kf8[s, :, p])
                else:
                    got_k = caches[li].kq[s, :, p].astype(np.float64) * np.repeat(
                        caches[li].ks[s, :, p].astype(np.float64), 32, axis=-1)
                assert np.array_equal(got_k, np.array(bf_cache[li]["k"][s])[:, p])
        pos = pos + 1
        tok = nt


@pytest.mark.parametrize("kind,kfrom,vfrom", [("q8k_f16v", "q8_0", "f16"), ("f16k_q8v", "f16", "q8_0")])
def test_mixed_cache_formats_route_each_tensor(kind, kfrom, vfrom):
    # keys and values in different formats: appending and reading a mixed cache
    # must give, tensor by tensor, exactly what the pure fp16 and Q8_0 caches give
    # (a swapped format or tensor would fail)
    st = synth.Streams(7100)
    n_slots, n_kv, cap, hd = 2, 2, 64, 64
    f16c = synth.kv_cache("f16", st.next(), st.next(), n_slots, n_kv, cap, hd, [40, 17])
    q8c = synth.kv_cache("q8_0", st.next(), st.next(), n_slots, n_kv, cap, hd, [40, 17])
    pure = {"f16": f16c, "q8_0": q8c}
    mixed = synth.KVLayerMixed()
    for name, src in (("k", pure[kfrom]), ("v", pure[vfrom])):
        for f in (name, name + "q", name + "s"):
            if hasattr(src, f):
                setattr(mixed, f, getattr(src, f).copy())
    rng = st.next()
    for slot, pos in ((0, 40), (1, 17), (1, 63)):
        k = rng.standard_normal((n_kv, hd)) * 3.0
        v = rng.standard_normal((n_kv, hd)) * 0.01
        S.kv_append(mixed, kind, slot, pos, k, v)
        S.kv_append(pure[kfrom], kfrom, slot, pos, k, v)
        S.kv_append(pure[vfrom], vfrom, slot, pos, k, v)
        km, vm = S.kv_read(mixed, kind, slot, pos + 1)
        assert np.array_equal(km, S.kv_read(pure[kfrom], kfrom, slot, pos + 1)[0])
        assert np.array_equal(vm, S.kv_read(pure[vfrom], vfrom, slot, pos + 1)[1])
    with pytest.raises(ValueError):
        S.kv_read(mixed, "q4_0", 0, 1)


@pytest.mark.parametrize("kind", ["f16", "q8_0", "fp8", "q8k_f16v"])
def test_paged_read_is_the_contiguous_cache_split_into_pages(kind):
    # a slot of capacity C cut into pages of P tokens, the pages scattered over
    # a shuffled pool: every paged read, append and attention equals the
    # contiguous one exactly
    st = synth.Streams(7300)
    n_slots, n_kv, cap, hd, P = 2, 2, 128, 64, 32
    cont = synth.kv_cache(kind, st.next(), st.next(), n_slots, n_kv, cap, hd, [100, 128])
    npp = cap // P
    perm = st.next().permutation(n_slots * npp)          # logical page j of slot s -> physical perm[s*npp+j]
    pool = copy.deepcopy(cont)
    for name, arr in vars(cont).items():
        if arr is None:
            continue
        pages = arr.reshape((n_slots, n_kv, npp, P) + arr.shape[3:]).transpose(0, 2, 1, 3, 4)
        pages = pages.reshape((n_slots * npp, n_kv, P) + arr.shape[3:])
        phys = np.empty_like(pages)
        phys[perm] = pages
        setattr(pool, name, phys)
    table = [perm[s * npp:(s + 1) * npp] for s in range(n_slots)]
    rng = st.next()
    for s, n in ((0, 100), (1, 128), (0, 1), (1, 33)):
        kc, vc = S.kv_read(cont, kind, s, n)
        kp, vp = S.kv_read_paged(pool, kind, table[s], P, n)
        assert np.array_equal(kc, kp) and np.array_equal(vc, vp)
    k = rng.standard_normal((n_kv, hd)) * 2
    v = rng.standard_normal((n_kv, hd))
    S.kv_append(cont, kind, 0, 100, k, v)
    S.kv_append_paged(pool, kind, table[0], P, 100, k, v)
    q = rng.standard_normal((2, 4, hd))
    a = S.attention_batch(q, cont, kind, [0, 1], [101, 77], 0.125)
    b = S.attention_batch_paged(q, pool, kind, table, P, [101, 77], 0.125)
    assert np.array_equal(a, b)


def _scatter_into_pool(cont, n_slots, P, perm):
    """The slots of a contiguous cache cut into pages of P tokens, page j of
    slot s stored at physical page perm[s * npp + j] of a pool."""
    pool = copy.deepcopy(cont)
    for name, arr in vars(cont).items():
        if arr is None:
            continue
        npp = arr.shape[2] // P
        pages = arr.reshape((n_slots, arr.shape[1], npp, P) + arr.shape[3:]).transpose(0, 2, 1, 3, 4)
        pages = pages.reshape((n_slots * npp, arr.shape[1], P) + arr.shape[3:])
        phys = np.empty_like(pages)
        phys[perm] = pages
        setattr(pool, name, phys)
    return pool


@pytest.mark.parametrize("kind", ["f16", "q8_0", "fp8"])
def test_unmapped_pages_drop_out_of_the_context(kind):
    # a table entry of -1 (or past the pool) maps nothing: the paged read is the
    # contiguous read with that page's tokens removed (picked out by index here),
    # attention over it equals attention over exactly those tokens, a store to it
    # is dropped, and a sequence with no mapped page attends to nothing (O = 0)
    st = synth.Streams(7310)
    n_slots, n_kv, cap, hd, P = 2, 2, 128, 64, 32
    cont = synth.kv_cache(kind, st.next(), st.next(), n_slots, n_kv, cap, hd, [128, 128])
    npp = cap // P
    perm = st.next().permutation(n_slots * npp)
    pool = _scatter_into_pool(cont, n_slots, P, perm)
    table = np.array([perm[s * npp:(s + 1) * npp] for s in range(n_slots)])
    holed = table.copy()
    holed[0, 1] = -1                    # tokens 32..63 of sequence 0
    holed[1, 3] = n_slots * npp         # past the pool: tokens 96..127 of sequence 1
    keep0 = np.r_[0:32, 64:100]
    kc, vc = S.kv_read(cont, kind, 0, 128)
    kp, vp = S.kv_read_paged(pool, kind, holed[0], P, 100)
    assert np.array_equal(kp, kc[:, keep0]) and np.array_equal(vp, vc[:, keep0])
    rng = st.next()
    q = rng.standard_normal((2, 4, hd))
    got = S.attention_batch_paged(q, pool, kind, holed, P, [100, 128], 0.125)
    kc1, vc1 = S.kv_read(cont, kind, 1, 96)
    assert np.array_equal(got[0], S.attention(q[0], kc[:, keep0], vc[:, keep0], 0.125))
    assert np.array_equal(got[1], S.attention(q[1], kc1, vc1, 0.125))
    before = copy.deepcopy(pool)
    assert not S.kv_append_paged(pool, kind, holed[0], P, 40, rng.standard_normal((n_kv, hd)),
                                 rng.standard_normal((n_kv, hd)))
    assert not S.kv_append_paged(pool, kind, holed[0], P, cap, rng.standard_normal((n_kv, hd)),
                                 rng.standard_normal((n_kv, hd)))
    for name in vars(pool):
        if getattr(pool, name) is not None:
            assert np.array_equal(getattr(pool, name), getattr(before, name))
    none = np.full((1, npp), -1)
    assert not S.attention_batch_paged(q[:1], pool, kind, none, P, [77], 0.125).any()


@pytest.mark.parametrize("kind", ["f16", "q8_0"])
def test_paged_decode_step_equals_arena_step(kind):
    # the toy decoder over pools whose pages hold the arena's slots scattered:
    # logits, tokens and every stored entry equal the slot-arena step bitwise
    model, caches, tok = _toy(kind=kind, length=120)     # capacity 128: four pages of 32
    P = 32
    cap = caches[0].k.shape[2] if getattr(caches[0], "k", None) is not None else caches[0].kq.shape[2]
    cap = cap // P * P
    for c in caches:
        for name, arr in vars(c).items():
            if arr is not None:
                setattr(c, name, np.ascontiguousarray(arr[:, :, :cap]))
    npp = cap // P
    perm = np.random.default_rng(7320).permutation(2 * npp)
    pools = [_scatter_into_pool(c, 2, P, perm) for c in caches]
    table = np.array([perm[s * npp:(s + 1) * npp] for s in range(2)])
    pos = np.array([120, 120])
    lg_a, nt_a = S.decode_step(model, caches, kind, [0, 1], pos, tok)
    lg_p, nt_p = S.decode_step_paged(model, pools, kind, table, P, pos, tok)
    assert np.array_equal(lg_a, lg_p) and np.array_equal(nt_a, nt_p)
    for c, pl in zip(caches, pools):
        again = _scatter_into_pool(c, 2, P, perm)
        for name in vars(c):
            if getattr(c, name) is not None:
                assert np.array_equal(getattr(pl, name), getattr(again, name))


@pytest.mark.parametrize("kind", ["f16", "q8_0"])
def test_prefill_is_one_step_over_the_prompt_rows(kind):
    # the prompt's tokens as the rows of one decode step (same slot,
    # consecutive positions) give bitwise the sequential prefill: row b's
    # keys and values are appended before any later row attends, and each
    # row's arithmetic is its own
    model, caches, _ = _toy(kind=kind, batch=1, length=20)
    for c in caches:
        for name, arr in vars(c).items():
            if arr is not None:
                pad = np.zeros(arr.shape[:2] + (64,) + arr.shape[3:], arr.dtype)
                setattr(c, name, np.concatenate([arr, pad], axis=2))
    prompt = synth.tokens(np.random.default_rng(3), 12, model.dims.vocab)
    seq = copy.deepcopy(caches)
    lg, nt = S.prefill(model, seq, kind, 0, 20, prompt)
    rows = copy.deepcopy(caches)
    lg_rows, nt_rows = S.decode_step(model, rows, kind, [0] * 12, 20 + np.arange(12), prompt)
    assert np.array_equal(lg_rows[-1], lg) and nt_rows[-1] == nt
    for a, b in zip(seq, rows):
        for name in vars(a):
            if getattr(a, name) is not None:
                assert np.array_equal(getattr(a, name), getattr(b, name))
