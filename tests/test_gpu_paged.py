"""Paged KV pool on the GPU: attention and append against the oracle, and
against the slot-arena path on the same data."""
import copy
import math

import numpy as np
import pytest

import synth
from oracle import step as OS
from quantized_decode_amd.pager import PagePool
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


def _pool_from(cont, lengths, P, n_pages, rng, room=0):
    """Copy each sequence's tokens of a contiguous cache (slot b = sequence b)
    into pages handed out by a PagePool after some shuffling admissions; the
    pages nobody holds, and every position past a sequence's length, are
    poisoned (NaN or NaN codes)."""
    n_pad = n_pages // 3
    pool = PagePool(n_pages + n_pad, P)
    # scatter the allocations: one-page dummies first, every other one released
    # (n_pad // 2 stay held, so at least n_pages pages are free afterwards)
    for j in range(n_pad):
        pool.admit(("pad", j), int(rng.integers(1, P + 1)))
    for j in range(0, n_pad, 2):
        pool.release(("pad", j))
    for b, n in enumerate(lengths):
        pool.admit(b, n + room)
    max_pages = max(len(pool.pages(b)) for b in range(len(lengths)))
    table = pool.table(range(len(lengths)), max_pages)
    out = copy.deepcopy(cont)
    for name, arr in vars(cont).items():
        if arr is None:
            continue
        if arr.dtype == np.float16:
            poison = np.float16(np.nan)
        elif arr.dtype == np.int8:
            poison = 127
        else:
            poison = 0x7F
        phys = np.full((pool.n_pages,) + arr.shape[1:2] + (P,) + arr.shape[3:], poison, dtype=arr.dtype)
        for b, n in enumerate(lengths):
            for j, pg in enumerate(pool.pages(b)):
                take = max(0, min(P, n - j * P))
                phys[pg, :, :take] = arr[b, :, j * P:j * P + take]
        setattr(out, name, phys)
    return out, table, pool


def _attn_paged(qd, dkv, table, n_ctx, q, scale):
    import torch
    from quantized_decode_amd.tensors import dev
    b, hq, d = q.shape
    qt = dev(q.view(np.uint16)).view(torch.float16)
    o = torch.empty((b, hq, d), dtype=torch.float32, device="cuda")
    mp = table.shape[1]
    w = ws(qd.qkdec_attn_paged_workspace_size(b, hq, dkv.desc, mp))
    qd.qkdec_attn_decode_paged(dkv.desc, _dev(table), mp, _dev(np.asarray(n_ctx, np.int32)), b, qt, hq, scale, o=o,
                               workspace=w)
    sync()
    return o.cpu().numpy()


CASES = [
    ("f16", 8, 2, 64, 32, [1, 31, 200]),
    ("f16", 32, 8, 128, 64, [1000, 65, 128, 3]),
    ("q8_0", 32, 8, 128, 256, [700, 1, 513]),
    ("fp8", 32, 8, 128, 128, [300, 129, 1024]),
    ("fp8", 8, 2, 64, 32, [33, 64, 5]),
    ("q8k_f16v", 16, 4, 128, 64, [257, 90]),
    ("f16", 16, 4, 128, 32, [2000, 1025, 4096, 1024]),   # runs of up to 32 one-tile pages
]


@pytest.mark.parametrize("kind,hq,hkv,d,P,lens", CASES)
def test_paged_attention_matches_oracle(qd, kind, hq, hkv, d, P, lens):
    from quantized_decode_amd.tensors import upload_cache
    st = synth.Streams(8100 + P + d + len(lens))
    cap = max(lens) + P
    cap = (cap + P - 1) // P * P
    cont = synth.kv_cache(kind, st.next(), st.next(), len(lens), hkv, cap, d, lens)
    rng = st.next()
    n_pages = sum((n + P - 1) // P for n in lens) + 12
    pool, table, _ = _pool_from(cont, lens, P, n_pages, rng)
    dkv = upload_cache(pool)
    q = synth.f16_normal(st.next(), (len(lens), hq, d))
    scale = 1 / math.sqrt(d)
    got = _attn_paged(qd, dkv, table, lens, q, scale)
    ref = OS.attention_batch_paged(q.astype(np.float64), pool, kind, table, P, lens, scale)
    assert_rel(got, ref, what=f"paged {kind} P={P} lens={lens}")


@pytest.mark.parametrize("kind", ["f16", "q8_0", "fp8"])
def test_paged_equals_arena_bitwise(qd, kind):
    # the same tokens in a slot arena and scattered over a pool with
    # max_pages * P = capacity: the same runs, tiles and arithmetic
    import torch
    from quantized_decode_amd.tensors import dev, upload_cache
    st = synth.Streams(8200 + len(kind))
    hq, hkv, d, P, lens = 32, 8, 128, 128, [900, 17, 1024, 385]
    cap = 1024
    cont = synth.kv_cache(kind, st.next(), st.next(), len(lens), hkv, cap, d, lens)
    pool, table, _ = _pool_from(cont, lens, P, 40, st.next())
    table = np.pad(table, ((0, 0), (0, cap // P - table.shape[1])), constant_values=-1)
    q = synth.f16_normal(st.next(), (len(lens), hq, d))
    got_p = _attn_paged(qd, upload_cache(pool), table, lens, q, 0.088)
    dkv = upload_cache(cont)
    qt = dev(q.view(np.uint16)).view(torch.float16)
    o = torch.empty((len(lens), hq, d), dtype=torch.float32, device="cuda")
    w = ws(qd.qkdec_attn_workspace_size(len(lens), hq, dkv.desc))
    qd.qkdec_attn_decode(dkv.desc, _dev(np.arange(len(lens), dtype=np.int32)), _dev(np.asarray(lens, np.int32)),
                         len(lens), qt, hq, 0.088, o=o, workspace=w)
    sync()
    assert np.array_equal(got_p.view(np.uint32), o.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("kind", ["f16", "q8_0", "fp8"])
def test_paged_append_bit_exact(qd, kind):
    from quantized_decode_amd.tensors import upload_cache
    st = synth.Streams(8300 + len(kind))
    hkv, d, P, lens = 8, 128, 64, [100, 64, 5]
    cont = synth.kv_cache(kind, st.next(), st.next(), len(lens), hkv, 256, d, lens)
    pool, _, pager = _pool_from(cont, lens, P, 20, st.next())
    for b, n in enumerate(lens):
        pager.reserve(b, n + 1)                     # room for the new token
    table = pager.table(range(len(lens)), 3)
    dkv = upload_cache(pool)
    rng = st.next()
    k = (rng.standard_normal((3, hkv, d)) * 3).astype(np.float32)
    v = rng.standard_normal((3, hkv, d)).astype(np.float32)
    pos = np.array(lens, np.int32)
    err = _dev(np.zeros(1, np.int32))
    qd.qkdec_kv_append_paged(dkv.desc, _dev(table), 3, _dev(pos), _dev(k), _dev(v), 3, err=err)
    sync()
    got = dkv.logical()
    want = copy.deepcopy(pool)
    for b in range(3):
        OS.kv_append_paged(want, kind, table[b], P, int(pos[b]), k[b].astype(np.float64), v[b].astype(np.float64))
    for name in ("k", "kq", "ks", "v", "vq", "vs", "kf8", "vf8"):
        w = getattr(want, name, None)
        if w is None:
            continue
        assert np.array_equal(getattr(got, name).view(np.uint8), w.view(np.uint8)), name
    assert int(err.cpu()[0]) == 0
    # a position past the table, or in a page the sequence was not given (a -1
    # entry), stores nothing and raises the flag
    assert table[2, 1] == -1
    for pos_bad, bb in (([192, 0, 0], 1), ([192, 192, 64], 3)):
        err = _dev(np.zeros(1, np.int32))
        qd.qkdec_kv_append_paged(dkv.desc, _dev(table), 3, _dev(np.array(pos_bad, np.int32)), _dev(k), _dev(v), bb,
                                 err=err)
        sync()
        assert int(err.cpu()[0]) == -5, pos_bad
    after = dkv.logical()
    for name in ("k", "kq", "v", "vq", "kf8", "vf8"):
        if getattr(got, name, None) is not None:
            assert np.array_equal(getattr(after, name).view(np.uint8), getattr(got, name).view(np.uint8))


@pytest.mark.parametrize("P,lens,cap", [
    (256, [2400, 512, 6900, 1, 3000, 2401, 777, 4096], 7168),
    # pages of one tile and runs of up to 4096 tokens: up to 129 page entries
    # staged per run
    (32, [16384, 9000, 1, 16383, 4097, 12345, 2048, 16000], 16384),
])
def test_paged_attention_full_shape(qd, P, lens, cap):
    # B = 8 sequences of a Qwen-shaped layer, ragged contexts
    from quantized_decode_amd.tensors import upload_cache
    st = synth.Streams(8400 + P)
    hq, hkv, d = 32, 8, 128
    cont = synth.kv_cache("f16", st.next(), st.next(), len(lens), hkv, cap, d, lens)
    pool, table, _ = _pool_from(cont, lens, P, sum((n + P - 1) // P for n in lens) + 4, st.next())
    q = synth.f16_normal(st.next(), (len(lens), hq, d))
    got = _attn_paged(qd, upload_cache(pool), table, lens, q, 1 / math.sqrt(d))
    ref = OS.attention_batch_paged(q.astype(np.float64), pool, "f16", table, P, lens, 1 / math.sqrt(d))
    assert_rel(got, ref, what="paged full shape")


STEP_CASES = [
    ("toy", "f16", 2, 128, 32, 160),
    ("toy", "q8_0", 2, 128, 64, 192),
    ("toy", "fp8", 2, 128, 32, 160),
    ("full", "f16", 4, 300, 64, 320),
    ("full", "q8_0", 4, 300, 64, 320),
    ("full", "fp8", 4, 300, 64, 320),
]


@pytest.mark.parametrize("shape,kind,bsz,L,P,cap", STEP_CASES)
def test_paged_step_equals_arena_step(qd, shape, kind, bsz, L, P, cap):
    # three decode steps over pools whose pages are scattered, against the
    # slot-arena step on the same data (itself checked against the oracle in
    # test_gpu_step.py): with max_pages * P = capacity every kernel does the
    # same arithmetic, so logits, tokens, positions and every cached byte
    # must be identical
    import torch
    from quantized_decode_amd.tensors import upload_cache
    from tests.test_gpu_step import GpuStep, build
    dims = synth.TOY if shape == "toy" else synth.QWEN_SHAPED
    model, caches, tok = build(dims, 1200 + P, kind, bsz, L, cap, n_layers=None if shape == "toy" else 1)
    steps = 3
    arena = GpuStep(qd, model, caches, bsz, list(range(bsz)))
    arena.set([L] * bsz, tok)
    n_pages = bsz * (cap // P) + 6
    pools, table = [], None
    for c in caches:   # the same rng per layer: one page table for all layers
        pool, t, _ = _pool_from(c, [L] * bsz, P, n_pages, np.random.default_rng(99), room=steps)
        assert table is None or np.array_equal(t, table)
        pools.append(pool)
        table = t
    max_pages = cap // P
    table = np.pad(table, ((0, 0), (0, max_pages - table.shape[1])), constant_values=-1)
    dpools = [upload_cache(p) for p in pools]
    sm = qd.StepModel(dims, arena.embed, arena.lm_head, arena.norm, arena.layers, [d.desc for d in dpools])
    pos = _dev(np.full(bsz, L, np.int32))
    tk = _dev(np.asarray(tok, np.int32))
    logits = torch.empty((bsz, dims.vocab), dtype=torch.float32, device="cuda")
    wsp = ws(qd.qkdec_step_paged_workspace_size(sm, bsz, max_pages))
    qd.qkdec_workspace_init(wsp)
    tdev = _dev(table)
    for i in range(steps):
        la, ta, pa = arena.step()
        qd.qkdec_step_paged(sm, tdev, max_pages, pos, tk, bsz, wsp, logits=logits)
        sync()
        assert np.array_equal(logits.cpu().numpy().view(np.uint32), la.view(np.uint32)), f"step {i}: logits"
        assert np.array_equal(tk.cpu().numpy(), ta) and np.array_equal(pos.cpu().numpy(), pa), f"step {i}"
    assert qd.qkdec_step_status(wsp) == 0
    n_now = L + steps
    for li, (dp, da) in enumerate(zip(dpools, arena.kv)):
        gp, ga = dp.logical(), da.logical()
        for name, arr in vars(ga).items():
            if arr is None:
                continue
            parr = getattr(gp, name)
            for b in range(bsz):
                for j in range((n_now + P - 1) // P):
                    take = min(P, n_now - j * P)
                    assert np.array_equal(parr[table[b, j], :, :take].view(np.uint8),
                                          arr[b, :, j * P:j * P + take].view(np.uint8)), (li, name, b, j)


@pytest.mark.parametrize("kind", ["f16", "q8_0", "fp8"])
def test_paged_attention_unmapped_pages_are_masked(qd, kind):
    # table entries of -1 (a page never handed out) and past the pool inside
    # n_ctx: the tokens they would hold drop out of the softmax, exactly as in
    # the oracle; a sequence with no mapped page attends to nothing (O = 0).
    # Every page nobody holds is poisoned (NaN), so a tile that was not masked
    # would show.
    from quantized_decode_amd.tensors import upload_cache
    st = synth.Streams(8500 + len(kind))
    hq, hkv, d, P = 32, 8, 128, 64
    lens = [700, 300, 129, 513]
    cont = synth.kv_cache(kind, st.next(), st.next(), len(lens), hkv, 768, d, lens)
    pool, table, _ = _pool_from(cont, lens, P, 40, st.next())
    table = table.copy()
    table[0, 2] = -1                       # tokens 128..191 of sequence 0
    table[0, 7] = -1                       # and 448..511
    n_pool = next(a for a in vars(pool).values() if a is not None).shape[0]
    table[1, 0] = n_pool                   # past the pool: tokens 0..63 of sequence 1
    table[2, :] = -1                       # nothing mapped
    q = synth.f16_normal(st.next(), (len(lens), hq, d))
    scale = 1 / math.sqrt(d)
    got = _attn_paged(qd, upload_cache(pool), table, lens, q, scale)
    ref = OS.attention_batch_paged(q.astype(np.float64), pool, kind, table, P, lens, scale)
    assert not got[2].any()
    assert_rel(got, ref, what=f"paged {kind} with unmapped pages")


def _host_pool_write(pool, seq_cache, pages, n, P):
    """Copy the first n tokens of slot 0 of a logical cache into the pages."""
    for name, arr in vars(seq_cache).items():
        if arr is None:
            continue
        dst = getattr(pool, name)
        for j, pg in enumerate(pages):
            take = max(0, min(P, n - j * P))
            dst[pg, :, :take] = arr[0, :, j * P:j * P + take]


@pytest.mark.parametrize("kind", ["f16", "q8_0"])
def test_paged_steps_with_admission_and_release_match_oracle(qd, kind):
    # continuous batching on one pool (P1 "What I am building next"): sequences
    # A (100 cached tokens) and B (60) decode two steps; then A finishes and
    # returns its pages, C (40 cached tokens) is admitted into the running
    # batch and gets pages A held (their stale contents beyond C's length must
    # not matter), and B, C decode two more steps.  Every step is compared with
    # the oracle's paged step run on the GPU's own pool contents, positions and
    # tokens from before that step (teacher forcing): logits, argmax, the new
    # positions, and no byte of any other sequence's pages touched.
    import torch
    from quantized_decode_amd.tensors import upload_cache, upload_model
    from tests.gpu_util import LOGIT_ABS_TOL, top2_gap
    dims = synth.TOY
    P, n_pages, max_pages = 32, 14, 6
    model = synth.make_model(dims, 1300)
    st = synth.Streams(1301)
    pager = PagePool(n_pages, P)
    hist = {s: [synth.kv_cache(kind, st.next(), st.next(), 1, dims.n_kv_heads, 128, dims.head_dim, [n])
                for _ in model.layers] for s, n in (("A", 100), ("B", 60), ("C", 40))}
    length = {"A": 100, "B": 60, "C": 40}
    # host pools, every page poisoned until a sequence's history is written into it
    pools = []
    for li in range(dims.n_layers):
        p = copy.deepcopy(hist["A"][li])
        for name, arr in vars(p).items():
            if arr is None:
                continue
            poison = np.float16(np.nan) if arr.dtype == np.float16 else (127 if arr.dtype == np.int8 else 0x7F)
            setattr(p, name, np.full((n_pages,) + arr.shape[1:2] + (P,) + arr.shape[3:], poison, dtype=arr.dtype))
        pools.append(p)
    for s in ("A", "B"):
        pager.admit(s, length[s])
        for li in range(dims.n_layers):
            _host_pool_write(pools[li], hist[s][li], pager.pages(s), length[s], P)
    embed, lm_head, norm, layers = upload_model(model)
    tok = {s: int(t) for s, t in zip("ABC", synth.tokens(st.next(), 3, dims.vocab))}
    batch = ["A", "B"]
    logits = torch.empty((2, dims.vocab), dtype=torch.float32, device="cuda")
    for step in range(4):
        if step == 2:                      # A leaves, C joins between steps
            pager.release("A")
            batch = ["B", "C"]
            pager.admit("C", length["C"])
            for li in range(dims.n_layers):
                _host_pool_write(pools[li], hist["C"][li], pager.pages("C"), length["C"], P)
        for s in batch:
            pager.reserve(s, length[s] + 1)
        table = pager.table(batch, max_pages)
        dpools = [upload_cache(p) for p in pools]
        sm = qd.StepModel(dims, embed, lm_head, norm, layers, [dp.desc for dp in dpools])
        pos = _dev(np.array([length[s] for s in batch], np.int32))
        tk = _dev(np.array([tok[s] for s in batch], np.int32))
        wsp = ws(qd.qkdec_step_paged_workspace_size(sm, 2, max_pages))
        qd.qkdec_workspace_init(wsp)
        qd.qkdec_step_paged(sm, _dev(table), max_pages, pos, tk, 2, wsp, logits=logits)
        sync()
        assert qd.qkdec_step_status(wsp) == 0, f"step {step}"
        ref_pools = copy.deepcopy(pools)
        ref, rtok = OS.decode_step_paged(model, ref_pools, kind, table, P, [length[s] for s in batch],
                                         [tok[s] for s in batch])
        lg, gt = logits.cpu().numpy(), tk.cpu().numpy()
        d = float(np.abs(lg - ref).max())
        assert d <= LOGIT_ABS_TOL, f"step {step}: max |dlogit| {d:.3e}"
        for b in range(2):
            if top2_gap(ref[b]) > 1e-3:
                assert gt[b] == rtok[b], f"step {step}: argmax of {batch[b]}"
        assert np.array_equal(pos.cpu().numpy(), [length[s] + 1 for s in batch])
        # the GPU's pool after the step: only the batch's new positions changed
        new = [dp.logical() for dp in dpools]
        for li in range(dims.n_layers):
            for name, arr in vars(pools[li]).items():
                if arr is None:
                    continue
                got = getattr(new[li], name)
                changed = np.argwhere((got.view(np.uint8) != arr.view(np.uint8)).reshape(arr.shape[0], -1).any(1))
                allowed = {int(table[b, length[s] // P]) for b, s in enumerate(batch)}
                assert set(changed.ravel().tolist()) <= allowed, (step, li, name)
                setattr(pools[li], name, got)
        for b, s in enumerate(batch):
            length[s] += 1
            tok[s] = int(gt[b])
