"""Prefill (qkdec_prefill) on the GPU: the prompt's keys and values appended
to the cache and the first generated token, against the oracle's prefill
(the decode step over the prompt's tokens in order)."""
import copy

import numpy as np
import pytest

import synth
from oracle import step as OS
from tests.gpu_util import LOGIT_ABS_TOL, sync, top2_gap, ws

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qd():
    import quantized_decode_amd as m
    m.load_library()
    return m


def _prefill(qd, model, caches, slot, start, prompt):
    import torch
    from quantized_decode_amd.tensors import dev, upload_cache, upload_model
    embed, lm_head, norm, layers = upload_model(model)
    kv = [upload_cache(c) for c in caches]
    sm = qd.StepModel(model.dims, embed, lm_head, norm, layers, [k.desc for k in kv])
    w = ws(qd.qkdec_prefill_workspace_size(sm))
    qd.qkdec_workspace_init(w)
    logits = torch.empty(model.dims.vocab, dtype=torch.float32, device="cuda")
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    qd.qkdec_prefill(sm, slot, start, dev(np.asarray(prompt, np.int32)), len(prompt), tok, w, logits=logits)
    sync()
    return logits.cpu().numpy(), int(tok.item()), kv, (sm, w, embed, lm_head, norm, layers)


def _toy_case(qd, dims, kind, n, seed):
    model = synth.make_model(dims, seed)
    st = synth.Streams(seed + 1)
    cap = (20 + n + 31) // 32 * 32 + 32
    caches = [synth.kv_cache(kind, st.next(), st.next(), 3, dims.n_kv_heads, cap, dims.head_dim, [30, 20, 50])
              for _ in model.layers]
    prompt = synth.tokens(st.next(), n, dims.vocab)
    lg, tok, kv, _ = _prefill(qd, model, caches, 1, 20, prompt)
    ref_caches = copy.deepcopy(caches)
    ref, rtok = OS.prefill(model, ref_caches, kind, 1, 20, prompt)
    d = float(np.abs(lg - ref).max())
    assert d <= LOGIT_ABS_TOL, f"max |dlogit| {d:.3e}"
    if top2_gap(ref) > 1e-3:
        assert tok == rtok
    # the other slots, the history of slot 1 and everything past the prompt untouched
    for li in range(dims.n_layers):
        got, was = kv[li].logical(), caches[li]
        for name, arr in vars(was).items():
            if arr is None:
                continue
            g = getattr(got, name)
            assert np.array_equal(g[[0, 2]].view(np.uint8), arr[[0, 2]].view(np.uint8)), (li, name)
            assert np.array_equal(g[1, :, :20].view(np.uint8), arr[1, :, :20].view(np.uint8)), (li, name)
            assert not g[1, :, 20 + n:].view(np.uint8).any(), (li, name)


@pytest.mark.parametrize("kind", ["f16", "q8_0"])
@pytest.mark.parametrize("n", [1, 16, 40, 64, 100, 300])
def test_prefill_toy_matches_oracle(qd, kind, n):
    # the toy decoder, a prompt of n tokens appended after 20 cached tokens of
    # slot 1 of 3: one token, part of a 64-row tile, one tile, 64 + 36 rows,
    # and 300 rows (attention calls of 256 + 44 rows)
    _toy_case(qd, synth.TOY, kind, n, 1700)


@pytest.mark.parametrize("kind", ["fp8", "q8k_f16v", "f16k_q8v"])
def test_prefill_toy_other_caches(qd, kind):
    # the remaining cache formats, 64 + 6 prompt tokens
    _toy_case(qd, synth.TOY, kind, 70, 1720)


@pytest.mark.parametrize("heads,kind", [((4, 2), "f16"), ((8, 1), "q8_0"), ((8, 1), "f16"), ((16, 1), "f16"),
                                        ((12, 4), "f16"), ((12, 4), "q8_0")])
def test_prefill_group_sizes(qd, heads, kind):
    # query heads per KV head G = 2, 8, 16 and 3: the flash kernel takes
    # min(G, 4) heads of 64 / min(G, 4) rows per work-group for G a power of
    # two; G = 3 runs the split-K kernel, one row per work item
    hq, hkv = heads
    dims = synth.ModelDims(n_layers=2, hidden=512, n_q_heads=hq, n_kv_heads=hkv, head_dim=64, ffn=1536,
                           vocab=4096)
    _toy_case(qd, dims, kind, 70, 1740)


def _vs_decode_steps(qd, dims, kind, n_cached, n_prompt, seed):
    # the prefill's first generated token and logits against n_prompt
    # single-token decode steps on the GPU, and the appended keys and values of
    # the two paths agree
    import torch
    from quantized_decode_amd.tensors import dev, upload_cache
    model = synth.make_model(dims, seed)
    st = synth.Streams(seed + 1)
    cap = (n_cached + n_prompt + 31) // 32 * 32 + 32
    caches = [synth.kv_cache(kind, st.next(), st.next(), 1, dims.n_kv_heads, cap, dims.head_dim, [n_cached])
              for _ in model.layers]
    prompt = synth.tokens(st.next(), n_prompt, dims.vocab)
    lg, tok, kv, (sm, w, embed, lm_head, norm, layers) = _prefill(qd, model, caches, 0, n_cached, prompt)
    kv2 = [upload_cache(c) for c in caches]
    sm2 = qd.StepModel(dims, embed, lm_head, norm, layers, [k.desc for k in kv2])
    w2 = ws(qd.qkdec_step_workspace_size(sm2, 1))
    qd.qkdec_workspace_init(w2)
    slot = dev(np.zeros(1, np.int32))
    logits = torch.empty((1, dims.vocab), dtype=torch.float32, device="cuda")
    for i, t in enumerate(prompt):
        pos = dev(np.array([n_cached + i], np.int32))
        tk = dev(np.array([t], np.int32))
        qd.qkdec_step(sm2, slot, pos, tk, 1, w2, logits=logits)
    sync()
    ref = logits.cpu().numpy()[0]
    d = float(np.abs(lg - ref).max())
    assert d <= LOGIT_ABS_TOL, f"prefill vs decode steps: max |dlogit| {d:.3e}"
    if top2_gap(ref) > 1e-3:
        assert tok == int(np.argmax(ref))
    if kind != "f16":
        return   # the appended codes are checked through the logits
    end = n_cached + n_prompt
    for a, b in zip(kv, kv2):
        ka, va = a.logical_f16()
        kb, vb = b.logical_f16()
        for x, y in ((ka, kb), (va, vb)):
            x64, y64 = x[0, :, n_cached:end].astype(np.float64), y[0, :, n_cached:end].astype(np.float64)
            assert np.abs(x64 - y64).max() <= 1e-3 * np.abs(y64).max()


@pytest.mark.parametrize("kind", ["f16", "q8_0"])
def test_prefill_full_width_equals_decode_steps(qd, kind):
    # a two-layer decoder of the full width (every projection on the kernels
    # the bench times), 270 prompt tokens after 300 cached ones
    dims = synth.ModelDims(n_layers=2, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=12288,
                           vocab=16384)
    _vs_decode_steps(qd, dims, kind, 300, 270, 1710)


@pytest.mark.parametrize("kind", ["f16", "q8_0"])
def test_prefill_two_passes_equals_decode_steps(qd, kind):
    # the toy decoder, 2100 prompt tokens after 40 cached ones: a pass of 2048
    # rows of the layers, then one of 52 (the oracle's prefill of this many
    # tokens takes minutes; the decode step it is checked against is itself
    # checked against the oracle)
    _vs_decode_steps(qd, synth.TOY, kind, 40, 2100, 1770)


@pytest.mark.parametrize("kind,P,cap,n", [("f16", 32, 192, 100), ("q8_0", 64, 192, 100), ("fp8", 32, 192, 100),
                                          ("f16", 256, 2304, 2100), ("q8_0", 128, 2304, 2100)])
def test_prefill_paged_equals_arena(qd, kind, P, cap, n):
    # the toy decoder, n prompt tokens after 20 cached ones, into slot 1 of a
    # slot arena and into the same sequence's pages scattered over a pool
    # (max_pages * P = the arena's capacity): the same kernels on the same
    # values, so the logits, the token and every byte of the sequence's
    # cache must be identical.  n = 2100 takes two passes of the layers (2048
    # rows, then 52), the second one's rows on pages the first one filled
    import torch
    from quantized_decode_amd.tensors import dev, upload_cache
    from tests.test_gpu_paged import _pool_from
    dims = synth.TOY
    model = synth.make_model(dims, 1780)
    st = synth.Streams(1781)
    lens, b = [30, 20, 50], 1
    caches = [synth.kv_cache(kind, st.next(), st.next(), 3, dims.n_kv_heads, cap, dims.head_dim, lens)
              for _ in model.layers]
    prompt = synth.tokens(st.next(), n, dims.vocab)
    lg, tok, kv, (sm, w, embed, lm_head, norm, layers) = _prefill(qd, model, caches, b, lens[b], prompt)
    n_pages = sum((x + n + P - 1) // P for x in lens) + 6
    pools, table = [], None
    for c in caches:   # the same rng per layer: one page table for all layers
        pool, t, _ = _pool_from(c, lens, P, n_pages, np.random.default_rng(7), room=n)
        assert table is None or np.array_equal(t, table)
        pools.append(pool)
        table = t
    max_pages = cap // P
    table = np.pad(table, ((0, 0), (0, max_pages - table.shape[1])), constant_values=-1)
    dpools = [upload_cache(p) for p in pools]
    smp = qd.StepModel(dims, embed, lm_head, norm, layers, [d.desc for d in dpools])
    wp = ws(qd.qkdec_prefill_paged_workspace_size(smp))
    qd.qkdec_workspace_init(wp)
    logits = torch.empty(dims.vocab, dtype=torch.float32, device="cuda")
    tk = torch.zeros(1, dtype=torch.int32, device="cuda")
    qd.qkdec_prefill_paged(smp, dev(np.ascontiguousarray(table[b])), max_pages, lens[b],
                           dev(np.asarray(prompt, np.int32)), n, tk, wp, logits=logits)
    sync()
    assert qd.qkdec_step_status(wp) == 0
    assert np.array_equal(logits.cpu().numpy().view(np.uint32), lg.view(np.uint32))
    assert int(tk.item()) == tok
    end = lens[b] + n
    for li, (dp, da) in enumerate(zip(dpools, kv)):
        gp, ga = dp.logical(), da.logical()
        for name, arr in vars(ga).items():
            if arr is None:
                continue
            parr = getattr(gp, name)
            for j in range((end + P - 1) // P):
                take = min(P, end - j * P)
                assert np.array_equal(parr[table[b, j], :, :take].view(np.uint8),
                                      arr[b, :, j * P:j * P + take].view(np.uint8)), (li, name, j)


def test_prefill_paged_unmapped_page_flags_capacity(qd):
    # a page table entry of -1 inside the prompt: its tokens are not stored,
    # the error word says QKDEC_E_CAPACITY, and no other page changes
    import torch
    from quantized_decode_amd.tensors import dev, upload_cache, upload_model
    from tests.test_gpu_paged import _pool_from
    dims = synth.TOY
    model = synth.make_model(dims, 1790)
    st = synth.Streams(1791)
    P, cap, lens, n = 32, 128, [40], 60
    caches = [synth.kv_cache("f16", st.next(), st.next(), 1, dims.n_kv_heads, cap, dims.head_dim, lens)
              for _ in model.layers]
    pools, table = [], None
    for c in caches:
        pool, t, _ = _pool_from(c, lens, P, 8, np.random.default_rng(11), room=n)
        pools.append(pool)
        table = t
    table = np.pad(table, ((0, 0), (0, cap // P - table.shape[1])), constant_values=-1)
    row = table[0].copy()
    lost = row[2]
    row[2] = -1   # positions 64..95 of the prompt's range have no page
    dpools = [upload_cache(p) for p in pools]
    embed, lm_head, norm, layers = upload_model(model)
    smp = qd.StepModel(dims, embed, lm_head, norm, layers, [d.desc for d in dpools])
    wp = ws(qd.qkdec_prefill_paged_workspace_size(smp))
    qd.qkdec_workspace_init(wp)
    tk = torch.zeros(1, dtype=torch.int32, device="cuda")
    qd.qkdec_prefill_paged(smp, dev(row), cap // P, lens[0], dev(np.asarray(synth.tokens(st.next(), n, dims.vocab),
                                                                              np.int32)), n, tk, wp)
    sync()
    assert qd.qkdec_step_status(wp) == -5   # QKDEC_E_CAPACITY
    for dp, was in zip(dpools, pools):
        got = dp.logical()
        for name, arr in vars(was).items():
            if arr is None:
                continue
            assert np.array_equal(getattr(got, name)[lost].view(np.uint8), arr[lost].view(np.uint8)), name
