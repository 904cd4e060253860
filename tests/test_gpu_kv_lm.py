"""KV append (bit-exact) and the LM head + argmax on the GPU against the oracle."""
import numpy as np
import pytest

import synth
from oracle import formats as OF
from oracle import ops as OO
from tests.gpu_util import LOGIT_ABS_TOL, sync, top2_gap, ws

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qd():
    import quantized_decode_amd as m
    m.load_library()
    return m


def _dev(a):
    from quantized_decode_amd.tensors import dev
    return dev(a)


@pytest.mark.parametrize("d,nkv", [(64, 2), (128, 8)])
def test_append_f16_bit_exact(qd, d, nkv):
    from quantized_decode_amd.tensors import upload_kv_f16
    rng = np.random.default_rng(d)
    slots_n, cap, bsz = 5, 96, 4
    k0 = rng.standard_normal((slots_n, nkv, cap, d)).astype(np.float16)
    v0 = rng.standard_normal((slots_n, nkv, cap, d)).astype(np.float16)
    dkv = upload_kv_f16(k0, v0)
    slot = np.array([3, 0, 4, 1], np.int32)
    pos = np.array([0, 95, 37, 64], np.int32)
    k = (rng.standard_normal((bsz, nkv, d)) * 10.0 ** rng.integers(-6, 5, (bsz, nkv, 1))).astype(np.float32)
    v = (rng.standard_normal((bsz, nkv, d)) * 1e3).astype(np.float32)
    k[0, 0, :4] = [65504.0, 65520.0, 1e-8, -2.0 ** -25]
    err = _dev(np.zeros(1, np.int32))
    qd.qkdec_kv_append_f16(dkv.desc, _dev(slot), _dev(pos), _dev(k), _dev(v), bsz, err=err)
    sync()
    kk, vv = dkv.logical_f16()
    want_k, want_v = k0.copy(), v0.copy()
    with np.errstate(over="ignore"):     # 65520 rounds to +inf, as on the GPU
        for b in range(bsz):
            want_k[slot[b], :, pos[b]] = k[b].astype(np.float64).astype(np.float16)
            want_v[slot[b], :, pos[b]] = v[b].astype(np.float64).astype(np.float16)
    assert np.array_equal(kk.view(np.uint16), want_k.view(np.uint16))
    assert np.array_equal(vv.view(np.uint16), want_v.view(np.uint16))
    assert int(err.cpu()[0]) == 0


@pytest.mark.parametrize("d,nkv", [(64, 2), (128, 8)])
def test_append_q8_0_bit_exact(qd, d, nkv):
    from quantized_decode_amd.tensors import upload_kv_q8
    rng = np.random.default_rng(100 + d)
    slots_n, cap, bsz = 3, 64, 3
    shape = (slots_n, nkv, cap, d)
    sshape = (slots_n, nkv, cap, d // 32)
    kq0 = rng.integers(-127, 128, shape, dtype=np.int8)
    vq0 = rng.integers(-127, 128, shape, dtype=np.int8)
    ks0 = (np.abs(rng.standard_normal(sshape)) * 0.02).astype(np.float16)
    vs0 = (np.abs(rng.standard_normal(sshape)) * 0.02).astype(np.float16)
    dkv = upload_kv_q8(kq0, ks0, vq0, vs0)
    slot = np.array([2, 0, 1], np.int32)
    pos = np.array([63, 0, 17], np.int32)
    k = (rng.standard_normal((bsz, nkv, d)) * 10.0 ** rng.integers(-9, 4, (bsz, nkv, 1))).astype(np.float32)
    v = (rng.standard_normal((bsz, nkv, d)) * 20).astype(np.float32)
    k[0, 0, :32] = 0.0                                  # all-zero block
    k[1, 0, :32] = np.arange(-16, 16) + 0.5             # amax 16.5 (no exact ties after scaling)
    k[1, 0, 0] = 127.0                                  # scale exactly 1.0: integer + 0.5 ties
    k[1, 0, 1:6] = [2.5, -2.5, 0.5, -0.5, 126.5]
    k[2, 0, :32] = 1e-7 * rng.standard_normal(32)       # subnormal fp16 scale
    v[0, 0, :32] = 127 * 1.4 * 2.0 ** -24              # scale rounds down: clamp at 127
    err = _dev(np.zeros(1, np.int32))
    qd.qkdec_kv_append_q8_0(dkv.desc, _dev(slot), _dev(pos), _dev(k), _dev(v), bsz, err=err)
    sync()
    kq, ks, vq, vs = dkv.logical_q8()
    wk, wks, wv, wvs = kq0.copy(), ks0.copy(), vq0.copy(), vs0.copy()
    for b in range(bsz):
        wk[slot[b], :, pos[b]], wks[slot[b], :, pos[b]] = OF.q8_0_quantize(k[b].astype(np.float64))
        wv[slot[b], :, pos[b]], wvs[slot[b], :, pos[b]] = OF.q8_0_quantize(v[b].astype(np.float64))
    assert np.array_equal(kq, wk) and np.array_equal(vq, wv)
    assert np.array_equal(ks.view(np.uint16), wks.view(np.uint16))
    assert np.array_equal(vs.view(np.uint16), wvs.view(np.uint16))
    assert int(err.cpu()[0]) == 0


@pytest.mark.parametrize("kind", ["q8k_f16v", "f16k_q8v", "fp8"])
def test_append_mixed_formats_bit_exact(qd, kind):
    # keys and values in different formats (or E4M3) through the generic entry
    # point, each stored exactly as the oracle stores that format
    import copy

    from oracle import step as OS
    from quantized_decode_amd.tensors import upload_cache
    st = synth.Streams(300 + len(kind))
    slots_n, nkv, cap, d, bsz = 3, 8, 64, 128, 3
    cache = synth.kv_cache(kind, st.next(), st.next(), slots_n, nkv, cap, d, [40, 64, 10])
    dkv = upload_cache(cache)
    rng = st.next()
    slot = np.array([2, 0, 1], np.int32)
    pos = np.array([63, 0, 17], np.int32)
    k = (rng.standard_normal((bsz, nkv, d)) * 10.0 ** rng.integers(-6, 3, (bsz, nkv, 1))).astype(np.float32)
    v = (rng.standard_normal((bsz, nkv, d)) * 20).astype(np.float32)
    if kind == "fp8":   # ties (to even), subnormal ties, saturation, signed zeros
        k[0, 0, :10] = [1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 15 * 2.0 ** -10, 1.9375, 464.0, -1e9, 0.0, -0.0]
        v[1, 2, :4] = [448.0, -449.0, 2.0 ** -9, -(2.0 ** -12)]
    err = _dev(np.zeros(1, np.int32))
    qd.qkdec_kv_append(dkv.desc, _dev(slot), _dev(pos), _dev(k), _dev(v), bsz, err=err)
    sync()
    got = dkv.logical()
    want = copy.deepcopy(cache)
    for b in range(bsz):
        OS.kv_append(want, kind, int(slot[b]), int(pos[b]), k[b].astype(np.float64), v[b].astype(np.float64))
    for name in ("k", "kq", "ks", "v", "vq", "vs", "kf8", "vf8"):
        w = getattr(want, name, None)
        if w is None:
            continue
        g = getattr(got, name)
        assert g.dtype == w.dtype and np.array_equal(g.view(np.uint8), w.view(np.uint8)), f"{kind}: {name}"
    assert int(err.cpu()[0]) == 0


def test_append_out_of_range_sets_flag_and_writes_nothing(qd):
    from quantized_decode_amd.tensors import upload_kv_f16
    k0 = np.zeros((2, 2, 32, 64), np.float16)
    dkv = upload_kv_f16(k0, k0)
    err = _dev(np.zeros(1, np.int32))
    kv = np.ones((2, 2, 64), np.float32)
    qd.qkdec_kv_append_f16(dkv.desc, _dev(np.array([0, 1], np.int32)), _dev(np.array([32, 5], np.int32)),
                           _dev(kv), _dev(kv), 2, err=err)
    sync()
    kk, vv = dkv.logical_f16()
    assert int(err.cpu()[0]) == -5
    assert not kk[0].any() and not vv[0].any()
    assert (kk[1, :, 5] == 1).all() and kk[1].sum() == 2 * 64


def _lm(qd, w, x, with_logits=True):
    import torch
    vocab, hidden = w.shape
    bsz = x.shape[0]
    wt = _dev(w.view(np.uint16)).view(torch.float16)
    xt = _dev(x.view(np.uint16)).view(torch.float16)
    tok = torch.empty(bsz, dtype=torch.int32, device="cuda")
    logits = torch.empty((bsz, vocab), dtype=torch.float32, device="cuda") if with_logits else None
    wsp = ws(qd.qkdec_lm_head_workspace_size(vocab, bsz))
    qd.qkdec_lm_head_argmax(wt, vocab, hidden, xt, bsz, tok, logits=logits, workspace=wsp)
    sync()
    return tok.cpu().numpy(), (logits.cpu().numpy() if with_logits else None)


@pytest.mark.parametrize("vocab,hidden,bsz", [(4096, 512, 1), (4096, 512, 2), (4096, 512, 16), (160, 256, 3)])
def test_lm_head_small(qd, vocab, hidden, bsz):
    st = synth.Streams(vocab + hidden + bsz)
    w = synth.f16_normal(st.next(), (vocab, hidden), scale=1 / np.sqrt(hidden))
    x = synth.f16_normal(st.next(), (bsz, hidden))
    tok, lg = _lm(qd, w, x)
    ref = OO.dense_gemm(w, x)
    assert np.abs(lg - ref).max() <= LOGIT_ABS_TOL
    for b in range(bsz):
        if top2_gap(ref[b]) > 1e-3:
            assert tok[b] == int(np.argmax(ref[b]))
        assert tok[b] == int(np.argmax(lg[b]))   # the kernel's own argmax of its logits
    tok2, _ = _lm(qd, w, x, with_logits=False)
    assert np.array_equal(tok, tok2)


def test_lm_head_ties_take_lowest_index(qd):
    vocab, hidden = 4096, 512
    st = synth.Streams(5)
    w = synth.f16_normal(st.next(), (vocab, hidden), scale=1 / np.sqrt(hidden))
    x = synth.f16_normal(st.next(), (2, hidden))
    star = (x[0].astype(np.float64) * 0.05).astype(np.float16)
    for row in (3001, 7, 2500):          # identical rows in different tiles and work-groups
        w[row] = star
    tok, lg = _lm(qd, w, x)
    assert lg[0, 7] == lg[0, 3001] == lg[0, 2500] == lg[0].max()
    assert tok[0] == 7


def test_lm_head_full_vocab(qd):
    vocab, hidden, bsz = 151936, 4096, 8
    st = synth.Streams(1003)
    w = synth.f16_normal(st.next(), (vocab, hidden), scale=1 / np.sqrt(hidden))
    x = synth.f16_normal(st.next(), (bsz, hidden))
    tok, lg = _lm(qd, w, x)
    ref = OO.dense_gemm(w, x)
    assert np.abs(lg - ref).max() <= LOGIT_ABS_TOL
    for b in range(bsz):
        if top2_gap(ref[b]) > 1e-3:
            assert tok[b] == int(np.argmax(ref[b]))
