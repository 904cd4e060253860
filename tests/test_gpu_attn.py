"""Split-K flash-decode attention (fp16, Q8_0, mixed and E4M3 caches) on the GPU against the oracle."""
import math

import numpy as np
import pytest

import synth
from oracle import step as OS
from tests.gpu_util import assert_rel, sync, ws

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qd():
    import quantized_decode_amd as m
    m.load_library()
    return m


def _make(kind, seed, n_slots, n_kv, cap, d, filled):
    st = synth.Streams(seed)
    c = synth.kv_cache(kind, st.next(), st.next(), n_slots, n_kv, cap, d, filled)
    return c, st


def _run(qd, cache, kind, q, slots, n_ctx, scale, poison=False):
    import torch
    from quantized_decode_amd.tensors import dev, upload_cache
    dkv = upload_cache(cache)
    if poison:   # positions past n_ctx hold NaN / garbage: they must never reach the output
        kfmt, vfmt = synth.KV_FORMATS[kind]
        for s in range(dkv.desc.n_slots):
            used = max(int(n) for b, n in enumerate(n_ctx) if slots[b] == s) if s in list(slots) else 0
            if kfmt == "fp8":   # the E4M3 NaN codes
                dkv.k[s, :, used:] = 0x7F
                dkv.set_v_from(s, used, 0xFF)
                continue
            if kfmt == "f16":
                dkv.k[s, :, used:] = float("nan")
            else:
                dkv.k[s, :, used:] = 127
                dkv.k_scale[s, :, used:] = float("nan")
            if vfmt == "f16":
                dkv.set_v_from(s, used, float("nan"))
            else:
                dkv.set_v_from(s, used, -127)
                dkv.v_scale[s, :, used:] = float("inf")
    b, hq, d = q.shape
    qd_t = dev(q.view(np.uint16)).view(torch.float16)
    o = torch.empty((b, hq, d), dtype=torch.float32, device="cuda")
    o16 = torch.empty((b, hq, d), dtype=torch.float16, device="cuda")
    w = ws(qd.qkdec_attn_workspace_size(b, hq, dkv.desc))
    qd.qkdec_attn_decode(dkv.desc, dev(np.asarray(slots, np.int32)), dev(np.asarray(n_ctx, np.int32)), b, qd_t, hq,
                         scale, o=o, o16=o16, workspace=w)
    sync()
    return o.cpu().numpy(), o16.cpu().numpy()


CASES = [
    # (kind, hq, hkv, d, cap, n_ctx per sequence)
    ("f16", 8, 2, 64, 256, [1, 31]),
    ("f16", 8, 2, 64, 256, [32, 33]),
    ("f16", 8, 2, 64, 256, [127, 128]),
    ("f16", 8, 2, 64, 256, [129, 256]),
    ("f16", 32, 8, 128, 512, [1, 100, 128, 129, 300, 512]),
    ("f16", 16, 1, 128, 384, [383, 257, 5]),
    ("f16", 16, 16, 64, 160, [160, 65]),
    ("f16", 32, 4, 128, 288, [200, 288]),
    ("q8_0", 8, 2, 64, 256, [1, 31]),
    ("q8_0", 8, 2, 64, 256, [129, 256]),
    ("q8_0", 32, 8, 128, 512, [1, 100, 128, 129, 300, 512]),
    ("q8_0", 16, 1, 128, 384, [383, 257, 5]),
    ("q8_0", 32, 4, 128, 288, [200, 288]),
    # keys and values in different formats
    ("q8k_f16v", 8, 2, 64, 256, [1, 31]),
    ("q8k_f16v", 32, 8, 128, 512, [1, 100, 128, 129, 300, 512]),
    ("q8k_f16v", 16, 1, 128, 384, [383, 257, 5]),
    ("f16k_q8v", 8, 2, 64, 256, [129, 256]),
    ("f16k_q8v", 32, 8, 128, 512, [1, 100, 128, 129, 300, 512]),
    ("f16k_q8v", 32, 4, 128, 288, [200, 288]),
    ("fp8", 8, 2, 64, 256, [1, 31]),
    ("fp8", 8, 2, 64, 256, [32, 33]),
    ("fp8", 8, 2, 64, 256, [129, 256]),
    ("fp8", 32, 8, 128, 512, [1, 100, 128, 129, 300, 512]),
    ("fp8", 16, 1, 128, 384, [383, 257, 5]),
    ("fp8", 16, 16, 64, 160, [160, 65]),
    ("fp8", 32, 4, 128, 288, [200, 288]),
]


@pytest.mark.parametrize("kind,hq,hkv,d,cap,n_ctx", CASES)
def test_attention_small(qd, kind, hq, hkv, d, cap, n_ctx):
    bsz = len(n_ctx)
    n_slots = bsz + 1
    slots = list(np.random.default_rng(cap + bsz).permutation(n_slots)[:bsz])
    filled = [0] * n_slots
    for s, n in zip(slots, n_ctx):
        filled[s] = n
    cache, st = _make(kind, 50 + cap + d + hq, n_slots, hkv, cap, d, filled)
    q = synth.f16_normal(st.next(), (bsz, hq, d))
    scale = 1.0 / math.sqrt(d)
    o, o16 = _run(qd, cache, kind, q, slots, n_ctx, scale, poison=True)
    ref = OS.attention_batch(q.astype(np.float64), cache, kind, slots, n_ctx, scale)
    assert_rel(o, ref, what=f"{kind} hq={hq} hkv={hkv} d={d} n={n_ctx}")
    assert np.array_equal(o16, o.astype(np.float16))


@pytest.mark.parametrize("kind", ["f16", "q8_0", "q8k_f16v", "f16k_q8v", "fp8"])
def test_attention_full_config(qd, kind):
    # 32 query heads on 8 KV heads of 128, B = 8 sequences of 2400 tokens, one layer
    bsz, hq, hkv, d, L = 8, 32, 8, 128, 2400
    cap = 2432
    cache, st = _make(kind, 2024, bsz, hkv, cap, d, [L] * bsz)
    q = synth.f16_normal(st.next(), (bsz, hq, d))
    slots = list(range(bsz))
    o, _ = _run(qd, cache, kind, q, slots, [L] * bsz, 1 / math.sqrt(d))
    ref = OS.attention_batch(q.astype(np.float64), cache, kind, slots, [L] * bsz, 1 / math.sqrt(d))
    assert_rel(o, ref, what=f"{kind} full")


def test_attention_ragged_lengths(qd):
    bsz, hq, hkv, d = 8, 32, 8, 128
    lens = synth.ragged_lengths(np.random.default_rng(4242), bsz)
    cap = 8192
    cache, st = _make("f16", 4243, bsz, hkv, cap, d, list(lens))
    q = synth.f16_normal(st.next(), (bsz, hq, d))
    o, _ = _run(qd, cache, "f16", q, list(range(bsz)), list(lens), 1 / math.sqrt(d))
    ref = OS.attention_batch(q.astype(np.float64), cache, "f16", list(range(bsz)), list(lens), 1 / math.sqrt(d))
    assert_rel(o, ref, what=f"ragged {list(lens)}")


def test_attention_empty_sequence_gives_zero(qd):
    cache, st = _make("f16", 77, 2, 2, 64, 64, [10, 64])
    q = synth.f16_normal(st.next(), (2, 8, 64))
    o, _ = _run(qd, cache, "f16", q, [0, 1], [0, 64], 0.125)
    assert not o[0].any()
    ref = OS.attention_batch(q[1:].astype(np.float64), cache, "f16", [1], [64], 0.125)
    assert_rel(o[1:], ref)


def test_attention_deterministic(qd):
    cache, st = _make("q8_0", 78, 4, 8, 1024, 128, [1000, 17, 1024, 640])
    q = synth.f16_normal(st.next(), (4, 32, 128))
    o1, _ = _run(qd, cache, "q8_0", q, [0, 1, 2, 3], [1000, 17, 1024, 640], 0.088)
    o2, _ = _run(qd, cache, "q8_0", q, [0, 1, 2, 3], [1000, 17, 1024, 640], 0.088)
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))


def test_attention_workspace_reused_across_calls(qd):
    # the runs' partial results live in the workspace and the run count follows
    # each sequence's length: consecutive calls with different lengths (one
    # sequence empty, one negative) must each be exact
    import torch
    from quantized_decode_amd.tensors import dev, upload_cache
    bsz, hq, hkv, d, cap = 4, 32, 8, 128, 1024
    cache, st = _make("f16", 79, bsz, hkv, cap, d, [cap] * bsz)
    dkv = upload_cache(cache)
    q = synth.f16_normal(st.next(), (bsz, hq, d))
    qd_t = dev(q.view(np.uint16)).view(torch.float16)
    w = ws(qd.qkdec_attn_workspace_size(bsz, hq, dkv.desc))
    slots = dev(np.arange(bsz, dtype=np.int32))
    for lens in ([1024, 17, 600, 129], [0, 1024, 128, 1], [300, -5, 1000, 513], [1024, 17, 600, 129]):
        o = torch.empty((bsz, hq, d), dtype=torch.float32, device="cuda")
        qd.qkdec_attn_decode(dkv.desc, slots, dev(np.asarray(lens, np.int32)), bsz, qd_t, hq, 1 / math.sqrt(d),
                             o=o, workspace=w)
        sync()
        got = o.cpu().numpy()
        live = [b for b in range(bsz) if lens[b] > 0]
        for b in range(bsz):
            if lens[b] <= 0:
                assert not got[b].any(), f"{lens}: sequence {b} not zero"
        ref = OS.attention_batch(q[live].astype(np.float64), cache, "f16", live, [lens[b] for b in live],
                                 1 / math.sqrt(d))
        assert_rel(got[live], ref, what=f"lengths {lens}")


def test_attention_fp8_value_decode_exact(qd):
    # one cached token: the softmax weight is exactly 1, so O is the decoded
    # value row itself; the rows hold every finite E4M3 code (the two NaN codes
    # replaced by +-448), so the hardware conversion is checked code by code
    from oracle import formats as OF
    hq, hkv, d, cap = 4, 2, 128, 64
    cache = synth.kv_cache_fp8(np.random.default_rng(5), np.random.default_rng(6), 1, hkv, cap, d, [1])
    codes = np.arange(256, dtype=np.uint8)
    codes[0x7F], codes[0xFF] = 0x7E, 0xFE
    cache.vf8[0, :, 0, :] = codes.reshape(hkv, d)
    q = synth.f16_normal(np.random.default_rng(7), (1, hq, d))
    o, o16 = _run(qd, cache, "fp8", q, [0], [1], 1 / math.sqrt(d), poison=True)
    want = OF.fp8_e4m3_decode(codes).reshape(hkv, d)
    for h in range(hq):
        g = h // (hq // hkv)
        assert np.array_equal(o[0, h].astype(np.float64), want[g]), h
        assert np.array_equal(o16[0, h].astype(np.float64), want[g]), h


def _nan_ws(nbytes):
    """Workspace pre-filled with NaN: a run state the merge should not read
    (rows past a sequence's run count, stale rows of an earlier call) would
    turn the output into NaN."""
    import torch
    n = (max(int(nbytes), 256) + 3) // 4
    return torch.full((n,), float("nan"), dtype=torch.float32, device="cuda").view(torch.uint8)


@pytest.mark.parametrize("kind", ["f16", "q8_0"])
@pytest.mark.parametrize("bsz", [1, 2])
@pytest.mark.parametrize("L", [2400, 6900])
def test_attention_small_batch_many_runs_nan_workspace(qd, kind, bsz, L):
    # B = 1 and 2 sequences of a Qwen-shaped layer (32/8 heads of 128): the
    # runs per sequence (15 at L = 2400, 16-32 at L = 6900) fill the merge's
    # batches of eight partly, and every row the merge must not use is NaN
    import torch
    from quantized_decode_amd.tensors import dev, upload_cache
    hq, hkv, d = 32, 8, 128
    cap = (L + 31) // 32 * 32
    cache, st = _make(kind, 6000 + L + bsz, bsz, hkv, cap, d, [L] * bsz)
    q = synth.f16_normal(st.next(), (bsz, hq, d))
    dkv = upload_cache(cache)
    qt = dev(q.view(np.uint16)).view(torch.float16)
    o = torch.empty((bsz, hq, d), dtype=torch.float32, device="cuda")
    w = _nan_ws(qd.qkdec_attn_workspace_size(bsz, hq, dkv.desc))
    slots = list(range(bsz))
    qd.qkdec_attn_decode(dkv.desc, dev(np.asarray(slots, np.int32)), dev(np.full(bsz, L, np.int32)), bsz, qt, hq,
                         1 / math.sqrt(d), o=o, workspace=w)
    sync()
    ref = OS.attention_batch(q.astype(np.float64), cache, kind, slots, [L] * bsz, 1 / math.sqrt(d))
    assert_rel(o.cpu().numpy(), ref, what=f"{kind} B={bsz} L={L}")


@pytest.mark.parametrize("kind", ["f16", "q8_0"])
@pytest.mark.parametrize("L", [8192, 19000])
def test_attention_long_context(qd, kind, L):
    # the long-context points of the Q8_0 workload (B = 8 at L = 8192 and
    # 19000: eight runs per sequence, two rounds of the chip), one
    # Qwen-shaped layer, against the oracle; NaN workspace
    import torch
    from quantized_decode_amd.tensors import dev, upload_cache
    bsz, hq, hkv, d = 8, 32, 8, 128
    cap = (L + 31) // 32 * 32
    cache, st = _make(kind, 7000 + L, bsz, hkv, cap, d, [L] * bsz)
    q = synth.f16_normal(st.next(), (bsz, hq, d))
    dkv = upload_cache(cache)
    qt = dev(q.view(np.uint16)).view(torch.float16)
    o = torch.empty((bsz, hq, d), dtype=torch.float32, device="cuda")
    w = _nan_ws(qd.qkdec_attn_workspace_size(bsz, hq, dkv.desc))
    slots = list(range(bsz))
    qd.qkdec_attn_decode(dkv.desc, dev(np.asarray(slots, np.int32)), dev(np.full(bsz, L, np.int32)), bsz, qt, hq,
                         1 / math.sqrt(d), o=o, workspace=w)
    sync()
    del dkv
    ref = OS.attention_batch(q.astype(np.float64), cache, kind, slots, [L] * bsz, 1 / math.sqrt(d))
    assert_rel(o.cpu().numpy(), ref, what=f"{kind} B=8 L={L}")


@pytest.mark.parametrize("kind", ["q8_0", "fp8"])
def test_attention_ragged_lengths_quantized(qd, kind):
    # the ragged batch (lengths uniform in 512..8192) over the 8-bit caches
    bsz, hq, hkv, d = 8, 32, 8, 128
    lens = synth.ragged_lengths(np.random.default_rng(4244), bsz)
    cache, st = _make(kind, 4245, bsz, hkv, 8192, d, list(lens))
    q = synth.f16_normal(st.next(), (bsz, hq, d))
    o, _ = _run(qd, cache, kind, q, list(range(bsz)), list(lens), 1 / math.sqrt(d), poison=True)
    ref = OS.attention_batch(q.astype(np.float64), cache, kind, list(range(bsz)), list(lens), 1 / math.sqrt(d))
    assert_rel(o, ref, what=f"ragged {kind} {list(lens)}")
