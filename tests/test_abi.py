"""The C ABI library loads, exports every entry point include/qkdec.h declares,
and rejects bad arguments before touching the GPU (CPU only: no compute)."""
import ctypes
import os
import re

import pytest

import quantized_decode_amd as qd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qkdec.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qkdec_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(qd.LIB_PATH):
        pytest.fail("libqkdec.so is not built (run __graft_entry__.build())")
    return qd.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
    # and the binding declares a signature for each
    assert set(names) == set(qd._SIGNATURES)


def test_status_strings_and_version(lib):
    assert lib.qkdec_abi_version() == 1
    for code, name in qd.STATUS_NAMES.items():
        assert lib.qkdec_status_str(code).decode().startswith(name)
    assert b"unknown" in lib.qkdec_status_str(42)


def test_build_id_names_the_sources_it_was_built_from(lib):
    # the id is a hash of the sources; a stale build (sources edited since)
    # reports a different one, which is how recorded counter figures are dropped
    from quantized_decode_amd.build import source_id
    assert qd.qkdec_build_id() == source_id()


FAKE = 0x10000   # never dereferenced: every call below fails validation first


def test_gemm_validation(lib):
    ws = 1 << 20
    g = lib.qkdec_gemm_q4k
    assert g(None, 64, 256, FAKE, 256, 1, FAKE, 64, None, 0, FAKE, ws, None) == -1
    assert g(FAKE, 64, 256, FAKE, 256, 17, FAKE, 64, None, 0, FAKE, ws, None) == -2
    assert g(FAKE, 64, 256, FAKE, 256, 0, FAKE, 64, None, 0, FAKE, ws, None) == -2
    assert g(FAKE, 64, 300, FAKE, 300, 1, FAKE, 64, None, 0, FAKE, ws, None) == -2
    assert g(FAKE, 60, 256, FAKE, 256, 1, FAKE, 64, None, 0, FAKE, ws, None) == -2
    assert g(FAKE, 64, 256, FAKE, 128, 1, FAKE, 64, None, 0, FAKE, ws, None) == -2   # ldx < K
    assert g(FAKE + 4, 64, 256, FAKE, 256, 1, FAKE, 64, None, 0, FAKE, ws, None) == -3
    assert g(FAKE, 64, 256, FAKE + 2, 256, 1, FAKE, 64, None, 0, FAKE, ws, None) == -3
    assert g(FAKE, 64, 256, FAKE, 260, 1, FAKE, 64, None, 0, FAKE, ws, None) == -3
    assert g(FAKE, 64, 256, FAKE, 256, 1, None, 64, None, 0, FAKE, ws, None) == -1
    assert g(FAKE, 64, 256, FAKE, 256, 1, FAKE, 32, None, 0, FAKE, ws, None) == -2   # ldy < N
    assert g(FAKE, 64, 256, FAKE, 256, 1, FAKE, 64, None, 0, None, ws, None) == -4
    assert g(FAKE, 64, 256, FAKE, 256, 1, FAKE, 64, None, 0, FAKE, 4, None) == -4
    need = lib.qkdec_gemm_q4k_workspace_size(4096, 12288, 8)
    assert need > 0 and lib.qkdec_gemm_q4k_workspace_size(4096, 300, 8) == 0
    assert g(FAKE, 4096, 12288, FAKE, 12288, 8, FAKE, 4096, None, 0, FAKE, need - 1, None) == -4
    s = lib.qkdec_gemm_q4k_swiglu
    assert s(FAKE, 8, 256, FAKE, 256, 1, FAKE, 8, FAKE, ws, None) == -2      # 2F % 16
    assert s(FAKE, 64, 256, FAKE, 256, 1, None, 64, FAKE, ws, None) == -1
    assert s(FAKE, 64, 256, FAKE, 256, 1, FAKE, 32, FAKE, ws, None) == -2   # lda < F
    assert lib.qkdec_dequant_q4k(None, 1, FAKE, None) == -1
    assert lib.qkdec_dequant_q4k(FAKE, 0, FAKE, None) == -2


def _kv(**kw):
    d = dict(type=0, n_kv_heads=8, head_dim=128, capacity=2432, n_slots=8, k=FAKE, v=FAKE, k_scale=None, v_scale=None)
    d.update(kw)
    return qd.KVLayer(**d)


def test_kv_and_attention_validation(lib):
    app = lib.qkdec_kv_append_f16
    assert app(ctypes.byref(_kv(type=5)), FAKE, FAKE, FAKE, FAKE, 1, None, None) == -1
    assert app(ctypes.byref(_kv(head_dim=96)), FAKE, FAKE, FAKE, FAKE, 1, None, None) == -2
    assert app(ctypes.byref(_kv(capacity=33)), FAKE, FAKE, FAKE, FAKE, 1, None, None) == -2
    assert app(ctypes.byref(_kv(k=FAKE + 8)), FAKE, FAKE, FAKE, FAKE, 1, None, None) == -3
    assert app(ctypes.byref(_kv(type=1, k_scale=FAKE, v_scale=FAKE)), FAKE, FAKE, FAKE, FAKE, 1, None, None) == -1
    assert app(ctypes.byref(_kv()), FAKE, FAKE, FAKE, FAKE, 0, None, None) == -2
    assert app(ctypes.byref(_kv()), None, FAKE, FAKE, FAKE, 1, None, None) == -1
    q8 = lib.qkdec_kv_append_q8_0
    assert q8(ctypes.byref(_kv(type=1)), FAKE, FAKE, FAKE, FAKE, 1, None, None) == -1   # scales missing
    assert q8(ctypes.byref(_kv()), FAKE, FAKE, FAKE, FAKE, 1, None, None) == -1          # type mismatch
    # keys and values in different formats: only the Q8_0 tensor needs its scales;
    # the strict entry points reject the mixed types, the generic one validates them
    gen = lib.qkdec_kv_append
    assert gen(ctypes.byref(_kv(type=2, v_scale=FAKE)), FAKE, FAKE, FAKE, FAKE, 1, None, None) == -1   # k_scale
    assert gen(ctypes.byref(_kv(type=3, k_scale=FAKE)), FAKE, FAKE, FAKE, FAKE, 1, None, None) == -1   # v_scale
    assert gen(ctypes.byref(_kv(type=2, k_scale=FAKE + 2)), FAKE, FAKE, FAKE, FAKE, 1, None, None) == -3
    assert gen(ctypes.byref(_kv(type=5)), FAKE, FAKE, FAKE, FAKE, 1, None, None) == -1
    # E4M3 keys and values: no scales; only the generic entry point takes the type
    assert gen(ctypes.byref(_kv(type=4)), FAKE, FAKE, FAKE, FAKE, 17, None, None) == -2
    assert gen(ctypes.byref(_kv(type=4, v=FAKE + 4)), FAKE, FAKE, FAKE, FAKE, 1, None, None) == -3
    assert app(ctypes.byref(_kv(type=4)), FAKE, FAKE, FAKE, FAKE, 1, None, None) == -1
    assert q8(ctypes.byref(_kv(type=4)), FAKE, FAKE, FAKE, FAKE, 1, None, None) == -1
    assert gen(ctypes.byref(_kv(type=2, k_scale=FAKE)), FAKE, FAKE, FAKE, FAKE, 17, None, None) == -2
    assert app(ctypes.byref(_kv(type=2, k_scale=FAKE)), FAKE, FAKE, FAKE, FAKE, 1, None, None) == -1
    assert q8(ctypes.byref(_kv(type=3, v_scale=FAKE)), FAKE, FAKE, FAKE, FAKE, 1, None, None) == -1
    assert lib.qkdec_attn_workspace_size(8, 32, ctypes.byref(_kv(type=3, v_scale=FAKE))) > 0
    att = lib.qkdec_attn_decode
    kv = _kv()
    need = lib.qkdec_attn_workspace_size(8, 32, ctypes.byref(kv))
    # rows for up to 32 runs per (sequence, head): ceil(2432 / 1024) = 3 rounded
    # up to a multiple of the runs one sequence takes when alone (256 / 8)
    assert need == 8 * 32 * 32 * 130 * 4
    assert att(ctypes.byref(kv), FAKE, FAKE, 8, FAKE, 30, 0.1, FAKE, None, FAKE, need, None) == -2   # 30 % 8
    assert att(ctypes.byref(kv), FAKE, FAKE, 8, FAKE, 256, 0.1, FAKE, None, FAKE, need, None) == -2  # group 32
    assert att(ctypes.byref(kv), FAKE, FAKE, 17, FAKE, 32, 0.1, FAKE, None, FAKE, need, None) == -2
    assert att(ctypes.byref(kv), FAKE, FAKE, 8, FAKE, 32, 0.1, None, None, FAKE, need, None) == -1
    assert att(ctypes.byref(kv), FAKE, FAKE, 8, FAKE, 32, 0.1, FAKE, None, FAKE, need - 4, None) == -4
    assert att(ctypes.byref(kv), FAKE, FAKE, 8, FAKE + 2, 32, 0.1, FAKE, None, FAKE, need, None) == -3
    assert att(ctypes.byref(kv), FAKE, FAKE, 8, FAKE, 32, float("nan"), FAKE, None, FAKE, need, None) == -1


def test_lm_head_and_step_validation(lib):
    lm = lib.qkdec_lm_head_argmax
    ws = lib.qkdec_lm_head_workspace_size(151936, 8)
    assert ws > 0
    assert lm(FAKE, 151936, 4096, FAKE, 8, None, None, FAKE, ws, None) == -1
    assert lm(FAKE, 151930, 4096, FAKE, 8, None, FAKE, FAKE, ws, None) == -2
    assert lm(FAKE, 151936, 4000, FAKE, 8, None, FAKE, FAKE, ws, None) == -2
    assert lm(FAKE, 151936, 4096, FAKE, 8, None, FAKE, FAKE, 4, None) == -4
    layers = (qd.Layer * 2)(qd.Layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE), qd.Layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE))
    m = qd.Model(2, 512, 8, 2, 64, 1536, 4096, 1e-6, 1e6, FAKE, FAKE, FAKE, ctypes.cast(layers, ctypes.POINTER(qd.Layer)))
    kvs = (qd.KVLayer * 2)(_kv(n_kv_heads=2, head_dim=64, capacity=256, n_slots=2),
                            _kv(n_kv_heads=2, head_dim=64, capacity=256, n_slots=2))
    need = lib.qkdec_step_workspace_size(ctypes.byref(m), 2, kvs)
    assert need > 0
    step = lib.qkdec_step
    assert step(ctypes.byref(m), kvs, FAKE, FAKE, FAKE, 2, None, FAKE, need - 1, None) == -4
    assert step(ctypes.byref(m), kvs, FAKE, FAKE, FAKE, 17, None, FAKE, need, None) == -2
    assert step(ctypes.byref(m), kvs, None, FAKE, FAKE, 2, None, FAKE, need, None) == -1
    assert step(ctypes.byref(m), kvs, FAKE, FAKE, FAKE, 2, None, FAKE + 16, need, None) == -3
    kvs[1] = _kv(n_kv_heads=2, head_dim=64, capacity=288, n_slots=2)    # layers disagree
    assert step(ctypes.byref(m), kvs, FAKE, FAKE, FAKE, 2, None, FAKE, need, None) == -2
    assert lib.qkdec_step_workspace_size(ctypes.byref(m), 2, kvs) == 0
    kvs[1] = _kv(n_kv_heads=2, head_dim=64, capacity=256, n_slots=2)
    m.n_q_heads = 6                                                       # 6 % 4 ok, 6*64 % 256 != 0
    assert step(ctypes.byref(m), kvs, FAKE, FAKE, FAKE, 2, None, FAKE, need, None) == -2
    m.n_q_heads = 8
    m.vocab = 4095
    assert step(ctypes.byref(m), kvs, FAKE, FAKE, FAKE, 2, None, FAKE, need, None) == -2
    m.vocab = 4096
    layers[1].w_o = None
    assert step(ctypes.byref(m), kvs, FAKE, FAKE, FAKE, 2, None, FAKE, need, None) == -1
    p = ctypes.c_void_p()
    assert lib.qkdec_plan_create(ctypes.byref(p), ctypes.byref(m), kvs, FAKE, FAKE, FAKE, 2, None, FAKE, need,
                                 None) == -1   # a plan needs a real stream
    assert lib.qkdec_plan_launch(None, None) == -1
    lib.qkdec_plan_destroy(None)
    assert lib.qkdec_workspace_init(None, 16, None) == -1


def test_paged_validation(lib):
    # page size a power of two, a page table, max_pages >= 1, sizes checked before any launch
    att, app = lib.qkdec_attn_decode_paged, lib.qkdec_kv_append_paged
    pool = _kv(capacity=256, n_slots=64)
    need = lib.qkdec_attn_paged_workspace_size(8, 32, ctypes.byref(pool), 16)
    # rows for up to 32 runs per (sequence, head): ceil(16 * 256 / 1024) = 4
    # rounded up to a multiple of 256 / 8
    assert need == 8 * 32 * 32 * 130 * 4
    assert lib.qkdec_attn_paged_workspace_size(8, 32, ctypes.byref(pool), 0) == 0
    assert att(ctypes.byref(_kv(capacity=96)), FAKE, 4, FAKE, 8, FAKE, 32, 0.1, FAKE, None, FAKE, need, None) == -2
    assert att(ctypes.byref(pool), None, 4, FAKE, 8, FAKE, 32, 0.1, FAKE, None, FAKE, need, None) == -1
    assert att(ctypes.byref(pool), FAKE, 0, FAKE, 8, FAKE, 32, 0.1, FAKE, None, FAKE, need, None) == -2
    assert att(ctypes.byref(pool), FAKE, 1 << 23, FAKE, 8, FAKE, 32, 0.1, FAKE, None, FAKE, need, None) == -2
    assert att(ctypes.byref(pool), FAKE + 2, 16, FAKE, 8, FAKE, 32, 0.1, FAKE, None, FAKE, need, None) == -3
    assert att(ctypes.byref(pool), FAKE, 16, FAKE, 17, FAKE, 32, 0.1, FAKE, None, FAKE, need, None) == -2
    assert att(ctypes.byref(pool), FAKE, 16, FAKE, 8, FAKE, 30, 0.1, FAKE, None, FAKE, need, None) == -2
    assert att(ctypes.byref(pool), FAKE, 16, FAKE, 8, FAKE, 32, 0.1, FAKE, None, FAKE, need - 4, None) == -4
    assert att(ctypes.byref(pool), FAKE, 16, FAKE, 8, FAKE, 32, 0.1, None, None, FAKE, need, None) == -1
    assert app(ctypes.byref(_kv(capacity=96)), FAKE, 4, FAKE, FAKE, FAKE, 1, None, None) == -2
    assert app(ctypes.byref(pool), None, 4, FAKE, FAKE, FAKE, 1, None, None) == -1
    assert app(ctypes.byref(pool), FAKE, 4, FAKE, FAKE, FAKE, 0, None, None) == -2
    assert app(ctypes.byref(_kv(type=1, capacity=256)), FAKE, 4, FAKE, FAKE, FAKE, 1, None, None) == -1  # scales


def test_noalloc_step_validation(lib):
    # every rejection happens before any device work (this runs without a GPU)
    layers = (qd.Layer * 2)(qd.Layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE), qd.Layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE))
    m = qd.Model(2, 512, 8, 2, 64, 1536, 4096, 1e-6, 1e6, FAKE, FAKE, FAKE, ctypes.cast(layers, ctypes.POINTER(qd.Layer)))
    kvs = (qd.KVLayer * 2)(_kv(n_kv_heads=2, head_dim=64, capacity=256, n_slots=2),
                            _kv(n_kv_heads=2, head_dim=64, capacity=256, n_slots=2))
    cap = lib.qkdec_step_noalloc_max_bytes()
    assert cap == 32 << 20
    step = lib.qkdec_step_noalloc
    assert step(ctypes.byref(m), kvs, FAKE, FAKE, FAKE, 2, None, None, None) == -1       # no err word
    assert step(ctypes.byref(m), kvs, None, FAKE, FAKE, 2, None, FAKE, None) == -1
    assert step(ctypes.byref(m), kvs, FAKE, FAKE, FAKE, 0, None, FAKE, None) == -2
    # a cache so long that the attention partials alone exceed the scratch
    big = (qd.KVLayer * 2)(_kv(n_kv_heads=2, head_dim=64, capacity=1 << 25, n_slots=16),
                            _kv(n_kv_heads=2, head_dim=64, capacity=1 << 25, n_slots=16))
    assert lib.qkdec_step_workspace_size(ctypes.byref(m), 16, big) > cap
    assert step(ctypes.byref(m), big, FAKE, FAKE, FAKE, 16, None, FAKE, None) == -4


def test_prefill_validation(lib):
    layers = (qd.Layer * 2)(qd.Layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE), qd.Layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE))
    m = qd.Model(2, 512, 8, 2, 64, 1536, 4096, 1e-6, 1e6, FAKE, FAKE, FAKE, ctypes.cast(layers, ctypes.POINTER(qd.Layer)))
    kvs = (qd.KVLayer * 2)(_kv(n_kv_heads=2, head_dim=64, capacity=256, n_slots=2),
                            _kv(n_kv_heads=2, head_dim=64, capacity=256, n_slots=2))
    need = lib.qkdec_prefill_workspace_size(ctypes.byref(m), kvs)
    assert need > lib.qkdec_step_workspace_size(ctypes.byref(m), 16, kvs)
    pf = lib.qkdec_prefill
    assert pf(ctypes.byref(m), kvs, 0, 0, None, 4, None, FAKE, FAKE, need, None) == -1      # no tokens
    assert pf(ctypes.byref(m), kvs, 0, 0, FAKE, 4, None, None, FAKE, need, None) == -1      # no tok_out
    assert pf(ctypes.byref(m), kvs, 2, 0, FAKE, 4, None, FAKE, FAKE, need, None) == -2      # slot outside
    assert pf(ctypes.byref(m), kvs, 0, 0, FAKE, 0, None, FAKE, FAKE, need, None) == -2      # empty prompt
    assert pf(ctypes.byref(m), kvs, 0, 250, FAKE, 7, None, FAKE, FAKE, need, None) == -5    # past capacity
    assert pf(ctypes.byref(m), kvs, 0, 0, FAKE, 4, None, FAKE, FAKE, need - 1, None) == -4
    assert pf(ctypes.byref(m), kvs, 0, 0, FAKE, 4, None, FAKE, FAKE + 16, need, None) == -3


def test_prefill_paged_validation(lib):
    # pool page size a power of two, a page table, start + n within max_pages
    # pages, query heads per KV head a power of two; all before any launch
    layers = (qd.Layer * 2)(qd.Layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE), qd.Layer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE))
    m = qd.Model(2, 512, 8, 2, 64, 1536, 4096, 1e-6, 1e6, FAKE, FAKE, FAKE, ctypes.cast(layers, ctypes.POINTER(qd.Layer)))
    pools = (qd.KVLayer * 2)(_kv(n_kv_heads=2, head_dim=64, capacity=64, n_slots=32),
                              _kv(n_kv_heads=2, head_dim=64, capacity=64, n_slots=32))
    need = lib.qkdec_prefill_paged_workspace_size(ctypes.byref(m), pools)
    assert need > 0
    pf = lib.qkdec_prefill_paged
    assert pf(ctypes.byref(m), pools, None, 4, 0, FAKE, 4, None, FAKE, FAKE, need, None) == -1     # no table
    assert pf(ctypes.byref(m), pools, FAKE, 0, 0, FAKE, 4, None, FAKE, FAKE, need, None) == -2     # max_pages
    assert pf(ctypes.byref(m), pools, FAKE, 4, 0, None, 4, None, FAKE, FAKE, need, None) == -1     # no tokens
    assert pf(ctypes.byref(m), pools, FAKE, 4, 0, FAKE, 0, None, FAKE, FAKE, need, None) == -2     # empty prompt
    assert pf(ctypes.byref(m), pools, FAKE, 4, 250, FAKE, 7, None, FAKE, FAKE, need, None) == -5   # past 4 pages
    assert pf(ctypes.byref(m), pools, FAKE, 4, 0, FAKE, 4, None, FAKE, FAKE, need - 1, None) == -4
    assert pf(ctypes.byref(m), pools, FAKE + 2, 4, 0, FAKE, 4, None, FAKE, FAKE, need, None) == -3
    odd = (qd.KVLayer * 2)(_kv(n_kv_heads=2, head_dim=64, capacity=96, n_slots=32),
                            _kv(n_kv_heads=2, head_dim=64, capacity=96, n_slots=32))
    assert pf(ctypes.byref(m), odd, FAKE, 4, 0, FAKE, 4, None, FAKE, FAKE, need, None) == -2      # page size
    m3 = qd.Model(2, 512, 12, 4, 64, 1536, 4096, 1e-6, 1e6, FAKE, FAKE, FAKE,
                  ctypes.cast(layers, ctypes.POINTER(qd.Layer)))
    p3 = (qd.KVLayer * 2)(_kv(n_kv_heads=4, head_dim=64, capacity=64, n_slots=32),
                           _kv(n_kv_heads=4, head_dim=64, capacity=64, n_slots=32))
    assert pf(ctypes.byref(m3), p3, FAKE, 4, 0, FAKE, 4, None, FAKE, FAKE, need, None) == -2      # G = 3
