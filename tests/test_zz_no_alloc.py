"""qkdec_step_noalloc (the step on the library's fixed device scratch, for
callers that cannot allocate) against qkdec_step on the same inputs: two
calls in a row, the second with fewer sequences, each bitwise equal to the
workspace entry point (same kernels, same order of arithmetic)."""
import copy

import numpy as np
import pytest

import synth
from tests.gpu_util import sync, ws

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qd():
    import quantized_decode_amd as m
    m.load_library()
    return m


def _setup(qd, model, caches, bsz):
    import torch
    from quantized_decode_amd.tensors import dev, upload_cache, upload_model
    embed, lm_head, norm, layers = upload_model(model)
    kv = [upload_cache(c) for c in caches]
    sm = qd.StepModel(model.dims, embed, lm_head, norm, layers, [k.desc for k in kv])
    sm._keep = (embed, lm_head, norm, layers)
    return sm, kv


@pytest.mark.parametrize("shape,kind", [("toy", "f16"), ("toy", "q8_0"), ("full", "q8_0")])
def test_noalloc_step_equals_workspace_step(qd, shape, kind):
    # full: one Qwen-shaped layer, whose Q8_0 new tokens are staged in the
    # scratch by the QKV projection and appended by the attention kernel
    import torch
    from quantized_decode_amd.tensors import dev
    dims = synth.TOY if shape == "toy" else synth.QWEN_SHAPED
    n_layers = None if shape == "toy" else 1
    for call, (bsz, L) in enumerate([(4, 128), (2, 96)]):
        model = synth.make_model(dims, 1600 + call, n_layers=n_layers)
        st = synth.Streams(1610 + call)
        caches = [synth.kv_cache(kind, st.next(), st.next(), bsz, dims.n_kv_heads, 160, dims.head_dim, [L] * bsz)
                  for _ in model.layers]
        tok = synth.tokens(st.next(), bsz, dims.vocab)
        outs = []
        for which in ("workspace", "noalloc"):
            sm, kv = _setup(qd, model, copy.deepcopy(caches), bsz)
            slot = dev(np.arange(bsz, dtype=np.int32))
            pos = dev(np.full(bsz, L, np.int32))
            tk = dev(tok.astype(np.int32))
            logits = torch.empty((bsz, dims.vocab), dtype=torch.float32, device="cuda")
            if which == "workspace":
                w = ws(qd.qkdec_step_workspace_size(sm, bsz))
                qd.qkdec_workspace_init(w)
                for _ in range(2):
                    qd.qkdec_step(sm, slot, pos, tk, bsz, w, logits=logits)
                sync()
                assert qd.qkdec_step_status(w) == 0
            else:
                err = torch.zeros(1, dtype=torch.int32, device="cuda")
                for _ in range(2):
                    qd.qkdec_step_noalloc(sm, slot, pos, tk, bsz, err, logits=logits)
                sync()
                assert int(err.item()) == 0
            outs.append((logits.cpu().numpy(), tk.cpu().numpy(), pos.cpu().numpy(),
                         [k.logical() for k in kv]))
        (la, ta, pa, ca), (lb, tb, pb, cb) = outs
        assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)), f"call {call}: logits"
        assert np.array_equal(ta, tb) and np.array_equal(pa, pb) and (pa == L + 2).all(), f"call {call}"
        for x, y in zip(ca, cb):
            for name, arr in vars(x).items():
                assert np.array_equal(arr.view(np.uint8), getattr(y, name).view(np.uint8)), (call, name)


def test_noalloc_capacity_flag_and_size_limit(qd):
    import ctypes
    import torch
    from quantized_decode_amd.tensors import dev
    dims = synth.TOY
    model = synth.make_model(dims, 1620)
    st = synth.Streams(1621)
    caches = [synth.kv_cache("f16", st.next(), st.next(), 2, dims.n_kv_heads, 64, dims.head_dim, [32, 32])
              for _ in model.layers]
    sm, kv = _setup(qd, model, caches, 2)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    tk = dev(np.array([1, 2], np.int32))
    qd.qkdec_step_noalloc(sm, dev(np.array([0, 1], np.int32)), dev(np.array([64, 10], np.int32)), tk, 2, err)
    sync()
    assert int(err.item()) == -5
    # a cache whose attention partials alone exceed the scratch is refused
    big = [qd.kv_layer(qd.KV_F16, dims.n_kv_heads, dims.head_dim, 1 << 25, 16, k.k, k.v) for k in kv]
    sm_big = qd.StepModel(dims, *sm._keep, big)
    assert qd.qkdec_step_workspace_size(sm_big, 16) > qd.qkdec_step_noalloc_max_bytes()
    with pytest.raises(qd.QkdecError) as e:
        qd.qkdec_step_noalloc(sm_big, dev(np.zeros(16, np.int32)), dev(np.zeros(16, np.int32)),
                              dev(np.zeros(16, np.int32)), 16, err)
    assert e.value.status == -4
