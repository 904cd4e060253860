"""The Qwen-shaped step at the depth and batch sizes the bench times, against
the oracle: the last two layers of the full 36-layer step, a teacher-forced
run of consecutive steps, and the partly filled second row pass of the fused
projections (B = 3 and 12).

Each layer is checked stage by stage against the oracle fed with the GPU's
own input to that stage (check_layer_stages): with the synthetic weights a
single fp16 rounding that lands on the other side of a midpoint can move a
near-tied softmax, so the stage-wise comparison is the one whose bound holds
for every sequence.  The end-to-end logits of the teacher-forced run are also
compared with the oracle's whole step from the same state.
"""
import copy
from types import SimpleNamespace

import numpy as np
import pytest

import synth
from oracle import ops as OO
from oracle import step as OS
from tests.gpu_util import LOGIT_ABS_TOL, sync, ws
from tests.test_gpu_step import _View, _within_f16_ulp, check_layer_stages, compare_logits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qd():
    import quantized_decode_amd as m
    m.load_library()
    return m


@pytest.fixture
def memo_dequant(monkeypatch):
    """Memoize the oracle's Q4_K row dequantization (a pure function of the
    matrix bytes and the row range) for the duration of one test: the same
    full-width weights are otherwise decoded again by every GEMM of every
    step.  Results are unchanged; only repeated work is skipped."""
    from oracle import formats as OF
    from oracle import ops as OO_
    plain = OF.q4k_dequant_rows
    cache = {}

    def memo(mat, n_rows, n_cols, rows=None):
        key = (id(mat), n_rows, n_cols, None if rows is None else (rows.start, rows.stop, rows.step))
        hit = cache.get(key)
        if hit is None or hit[0] is not mat:
            hit = (mat, plain(mat, n_rows, n_cols, rows=rows))
            cache[key] = hit
        return hit[1]

    monkeypatch.setattr(OF, "q4k_dequant_rows", memo)
    monkeypatch.setattr(OO_, "q4k_dequant_rows", memo)
    yield
    cache.clear()


class DevState:
    """A step over device-resident layers and caches, run on truncated
    prefixes of the layer stack from the same (pos, tok) state."""

    def __init__(self, qd, dims, embed, lm_head, norm, layers, dkv, bsz):
        import torch
        self.qd, self.dims, self.bsz = qd, dims, bsz
        self.embed, self.lm_head, self.norm, self.layers, self.kv = embed, lm_head, norm, layers, dkv
        self.slot = torch.arange(bsz, dtype=torch.int32, device="cuda")
        self.pos = torch.zeros(bsz, dtype=torch.int32, device="cuda")
        self.tok = torch.zeros(bsz, dtype=torch.int32, device="cuda")
        self.logits = torch.empty((bsz, dims.vocab), dtype=torch.float32, device="cuda")
        self.sm = qd.StepModel(dims, embed, lm_head, norm, layers, [k.desc for k in dkv])
        self.ws = ws(qd.qkdec_step_workspace_size(self.sm, bsz))
        qd.qkdec_workspace_init(self.ws)

    def run(self, n_layers, pos, tok):
        """One step through layers[:n_layers] from (pos, tok); returns the views."""
        import torch
        self.pos.copy_(torch.as_tensor(np.asarray(pos, np.int32)))
        self.tok.copy_(torch.as_tensor(np.asarray(tok, np.int32)))
        sub = self.qd.StepModel(self.dims, self.embed, self.lm_head, self.norm, self.layers[:n_layers],
                                [k.desc for k in self.kv[:n_layers]])
        self.sm_run = sub
        self.qd.qkdec_step(sub, self.slot, self.pos, self.tok, self.bsz, self.ws, logits=self.logits)
        sync()
        assert self.qd.qkdec_step_status(self.ws) == 0
        return _View(self.qd, self, self.dims, self.bsz)


def _host_layer(ly):
    return SimpleNamespace(**{k: v.cpu().numpy() for k, v in ly.items()})


def _device_kv(qd, kind, k, v, ks, vs, n_kv, d, cap, n_slots):
    from quantized_decode_amd import KV_KINDS, kv_layer
    from quantized_decode_amd.tensors import DeviceKV
    return DeviceKV(KV_KINDS[kind], k, v, ks, vs, kv_layer(KV_KINDS[kind], n_kv, d, cap, n_slots, k, v, ks, vs))


@pytest.mark.parametrize("kind", ["f16", "q8_0"])
def test_last_two_layers_of_the_36_layer_step(qd, kind, memo_dequant):
    # The headline workload (36 layers, B = 8, L = 2400), model and caches drawn
    # on the GPU as the bench draws them.  Layers 34 and 35 are checked stage by
    # stage from the GPU's own residual stream: steps through 34, 35 and all 36
    # layers from the same state (each re-appends bitwise the same entries),
    # then the final norm, the full 151936-row LM head and the argmax.
    import torch
    import synth.device as sd
    dims = synth.QWEN_SHAPED
    bsz, L, cap = 8, 2400, 2432
    embed, lm_head, norm, layers = sd.model(dims, 1203)
    g = sd.generator(1204)
    dkv = [_device_kv(qd, kind, *sd.kv_cache(g, kind, bsz, dims.n_kv_heads, cap, dims.head_dim, L),
                      dims.n_kv_heads, dims.head_dim, cap, bsz) for _ in layers]
    tok = torch.randint(0, dims.vocab, (bsz,), generator=g, device="cuda").cpu().numpy()
    pos = np.full(bsz, L)
    before = {li: dkv[li].logical() for li in (34, 35)}
    st = DevState(qd, dims, embed, lm_head, norm, layers, dkv, bsz)
    x_in = st.run(34, pos, tok).x
    slots = list(range(bsz))
    for li in (34, 35):
        vw = st.run(li + 1, pos, tok)
        check_layer_stages(dims, kind, _host_layer(layers[li]), x_in, pos, vw, dkv[li], before[li], slots)
        x_in = vw.x
    nf = norm.cpu().numpy()
    _within_f16_ulp(vw.h, OO.rmsnorm(vw.x, nf, dims.rms_eps), "final RMSNorm")
    ref = OO.dense_gemm(lm_head.cpu().numpy(), vw.h)
    compare_logits(st.logits.cpu().numpy(), ref, st.tok.cpu().numpy(), f"LM head after 36 layers ({kind})")
    assert (st.pos.cpu().numpy() == pos + 1).all()


@pytest.mark.parametrize("kind", ["f16", "q8_0"])
def test_teacher_forced_steps_full_width(qd, kind, memo_dequant):
    # Four consecutive decode steps of a two-layer decoder of the full width
    # (hidden 4096, 32/8 heads of 128, FFN 12288: every projection runs the
    # kernels the bench times; vocabulary 16384), B = 8 at L = 2400.  Step t
    # starts from the GPU's own cache bytes, positions and tokens after step
    # t-1 (teacher forcing).  Per step: both layers stage by stage, the final
    # norm, LM head and argmax, and the end-to-end logits against the oracle's
    # whole step from the same state.
    from quantized_decode_amd.tensors import upload_cache, upload_model
    dims = synth.ModelDims(n_layers=2, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=12288,
                           vocab=16384)
    bsz, L, cap = 8, 2400, 2432
    model = synth.make_model(dims, 1403)
    stm = synth.Streams(1404)
    caches = [synth.kv_cache(kind, stm.next(), stm.next(), bsz, dims.n_kv_heads, cap, dims.head_dim, [L] * bsz)
              for _ in model.layers]
    tok = synth.tokens(stm.next(), bsz, dims.vocab)
    embed, lm_head, norm, layers = upload_model(model)
    dkv = [upload_cache(c) for c in caches]
    st = DevState(qd, dims, embed, lm_head, norm, layers, dkv, bsz)
    slots = list(range(bsz))
    pos = np.full(bsz, L)
    worst = 0.0
    for step in range(4):
        state = [d.logical() for d in dkv]                 # the GPU's cache before this step
        x_in = model.embed[tok].astype(np.float64)
        for li in range(dims.n_layers):
            vw = st.run(li + 1, pos, tok)
            check_layer_stages(dims, kind, model.layers[li], x_in, pos, vw, dkv[li], state[li], slots)
            x_in = vw.x
        _within_f16_ulp(vw.h, OO.rmsnorm(vw.x, model.norm_final, dims.rms_eps), f"final RMSNorm, step {step}")
        lg, gtok = st.logits.cpu().numpy(), st.tok.cpu().numpy()
        compare_logits(lg, OO.dense_gemm(model.lm_head, vw.h), gtok, f"LM head, step {step} ({kind})")
        assert (st.pos.cpu().numpy() == pos + 1).all()
        # end to end: the oracle's whole step from the same state
        ref, rtok = OS.decode_step(model, copy.deepcopy(state), kind, slots, pos, tok)
        worst = max(worst, compare_logits(lg, ref, gtok, f"end-to-end logits, step {step} ({kind})"))
        pos = pos + 1
        tok = gtok.astype(np.int32)
    assert worst <= LOGIT_ABS_TOL


@pytest.mark.parametrize("bsz,kind", [(3, "f16"), (12, "f16"), (12, "q8_0")])
def test_full_width_layer_middle_batch_sizes(qd, bsz, kind):
    # batch sizes whose sequences only partly fill the projections' second pass
    # of eight rows (B = 12) or the first (B = 3): one Qwen-shaped layer at
    # L = 300, stage by stage, then final norm, LM head and argmax
    from tests.test_gpu_step import GpuStep, build
    dims = synth.QWEN_SHAPED
    L = 300
    slots = list(range(bsz))
    model, caches, tok = build(dims, 1503 + bsz, kind, bsz, L, 320, n_layers=1)
    pos = np.full(bsz, L)
    g = GpuStep(qd, model, caches, bsz, slots)
    g.set(pos, tok)
    g.step()
    vw = _View(qd, g, dims, bsz)
    check_layer_stages(dims, kind, model.layers[0], model.embed[tok].astype(np.float64), pos, vw, g.kv[0], caches[0],
                       slots)
    _within_f16_ulp(vw.h, OO.rmsnorm(vw.x, model.norm_final, dims.rms_eps), "final RMSNorm")
    compare_logits(g.logits.cpu().numpy(), OO.dense_gemm(model.lm_head, vw.h), g.tok.cpu().numpy(),
                   f"LM head (B={bsz}, {kind})")
    assert (g.pos.cpu().numpy() == pos + 1).all()

