"""The full batched decode step (and its HIP-graph plan) on the GPU against the oracle."""
import copy

import numpy as np
import pytest

import synth
from oracle import step as OS
from tests.gpu_util import (LOGIT_ABS_TOL, assert_rel, attention_fp32_slack, f16_rounding_slack, propagate_slack,
                            rope_fp32_slack, sync, top2_gap, ws)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qd():
    import quantized_decode_amd as m
    m.load_library()
    return m


def _dev(a):
    from quantized_decode_amd.tensors import dev
    return dev(a)


def build(dims, seed, kind, bsz, length, cap, n_layers=None, n_slots=None):
    model = synth.make_model(dims, seed, n_layers=n_layers)
    st = synth.Streams(seed + 1)
    n_slots = bsz if n_slots is None else n_slots
    filled = [length] * n_slots
    caches = []
    for _ in model.layers:
        caches.append(synth.kv_cache(kind, st.next(), st.next(), n_slots, dims.n_kv_heads, cap, dims.head_dim,
                                     filled))
    tok = synth.tokens(st.next(), bsz, dims.vocab)
    return model, caches, tok


class GpuStep:
    def __init__(self, qd, model, caches, bsz, slots):
        import torch
        from quantized_decode_amd.tensors import upload_cache, upload_model
        self.qd = qd
        self.embed, self.lm_head, self.norm, self.layers = upload_model(model)
        self.kv = [upload_cache(c) for c in caches]
        self.sm = qd.StepModel(model.dims, self.embed, self.lm_head, self.norm, self.layers,
                               [k.desc for k in self.kv])
        self.bsz = bsz
        self.slot = _dev(np.asarray(slots, np.int32))
        self.pos = torch.zeros(bsz, dtype=torch.int32, device="cuda")
        self.tok = torch.zeros(bsz, dtype=torch.int32, device="cuda")
        self.logits = torch.empty((bsz, model.dims.vocab), dtype=torch.float32, device="cuda")
        self.ws = ws(qd.qkdec_step_workspace_size(self.sm, bsz))
        qd.qkdec_workspace_init(self.ws)

    def set(self, pos, tok):
        import torch
        self.pos.copy_(torch.as_tensor(np.asarray(pos, np.int32)))
        self.tok.copy_(torch.as_tensor(np.asarray(tok, np.int32)))

    def step(self):
        self.qd.qkdec_step(self.sm, self.slot, self.pos, self.tok, self.bsz, self.ws, logits=self.logits)
        sync()
        return self.logits.cpu().numpy(), self.tok.cpu().numpy(), self.pos.cpu().numpy()


def compare_logits(lg, ref, gtok, what):
    d = float(np.abs(lg - ref).max())
    assert d <= LOGIT_ABS_TOL, f"{what}: max |dlogit| {d:.3e}"
    for b in range(ref.shape[0]):
        if top2_gap(ref[b]) > 1e-3:
            assert gtok[b] == int(np.argmax(ref[b])), f"{what}: argmax differs for sequence {b}"
    return d


@pytest.mark.parametrize("kind", ["f16", "q8_0", "q8k_f16v", "f16k_q8v", "fp8"])
def test_toy_step_multi_step(qd, kind):
    # the toy workload: 2-layer decoder, B = 2 sequences with 128 cached tokens
    dims = synth.TOY
    model, caches, tok = build(dims, 1000, kind, 2, 128, 160)
    g = GpuStep(qd, model, caches, 2, [0, 1])
    pos = np.array([128, 128])
    g.set(pos, tok)
    ocaches = copy.deepcopy(caches)
    for step in range(4):
        ref, otok = OS.decode_step(model, ocaches, kind, [0, 1], pos, tok)
        lg, gtok, gpos = g.step()
        compare_logits(lg, ref, gtok, f"{kind} step {step}")
        assert (gpos == pos + 1).all()
        pos = pos + 1
        tok = otok
        g.set(pos, tok)      # both sides continue from the oracle's token


def test_toy_step_appends_match_oracle(qd):
    dims = synth.TOY
    model, caches, tok = build(dims, 1000, "f16", 2, 128, 160)
    g = GpuStep(qd, model, caches, 2, [0, 1])
    g.set([128, 128], tok)
    g.step()
    ocaches = copy.deepcopy(caches)
    OS.decode_step(model, ocaches, "f16", [0, 1], [128, 128], tok)
    for li in range(dims.n_layers):
        kk, vv = g.kv[li].logical_f16()
        # untouched history identical; the appended token within one fp16 ulp (fp32 vs fp64 rounding)
        assert np.array_equal(kk[:, :, :128].view(np.uint16), caches[li].k[:, :, :128].view(np.uint16))
        for got, want in ((kk[:, :, 128], ocaches[li].k[:, :, 128]), (vv[:, :, 128], ocaches[li].v[:, :, 128])):
            gd, wd = got.astype(np.float64), want.astype(np.float64)
            ulp = np.abs(np.spacing(want.astype(np.float16)).astype(np.float64))
            assert (np.abs(gd - wd) <= ulp + 1e-12).all()
        assert not kk[:, :, 129:].any()


def test_step_batch_invariant_and_plan_replay(qd):
    dims = synth.TOY
    model, caches, tok = build(dims, 1000, "f16", 2, 128, 192)
    a = GpuStep(qd, model, caches, 2, [0, 1])
    a.set([128, 128], tok)
    outs_a = [a.step() for _ in range(3)]
    # one sequence alone gives bitwise the same logits (only the weights are shared)
    model1, caches1, _ = build(dims, 1000, "f16", 2, 128, 192)
    c = GpuStep(qd, model1, caches1, 1, [1])
    c.set([128], tok[1:])
    lg1, t1, _ = c.step()
    assert np.array_equal(lg1[0].view(np.uint32), outs_a[0][0][1].view(np.uint32))
    # a captured plan replays as consecutive steps, identical to eager steps
    import torch
    model2, caches2, _ = build(dims, 1000, "f16", 2, 128, 192)
    b = GpuStep(qd, model2, caches2, 2, [0, 1])
    b.set([128, 128], tok)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        plan = qd.Plan(b.sm, b.slot, b.pos, b.tok, 2, b.ws, logits=b.logits, stream=stream)
    for i in range(3):
        plan.launch(stream=stream)
        stream.synchronize()
        lg = b.logits.cpu().numpy()
        assert np.array_equal(lg.view(np.uint32), outs_a[i][0].view(np.uint32)), f"replay {i}"
        assert np.array_equal(b.tok.cpu().numpy(), outs_a[i][1])
        torch.cuda.synchronize()
    plan.destroy()
    for li in range(dims.n_layers):
        ka, va = a.kv[li].logical_f16()
        kb, vb = b.kv[li].logical_f16()
        assert np.array_equal(ka.view(np.uint16), kb.view(np.uint16))
        assert np.array_equal(va.view(np.uint16), vb.view(np.uint16))


def test_step_capacity_flag(qd):
    dims = synth.TOY
    model, caches, tok = build(dims, 1001, "f16", 2, 32, 64)
    g = GpuStep(qd, model, caches, 2, [0, 1])
    g.set([63, 10], tok)
    g.step()
    assert qd.qkdec_step_status(g.ws) == 0
    g.set([64, 10], tok)      # sequence 0 is full
    g.step()
    assert qd.qkdec_step_status(g.ws) == -5
    assert qd.qkdec_step_status(g.ws) == 0    # the flag was cleared


class _View:
    """Typed numpy copies of the step workspace's stage buffers."""

    def __init__(self, qd, g, dims, bsz):
        import torch
        v = qd.qkdec_step_workspace_views(g.sm, bsz)
        raw = g.ws
        hq = dims.n_q_heads * dims.head_dim
        nqkv = (dims.n_q_heads + 2 * dims.n_kv_heads) * dims.head_dim

        def take(name, n, dt):
            nb = bsz * n * torch.tensor([], dtype=dt).element_size()
            return raw[v[name]:v[name] + nb].view(dt).view(bsz, n).cpu().numpy().astype(np.float64)

        self.x = take("x", dims.hidden, torch.float32)
        self.h = take("h", dims.hidden, torch.float16)
        self.qkv = take("qkv", nqkv, torch.float32)
        self.q16 = take("q16", hq, torch.float16)
        self.o16 = take("o16", hq, torch.float16)
        self.a = take("a", dims.ffn, torch.float32)


def _cache_from_device(dkv, kind):
    return dkv.logical()


def _within_f16_ulp(got, want, what, slack=None):
    # one rounding to fp16 of an fp32 result against one of the fp64 result;
    # slack: a bound on how far the fp32 value itself may be from the exact one
    want16 = np.asarray(want, dtype=np.float64).astype(np.float16)
    ulp = np.abs(np.spacing(want16).astype(np.float64))
    allow = ulp * 1.0001 + (0.0 if slack is None else np.asarray(slack, dtype=np.float64))
    bad = np.abs(np.asarray(got, np.float64) - want16.astype(np.float64)) > allow
    assert not bad.any(), f"{what}: {int(bad.sum())} values beyond one fp16 ulp"


def check_layer_stages(dims, kind, ly, x_in, pos, vw, cache_dev, cache_before, slots):
    """Each stage of one layer against the oracle applied to the GPU's own input to
    that stage, so that no rounding difference propagates into the next check."""
    from oracle import formats as OF, ops as OO
    hq, hkv, hd = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    qrows, krows = hq * hd, hkv * hd
    pre = OO.rmsnorm(x_in, ly.norm_attn, dims.rms_eps)
    h = OF.round_f16(pre)
    nqkv = qrows + 2 * krows
    slack = propagate_slack(f16_rounding_slack(pre), nqkv, lambda: OF.q4k_dequant_rows(ly.w_qkv, nqkv, dims.hidden))
    assert_rel(vw.qkv, OO.q4k_gemm(ly.w_qkv, nqkv, dims.hidden, h), what="qkv projection", slack=slack)
    got = _cache_from_device(cache_dev, kind)
    for b, s in enumerate(slots):
        p = int(pos[b])
        qx = vw.qkv[b, :qrows].reshape(hq, hd)
        kx = vw.qkv[b, qrows:qrows + krows].reshape(hkv, hd)
        q = OO.rope(qx, p, dims.rope_base)
        k = OO.rope(kx, p, dims.rope_base)
        v = vw.qkv[b, qrows + krows:].reshape(hkv, hd)
        _within_f16_ulp(vw.q16[b], q.reshape(-1), f"rotated q, sequence {b}",
                        slack=rope_fp32_slack(qx, p, dims.rope_base).reshape(-1))
        rot_slack = {"k": rope_fp32_slack(kx, p, dims.rope_base), "v": None}
        for name, want, fmt in (("k", k, synth.KV_FORMATS[kind][0]), ("v", v, synth.KV_FORMATS[kind][1])):
            if fmt == "f16":
                _within_f16_ulp(getattr(got, name)[s, :, p], want, f"appended {name}, sequence {b}",
                                slack=rot_slack[name])
                assert np.array_equal(getattr(got, name)[s, :, :p].view(np.uint16),
                                      getattr(cache_before, name)[s, :, :p].view(np.uint16))
            elif fmt == "fp8":
                # the GPU rounds its fp32 value, the oracle the fp64 one: a code
                # may differ only by one E4M3 step, at a near-tie
                gc = getattr(got, name + "f8")
                dg = OF.fp8_e4m3_decode(gc[s, :, p])
                do = OF.fp8_e4m3_decode(OF.fp8_e4m3_encode(want))
                e = np.maximum(np.floor(np.log2(np.maximum(np.abs(do), 2.0 ** -6))), -6)
                assert (np.abs(dg - do) <= 2.0 ** (e - 3) * 1.0001).all(), f"appended {name}, sequence {b}"
                assert np.mean(dg != do) < 0.01, f"appended {name}, sequence {b}"
                assert np.array_equal(gc[s, :, :p], getattr(cache_before, name + "f8")[s, :, :p])
            else:
                gq, gs = getattr(got, name + "q"), getattr(got, name + "s")
                wq, wd = OF.q8_0_quantize(want)
                dg = gs[s, :, p].astype(np.float64)
                do = wd.astype(np.float64)
                assert (np.abs(dg - do) <= np.abs(np.spacing(wd).astype(np.float64)) * 1.0001).all(), name
                deq_g = OF.q8_0_dequant(gq[s, :, p], gs[s, :, p])
                deq_o = OF.q8_0_dequant(wq, wd)
                step = np.repeat(np.maximum(dg, do), 32, axis=-1)
                assert (np.abs(deq_g - deq_o) <= 1.01 * step).all(), f"appended {name}, sequence {b}"
                assert np.array_equal(gq[s, :, :p], getattr(cache_before, name + "q")[s, :, :p])
        kd, vd = OS.kv_read(got, kind, s, p + 1)
        qb = vw.q16[b].reshape(hq, hd)
        o = OO.attention(qb, kd, vd, 1.0 / np.sqrt(hd)).reshape(-1)
        # the fp32 scores' error carried through the softmax (large only near a
        # tie between keys of very different values), and the fp16 rounding of O
        # that fp32 cannot decide
        a_slack = attention_fp32_slack(qb, kd, vd, 1.0 / np.sqrt(hd)).reshape(-1)
        a_slack = a_slack + f16_rounding_slack(o)
        assert_rel(vw.o16[b], OF.round_f16(o), what=f"attention, sequence {b}", slack=a_slack)
    x1 = x_in + OO.q4k_gemm(ly.w_o, dims.hidden, qrows, vw.o16)
    pre2 = OO.rmsnorm(x1, ly.norm_ffn, dims.rms_eps)
    h2 = OF.round_f16(pre2)
    f = dims.ffn
    gu = OO.q4k_gemm(ly.w_gate_up, 2 * f, dims.hidden, h2)
    gs = propagate_slack(f16_rounding_slack(pre2), 2 * f,
                         lambda: OF.q4k_dequant_rows(ly.w_gate_up, 2 * f, dims.hidden))
    # first order through silu(g) * u (|silu'| <= 1.1), with the product of the two bounds on top
    g_, u_ = gu[:, :f], gu[:, f:]
    sg = 1.0 / (1.0 + np.exp(-np.clip(g_, -700, 700)))
    dsilu = np.abs(sg * (1.0 + g_ * (1.0 - sg)))
    a_slack = dsilu * np.abs(u_) * gs[:, :f] + np.abs(OO.silu(g_)) * gs[:, f:] + 1.1 * gs[:, :f] * gs[:, f:]
    assert_rel(vw.a, OO.swiglu(g_, u_), what="SwiGLU activation", slack=a_slack)
    a16 = OF.round_f16_blocked(vw.a)
    assert_rel(vw.x, x1 + OO.q4k_gemm(ly.w_down, dims.hidden, dims.ffn, a16), what="residual after the layer")


@pytest.mark.parametrize("kind", ["f16", "q8_0", "q8k_f16v", "fp8"])
def test_full_width_step_stagewise(qd, kind):
    # the Qwen-shaped model (hidden 4096, 32/8 heads of 128, FFN 12288, vocab 151936), first two
    # layers, B = 8 sequences at L = 2400.  With random Q4_K bytes the weights have a
    # positive mean, activations reach ~1e5 and several sequences' attention has
    # near-tied top scores, so an fp32 path and the fp64 oracle may legitimately part
    # after the first fp16 rounding that lands differently; every stage is therefore
    # checked against the oracle fed with the GPU's own input to that stage.
    from oracle import formats as OF, ops as OO
    dims = synth.QWEN_SHAPED
    bsz, L = 8, 2400
    slots = list(range(bsz))
    model, caches, tok = build(dims, 1003, kind, bsz, L, 2432, n_layers=2)
    pos = np.full(bsz, L)
    g = GpuStep(qd, model, caches, bsz, slots)
    one = qd.StepModel(dims, g.embed, g.lm_head, g.norm, g.layers[:1], [k.desc for k in g.kv[:1]])
    # layer 0 alone: its stages, then the final norm, LM head and sampling
    g.set(pos, tok)
    qd.qkdec_step(one, g.slot, g.pos, g.tok, bsz, g.ws, logits=g.logits)
    sync()
    vw = _View(qd, g, dims, bsz)
    x_emb = model.embed[tok].astype(np.float64)
    check_layer_stages(dims, kind, model.layers[0], x_emb, pos, vw, g.kv[0], caches[0], slots)
    x_l0 = vw.x.copy()
    k0 = g.kv[0].k[:, :, L].clone()
    _within_f16_ulp(vw.h, OO.rmsnorm(vw.x, model.norm_final, dims.rms_eps), "final RMSNorm")
    lg = g.logits.cpu().numpy()
    ref = OO.dense_gemm(model.lm_head, vw.h)
    compare_logits(lg, ref, g.tok.cpu().numpy(), f"LM head ({kind})")
    assert (g.pos.cpu().numpy() == pos + 1).all()
    # both layers: layer 1's stages from the GPU's layer-0 residual (layer 0 recomputes
    # bitwise the same values and re-appends the same entries)
    g.set(pos, tok)
    g.step()
    vw2 = _View(qd, g, dims, bsz)
    check_layer_stages(dims, kind, model.layers[1], x_l0, pos, vw2, g.kv[1], caches[1], slots)
    import torch
    assert torch.equal(g.kv[0].k[:, :, L], k0), "layer 0 re-appended different keys"


@pytest.mark.parametrize("bsz,kind", [(1, "f16"), (1, "q8_0"), (2, "f16"), (2, "q8_0"), (16, "f16"), (16, "q8_0"),
                                      (16, "fp8")])
def test_full_width_step_stagewise_batch_sizes(qd, bsz, kind):
    # the Qwen-shaped layer at the ends of the batch range: B = 1 (the matvec
    # engine), B = 2 (the first MFMA batch size) and B = 16 (the projections
    # stage rows 8..15 in a second pass), one layer, L = 300, every stage
    # against the oracle fed with the GPU's own input to that stage
    _stagewise_one_layer(qd, synth.QWEN_SHAPED, bsz, kind, 1103 + bsz)


@pytest.mark.parametrize("kind", ["f16", "q8_0", "f16k_q8v"])
def test_full_width_head_dim_64(qd, kind):
    # hidden 4096 with 64 query and 8 KV heads of 64: the QKV projection's
    # finish with two tiles per rotation pair (the whole head in one work-group
    # for a Q8_0 cache), B = 4, L = 300
    dims = synth.ModelDims(n_layers=1, hidden=4096, n_q_heads=64, n_kv_heads=8, head_dim=64, ffn=12288,
                           vocab=8192)
    _stagewise_one_layer(qd, dims, 4, kind, 1163)


def _stagewise_one_layer(qd, dims, bsz, kind, seed):
    from oracle import ops as OO
    L = 300
    slots = list(range(bsz))
    model, caches, tok = build(dims, seed, kind, bsz, L, 320, n_layers=1)
    pos = np.full(bsz, L)
    g = GpuStep(qd, model, caches, bsz, slots)
    g.set(pos, tok)
    g.step()
    vw = _View(qd, g, dims, bsz)
    x_emb = model.embed[tok].astype(np.float64)
    check_layer_stages(dims, kind, model.layers[0], x_emb, pos, vw, g.kv[0], caches[0], slots)
    _within_f16_ulp(vw.h, OO.rmsnorm(vw.x, model.norm_final, dims.rms_eps), "final RMSNorm")
    ref = OO.dense_gemm(model.lm_head, vw.h)
    compare_logits(g.logits.cpu().numpy(), ref, g.tok.cpu().numpy(), f"LM head (B={bsz}, {kind})")
    assert (g.pos.cpu().numpy() == pos + 1).all()


@pytest.mark.parametrize("kind", ["q8_0", "q8k_f16v", "f16k_q8v"])
def test_full_width_q8_append_at_capacity_edge(qd, kind):
    # With a Q8_0 part the QKV projection stages the new token's key and value
    # and the last run of the attention quantizes and stores them.  One
    # Qwen-shaped layer, B = 2: sequence 0 appends at the cache's last
    # position (cap - 1, the last token of the run's last tile), sequence 1
    # one past it.  Sequence 0 is checked stage by stage against the oracle;
    # sequence 1 raises the capacity flag and its slot keeps every byte.
    dims = synth.QWEN_SHAPED
    bsz, cap = 2, 320
    model, caches, tok = build(dims, 1611, kind, bsz, cap - 1, cap, n_layers=1)
    pos = np.array([cap - 1, cap])
    g = GpuStep(qd, model, caches, bsz, [0, 1])
    g.set(pos, tok)
    g.step()
    assert qd.qkdec_step_status(g.ws) == -5
    vw = _View(qd, g, dims, bsz)
    check_layer_stages(dims, kind, model.layers[0], model.embed[tok].astype(np.float64), pos, vw, g.kv[0],
                       caches[0], [0])
    got = g.kv[0].logical()
    for name, arr in vars(caches[0]).items():
        if arr is None:
            continue
        assert np.array_equal(getattr(got, name)[1].view(np.uint8), arr[1].view(np.uint8)), name
