#!/usr/bin/env python3
"""Throughput of one batched quantized decode step on one MI355X.

Workload (the headline configuration): a synthetic Qwen-shaped decoder (36
layers, hidden 4096, 32 query / 8 KV heads of 128, SwiGLU FFN 12288, vocab
151936), Q4_K weights, fp16 KV cache, B = 8 sequences with L = 2400 cached
tokens each.  A step = every layer (RMSNorm, QKV GEMM, RoPE + KV append,
split-K attention, O GEMM + residual, RMSNorm, gate/up GEMM + SwiGLU, down
GEMM + residual), final norm, LM head and argmax, with the token fed back and
the position advanced on the device; the step is replayed from a HIP graph.
Inputs (weights, caches) are drawn on the GPU and resident in HBM before the
timed region.  Extra points on the same line: L = 6900, and the Q8_0 cache.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints one JSON line.  value = aggregate decode tokens/s = B * K / time.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
NL, H, HQ, HKV, D, FFN, VOCAB = 36, 4096, 32, 8, 128, 12288, 151936


def q4k_bytes(n, k):
    return n * (k // 256) * 144


LAYER_Q4K = (q4k_bytes((HQ + 2 * HKV) * D, H) + q4k_bytes(H, HQ * D) + q4k_bytes(2 * FFN, H)
             + q4k_bytes(H, FFN))
W_BYTES = NL * LAYER_Q4K + VOCAB * H * 2 + (2 * NL + 1) * H * 4     # shared bytes read once per step
KV_BYTES_PER_TOKEN = {"f16": NL * HKV * D * 2 * 2, "q8_0": NL * HKV * D * 2 * 34 // 32}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_point(qd, sd, dims, dev_model, batch, length, kind, capacity, seed):
    import torch
    from quantized_decode_amd import KV_F16, KV_Q8_0, kv_layer
    g = sd.generator(seed)
    kvs, keep = [], []
    for _ in range(dims.n_layers):
        k, v, ks, vs = sd.kv_cache(g, kind, batch, dims.n_kv_heads, capacity, dims.head_dim, length)
        keep.append((k, v, ks, vs))
        kvs.append(kv_layer(KV_F16 if kind == "f16" else KV_Q8_0, dims.n_kv_heads, dims.head_dim, capacity, batch,
                            k, v, ks, vs))
    embed, lm_head, norm, layers = dev_model
    sm = qd.StepModel(dims, embed, lm_head, norm, layers, kvs)
    sm._keep = keep
    return sm


def time_point(qd, sm, batch, length, steps, warmup, vocab, seed):
    import torch
    slot = torch.arange(batch, dtype=torch.int32, device="cuda")
    pos = torch.full((batch,), length, dtype=torch.int32, device="cuda")
    tok = torch.randint(0, vocab, (batch,), dtype=torch.int32, device="cuda",
                        generator=torch.Generator(device="cuda").manual_seed(seed))
    ws = torch.zeros(qd.qkdec_step_workspace_size(sm, batch), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    plan = qd.Plan(sm, slot, pos, tok, batch, ws, logits=None, stream=stream)
    for _ in range(warmup):
        plan.launch(stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        plan.launch(stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1)
    status = qd.qkdec_step_status(ws)
    plan.destroy()
    assert status == 0, f"step reported status {status}"
    assert int(pos[0].item()) == length + warmup + steps
    return ms / steps, wall


def kernel_timing(qd, sd, dev_model, batch, length, seed):
    """Per-kernel launch durations with HIP events on the launching stream,
    using the step's own entry points and shapes (one step's worth)."""
    import torch
    embed, lm_head, norm, layers = dev_model
    g = sd.generator(seed)
    x16 = sd.f16_normal(g, (batch, H))
    o16 = sd.f16_normal(g, (batch, HQ * D))
    a32 = torch.randn((batch, FFN), device="cuda", generator=g) * 100
    yq = torch.empty((batch, (HQ + 2 * HKV) * D), dtype=torch.float32, device="cuda")
    yx = torch.zeros((batch, H), dtype=torch.float32, device="cuda")
    ya = torch.empty((batch, FFN), dtype=torch.float32, device="cuda")
    wsz = max(qd.qkdec_gemm_q4k_workspace_size((HQ + 2 * HKV) * D, H, batch),
              qd.qkdec_gemm_q4k_workspace_size(H, HQ * D, batch),
              qd.qkdec_gemm_q4k_swiglu_workspace_size(FFN, H, batch),
              qd.qkdec_gemm_q4k_workspace_size(H, FFN, batch))
    ws = torch.zeros(wsz, dtype=torch.uint8, device="cuda")
    calls = []
    for ly in layers:
        calls.append((lambda ly=ly: qd.qkdec_gemm_q4k(ly["w_qkv"], (HQ + 2 * HKV) * D, H, x16, batch, yq, workspace=ws),
                      q4k_bytes((HQ + 2 * HKV) * D, H)))
        calls.append((lambda ly=ly: qd.qkdec_gemm_q4k(ly["w_o"], H, HQ * D, o16, batch, yx, residual=yx, workspace=ws),
                      q4k_bytes(H, HQ * D)))
        calls.append((lambda ly=ly: qd.qkdec_gemm_q4k_swiglu(ly["w_gate_up"], FFN, H, x16, batch, ya, workspace=ws),
                      q4k_bytes(2 * FFN, H)))
        calls.append((lambda ly=ly: qd.qkdec_gemm_q4k_xf32(ly["w_down"], H, FFN, a32, batch, yx, residual=yx,
                                                             workspace=ws), q4k_bytes(H, FFN)))
    for fn, _ in calls[:8]:
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
    for (fn, _), (a, b) in zip(calls, ev):
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    gemm_ms = sum(a.elapsed_time(b) for a, b in ev)
    gemm = {"launches": len(calls), "total_ms": gemm_ms, "bytes": sum(by for _, by in calls)}

    # attention over the fp16 cache at this context (36 layers' worth of distinct caches would be
    # 2.8 GB; one layer's cache is re-used here, 8 launches, reported per launch)
    from quantized_decode_amd import KV_F16, kv_layer
    cap = (length + 31) // 32 * 32
    k, v, _, _ = sd.kv_cache(g, "f16", batch, HKV, cap, D, length)
    desc = kv_layer(KV_F16, HKV, D, cap, batch, k, v)
    q = sd.f16_normal(g, (batch, HQ, D))
    o = torch.empty((batch, HQ, D), dtype=torch.float16, device="cuda")
    slot = torch.arange(batch, dtype=torch.int32, device="cuda")
    nctx = torch.full((batch,), length, dtype=torch.int32, device="cuda")
    aws = torch.zeros(qd.qkdec_attn_workspace_size(batch, HQ, desc), dtype=torch.uint8, device="cuda")
    qd.qkdec_attn_decode(desc, slot, nctx, batch, q, HQ, D ** -0.5, o16=o, workspace=aws)
    torch.cuda.synchronize()
    aev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(8)]
    for a, b in aev:
        a.record()
        qd.qkdec_attn_decode(desc, slot, nctx, batch, q, HQ, D ** -0.5, o16=o, workspace=aws)
        b.record()
    torch.cuda.synchronize()
    attn_ms = sum(a.elapsed_time(b) for a, b in aev) / len(aev)
    attn = {"per_launch_ms": attn_ms, "bytes_per_launch": batch * length * HKV * D * 2 * 2}
    del k, v

    tok = torch.empty(batch, dtype=torch.int32, device="cuda")
    lws = torch.zeros(qd.qkdec_lm_head_workspace_size(VOCAB, batch), dtype=torch.uint8, device="cuda")
    qd.qkdec_lm_head_argmax(lm_head, VOCAB, H, x16, batch, tok, workspace=lws)
    torch.cuda.synchronize()
    lev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4)]
    for a, b in lev:
        a.record()
        qd.qkdec_lm_head_argmax(lm_head, VOCAB, H, x16, batch, tok, workspace=lws)
        b.record()
    torch.cuda.synchronize()
    lm = {"per_launch_ms": sum(a.elapsed_time(b) for a, b in lev) / len(lev), "bytes_per_launch": VOCAB * H * 2}
    return gemm, attn, lm


def cpu_baseline(dims, dev_model, batch, length, seed):
    """The fp64 oracle on the host, on a bounded sample: layer 0 of the step (its
    four Q4_K GEMMs for all sequences, RoPE, append and attention over `length`
    cached tokens) and 1/36 of the LM head rows; the step estimate is 36 times
    the sample."""
    import numpy as np
    import torch

    import synth
    from oracle import formats as OF
    from oracle import ops as OO
    from oracle import step as OS
    embed, lm_head, norm, layers = dev_model
    ly = {k: v.cpu().numpy() for k, v in layers[0].items()}
    rng = np.random.default_rng(seed)
    kv = synth.kv_cache_f16(rng, rng, batch, dims.n_kv_heads, length + 32, dims.head_dim, [length] * batch)
    rows = VOCAB // 36 // 16 * 16
    lm = lm_head[:rows].cpu().numpy()
    x = synth.f16_normal(rng, (batch, H)).astype(np.float64)
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = None
    t0 = time.perf_counter()
    h = OF.round_f16(OO.rmsnorm(x, ly["norm_attn"], dims.rms_eps))
    qkv = OO.q4k_gemm(ly["w_qkv"], dims.qkv_rows, H, h)
    o = np.empty((batch, HQ * D))
    for b in range(batch):
        q = OO.rope(qkv[b, :HQ * D].reshape(HQ, D), length, dims.rope_base)
        k = OO.rope(qkv[b, HQ * D:(HQ + HKV) * D].reshape(HKV, D), length, dims.rope_base)
        OS.kv_append(kv, "f16", b, length, k, qkv[b, (HQ + HKV) * D:].reshape(HKV, D))
        kd, vd = OS.kv_read(kv, "f16", b, length + 1)
        o[b] = OO.attention(OF.round_f16(q), kd, vd, D ** -0.5).reshape(-1)
    x = x + OO.q4k_gemm(ly["w_o"], H, HQ * D, OF.round_f16(o))
    h2 = OF.round_f16(OO.rmsnorm(x, ly["norm_ffn"], dims.rms_eps))
    gu = OO.q4k_gemm(ly["w_gate_up"], 2 * FFN, H, h2)
    a = OF.round_f16_blocked(OO.swiglu(gu[:, :FFN], gu[:, FFN:]))
    x = x + OO.q4k_gemm(ly["w_down"], H, FFN, a)
    OO.dense_gemm(lm, OF.round_f16(OO.rmsnorm(x, np.ones(H), dims.rms_eps)))
    sample_s = time.perf_counter() - t0
    step_s = 36 * sample_s
    return {"value": batch / step_s, "unit": "tok/s", "cores": threads if threads else 1, "kind": "oracle",
            "sample": f"layer 0 of 36 (4 Q4_K GEMMs, RoPE, append, attention over {length} tokens, B={batch}) "
                      f"+ {rows} of {VOCAB} LM-head rows; fp64 numpy; step estimated as 36x the "
                      f"{sample_s:.1f} s sample", "sample_seconds": sample_s,
            "host_cpus": os.cpu_count()}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=8)
    ap.add_argument("--context", type=int, default=2400)
    ap.add_argument("--kv", choices=["f16", "q8_0"], default="f16")
    ap.add_argument("--points", choices=["all", "main"], default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; multi-GPU sharding is a design note, "
                                   "not implemented", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import quantized_decode_amd as qd
    import synth
    import synth.device as sd
    qd.load_library()
    dims = synth.QWEN_SHAPED
    log("drawing the synthetic model on the GPU")
    dev_model = sd.model(dims, 1003)
    torch.cuda.synchronize()

    points = [(args.batch, args.context, args.kv)]
    if args.points == "all":
        for p in [(8, 2400, "f16"), (8, 6900, "f16"), (8, 2400, "q8_0"), (8, 6900, "q8_0")]:
            if p not in points:
                points.append(p)
    results = []
    for i, (bsz, L, kind) in enumerate(points):
        cap = (L + args.warmup + args.steps + 2 + 31) // 32 * 32
        log(f"point B={bsz} L={L} kv={kind}: building caches (capacity {cap})")
        sm = build_point(qd, sd, dims, dev_model, bsz, L, kind, cap, 2000 + i)
        torch.cuda.synchronize()
        ms, wall = time_point(qd, sm, bsz, L, args.steps, args.warmup, dims.vocab, 3000 + i)
        l_mean = L + args.warmup + (args.steps - 1) / 2
        step_bytes = W_BYTES + bsz * l_mean * KV_BYTES_PER_TOKEN[kind]
        gbps = step_bytes / (ms * 1e-3) / 1e9
        results.append({"batch": bsz, "context": L, "kv": kind, "ms_per_step": ms, "tok_per_s": bsz / (ms * 1e-3),
                        "bytes_per_step": step_bytes, "achieved_GBps": gbps, "frac_of_8TBps": gbps / PEAK_HBM_GBPS,
                        "wall_s": wall})
        log(f"  {ms:.3f} ms/step, {bsz / (ms * 1e-3):.1f} tok/s, {gbps:.0f} GB/s on the byte model")
        del sm
        torch.cuda.empty_cache()

    main_pt = results[0]
    log("per-kernel timing (HIP events on the launching stream)")
    gemm, attn, lm = kernel_timing(qd, sd, dev_model, args.batch, args.context, 4000)
    gemm_avg_ms = gemm["total_ms"] / gemm["launches"]
    gemm_achieved = gemm["bytes"] / gemm["launches"] / (gemm_avg_ms * 1e-3) / 1e9
    roofline = {"kernel": "gemm_q4k (QKV, O, gate/up+SwiGLU, down: 144 launches per step)",
                "bound": "hbm", "achieved": gemm_achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": gemm_achieved / PEAK_HBM_GBPS, "traffic": None,
                "avg_launch_ms": gemm_avg_ms, "algorithmic_bytes_per_launch": gemm["bytes"] / gemm["launches"],
                "step_share_ms": gemm["total_ms"]}
    kernels = {"attn_decode": {"per_launch_ms": attn["per_launch_ms"],
                               "GBps": attn["bytes_per_launch"] / (attn["per_launch_ms"] * 1e-3) / 1e9},
               "lm_head_argmax": {"per_launch_ms": lm["per_launch_ms"],
                                  "GBps": lm["bytes_per_launch"] / (lm["per_launch_ms"] * 1e-3) / 1e9}}

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: fp64 oracle on a bounded sample")
        cpu = cpu_baseline(dims, dev_model, args.batch, args.context, 5000)

    out = {
        "metric": "aggregate decode tok/s at B=8, L=2.4k/6.9k; achieved HBM GB/s vs peak",
        "value": main_pt["tok_per_s"], "unit": "tok/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": main_pt["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"batched decode step, Qwen-shaped synthetic decoder (36 layers, hidden 4096, "
                               f"32/8 heads x 128, FFN 12288, vocab 151936), Q4_K weights, {main_pt['kv']} KV, "
                               f"B={main_pt['batch']}, L={main_pt['context']}",
                   "batch": main_pt["batch"], "context": main_pt["context"], "kv": main_pt["kv"]},
        "achieved_GBps": main_pt["achieved_GBps"], "frac_of_8TBps": main_pt["frac_of_8TBps"],
        "roofline": roofline, "kernels": kernels, "points": results, "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
