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
timed region.  Extra points on the same line ("points"): L = 6900; the Q8_0
cache and the two mixed caches (Q8_0 keys with fp16 values and the reverse);
the 8-bit float (E4M3) cache at L = 2400 and 6900; B = 1 at L = 2400; B = 16 at
L = 3400 (fp16 and Q8_0); Q8_0 at L = 8192 and 19000.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
    python bench.py --sweep [--sweep-kv f16,q8_0,fp8] [--sweep-batches 1,2,4,8,16]
                    [--sweep-contexts 32,2400,4700,6900,16000,32000]

--sweep measures the step over batch sizes x contexts x cache kinds instead
(one JSON line per point, then a summary line): the measured speedup of B
sequences over one at the same context, next to the byte model's prediction
(P2 "Where the private read overtakes the shared one"), the bandwidth-bound
ceiling at the box's measured read rate (P3 "What the sagging ceiling costs in
tokens per second") and the context per sequence the 0.85-of-memory budget
holds on this GPU (P1 "Where it stops, and the argument I got wrong in May").

Prints one JSON line.  value = aggregate decode tokens/s = B * K / time of the
K timed replays (mean); per-replay p10/p50/p90 are in "points".  "roofline" is
for the kernel that takes the largest share of the step, timed with HIP events
over the 36 layers' own weights (or caches); "cpu_baseline" is the fp64 oracle
on a bounded sample of the same step on the host cores.
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


def _byte_model():
    from quantized_decode_amd import planner as P
    w = P.model_weight_bytes(NL, H, HQ, HKV, D, FFN, VOCAB)          # shared bytes read once per step
    k = {kind: P.kv_bytes_per_token(NL, HKV, D, kind) for kind in ("f16", "q8_0", "q8k_f16v", "f16k_q8v", "fp8")}
    return w, k


W_BYTES, KV_BYTES_PER_TOKEN = _byte_model()


# HBM bytes per launch counted by rocprofv3 (FETCH_SIZE and WRITE_SIZE runs,
# calibrated against a plain 1 GiB copy) live in profiles/counted_traffic.json,
# written by `bench.py --traffic-from ...` together with the build id of the
# library the counters ran on.  They are used only while the loaded library
# has that build id: once a kernel source changes, the figure is stale and
# the bench reports traffic as null.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "counted_traffic.json")

# the kernels (demangled-name prefixes) behind each kernel kind of the bench,
# by KV cache kind where the kernel depends on it
_ATTN_FMT = {"f16": (0, 0), "q8_0": (1, 1), "q8k_f16v": (1, 0), "f16k_q8v": (0, 1), "fp8": (2, 2)}


def kind_kernels(name, kv):
    if name.startswith("attention (split + merge)"):
        kf, vf = _ATTN_FMT[kv]
        return [f"void qk::attn_split_kernel<128, {kf}, {vf}, false, false>", "qk::attn_combine_kernel"]
    if name == "lm_head_argmax":
        return ["qk::lm_head_kernel", "qk::lm_argmax_reduce_kernel"]
    return None


def compute_dtype(kv):
    """Arithmetic type of the path: every contraction (Q4_K GEMMs, attention,
    LM head) runs as fp16 MFMA with fp32 accumulation; the weights (Q4_K) and
    the cache (fp16, Q8_0, E4M3) are storage formats decoded exactly to fp16
    in the kernels, so the arithmetic is f16 whatever `kv` is."""
    assert kv in _ATTN_FMT
    return "f16"


def counted_traffic(qd, name, batch, context, kv):
    """Counted HBM bytes per launch of kernel kind `name` at this point, or
    None when no count was taken on this build of the library."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("build_id") != qd.qkdec_build_id():
        return None
    cfg = rec.get("config", {})
    if (cfg.get("batch"), cfg.get("context"), cfg.get("kv")) != (batch, context, kv):
        return None
    names = kind_kernels(name, kv)
    if not names:
        return None
    total = 0.0
    for prefix in names:
        hits = [v for k, v in rec["kernels"].items() if k.startswith(prefix)]
        if len(hits) != 1:
            return None
        total += hits[0]["fetched_bytes"] + hits[0]["written_bytes"]
    return int(round(total))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_point(qd, sd, dims, dev_model, batch, length, kind, capacity, seed):
    import torch
    from quantized_decode_amd import KV_KINDS, kv_layer
    g = sd.generator(seed)
    kvs, keep = [], []
    for _ in range(dims.n_layers):
        k, v, ks, vs = sd.kv_cache(g, kind, batch, dims.n_kv_heads, capacity, dims.head_dim, length)
        keep.append((k, v, ks, vs))
        kvs.append(kv_layer(KV_KINDS[kind], dims.n_kv_heads, dims.head_dim, capacity, batch, k, v, ks, vs))
    embed, lm_head, norm, layers = dev_model
    sm = qd.StepModel(dims, embed, lm_head, norm, layers, kvs)
    sm._keep = keep
    return sm


def time_point(qd, sm, batch, length, steps, warmup, vocab, seed):
    """Replay the captured step; returns per-replay durations (ms) and the wall time."""
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
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        plan.launch(stream=stream)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    status = qd.qkdec_step_status(ws)
    plan.destroy()
    assert status == 0, f"step reported status {status}"
    got = pos.cpu().tolist()
    want = length + warmup + steps
    assert all(x == want for x in got), f"step: positions {got}, expected {want} (one per replay)"
    return per, wall


def time_paged_step(qd, sd, dims, dev_model, batch, length, kind, steps, warmup, seed, page_tokens=256):
    """The same step over paged pools (qkdec_step_paged): pages of
    `page_tokens`, each sequence's pages scattered by a random permutation of
    the pool; one step captured in a HIP graph and replayed like the arena
    step.  Returns per-replay durations (ms)."""
    import torch
    from quantized_decode_amd import KV_KINDS, kv_layer
    from quantized_decode_amd import planner as PL
    P = page_tokens
    max_pages = (PL.slot_capacity(length, warmup + steps + 2) + P - 1) // P
    n_pages = batch * max_pages
    g = sd.generator(seed)
    pools, keep = [], []
    for _ in range(dims.n_layers):
        k, v, ks, vs = sd.kv_cache(g, kind, n_pages, dims.n_kv_heads, P, dims.head_dim, P)
        keep.append((k, v, ks, vs))
        pools.append(kv_layer(KV_KINDS[kind], dims.n_kv_heads, dims.head_dim, P, n_pages, k, v, ks, vs))
    table = torch.randperm(n_pages, device="cuda", generator=g).to(torch.int32).reshape(batch, max_pages).contiguous()
    embed, lm_head, norm, layers = dev_model
    sm = qd.StepModel(dims, embed, lm_head, norm, layers, pools)
    pos = torch.full((batch,), length, dtype=torch.int32, device="cuda")
    tok = torch.randint(0, dims.vocab, (batch,), dtype=torch.int32, device="cuda", generator=g)
    ws = torch.zeros(qd.qkdec_step_paged_workspace_size(sm, batch, max_pages), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    run = lambda: qd.qkdec_step_paged(sm, table, max_pages, pos, tok, batch, ws, stream=stream)
    # the pools, table, positions and workspace were written on the default
    # stream: they must be complete before the side stream reads them
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        run()                                   # one eager step (pos advances)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        run()
    per = []
    with torch.cuda.stream(stream):
        for i in range(warmup + steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            graph.replay()
            b.record(stream)
            torch.cuda.synchronize()
            if i >= warmup:
                per.append(a.elapsed_time(b))
    status = qd.qkdec_step_status(ws)
    assert status == 0, f"paged step reported status {status}"
    got = pos.cpu().tolist()
    want = length + 1 + warmup + steps
    assert all(x == want for x in got), f"paged step: positions {got}, expected {want}"
    del graph
    return per


def _timed(calls, stream, replays=5):
    """Average duration (ms) of one call of `calls`: the calls are captured in
    order into one HIP graph on `stream` and replayed between HIP events on
    that stream, so host launch gaps are not counted; median over `replays`."""
    import torch
    torch.cuda.synchronize()                         # inputs and workspaces were made on the default stream
    with torch.cuda.stream(stream):
        calls[0]()                                   # first launch of the kernel: not timed
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for fn in calls:
            fn()
    graph.replay()
    torch.cuda.synchronize()
    per = []
    with torch.cuda.stream(stream):          # replay() launches on the current stream
        for _ in range(replays):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            graph.replay()
            b.record(stream)
            torch.cuda.synchronize()
            per.append(a.elapsed_time(b) / len(calls))
    del graph
    return sorted(per)[len(per) // 2]


def kernel_timing(qd, sd, dev_model, sm, batch, length, seed):
    """Per-launch durations of the step's kernels: each kind's 36 launches over
    the 36 layers' own weights and caches (so no launch finds its data in the
    last-level cache), captured in a HIP graph and timed with HIP events on the
    stream they are launched on."""
    import torch
    embed, lm_head, norm, layers = dev_model
    g = sd.generator(seed)
    stream = torch.cuda.Stream()
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
    kinds = {
        "gemm_qkv": (lambda ly: qd.qkdec_gemm_q4k(ly["w_qkv"], (HQ + 2 * HKV) * D, H, x16, batch, yq, workspace=ws,
                                                  stream=stream),
                     q4k_bytes((HQ + 2 * HKV) * D, H) + batch * H * 2 + batch * (HQ + 2 * HKV) * D * 4),
        "gemm_o": (lambda ly: qd.qkdec_gemm_q4k(ly["w_o"], H, HQ * D, o16, batch, yx, residual=yx, workspace=ws,
                                                stream=stream),
                   q4k_bytes(H, HQ * D) + batch * HQ * D * 2 + 2 * batch * H * 4),
        "gemm_gate_up_swiglu": (lambda ly: qd.qkdec_gemm_q4k_swiglu(ly["w_gate_up"], FFN, H, x16, batch, ya,
                                                                    workspace=ws, stream=stream),
                                q4k_bytes(2 * FFN, H) + batch * H * 2 + batch * FFN * 4),
        "gemm_down": (lambda ly: qd.qkdec_gemm_q4k_xf32(ly["w_down"], H, FFN, a32, batch, yx, residual=yx,
                                                        workspace=ws, stream=stream),
                      q4k_bytes(H, FFN) + batch * FFN * 4 + 2 * batch * H * 4),
    }
    out = {}
    notes = {
        "gemm_qkv": "ABI entry, fp16 activations, two tiles per work-group; the step runs this shape with the "
                    "RMSNorm fused and the RoPE / fp16-append finish (one head's tile pair per work-group)",
        "gemm_o": "same kernel as the step's O projection",
        "gemm_gate_up_swiglu": "ABI entry, fp16 activations; the step runs the same multi-item kernel with the "
                               "RMSNorm fused",
        "gemm_down": "same kernel as the step's down projection",
    }
    for name, (fn, nbytes) in kinds.items():
        ms = _timed([lambda ly=ly: fn(ly) for ly in layers], stream)
        out[name] = {"launches_per_step": len(layers), "avg_ms": ms, "bytes_per_launch": nbytes,
                     "note": notes[name]}

    # attention over the 36 per-layer caches of the timed workload, n_ctx = L
    q = sd.f16_normal(g, (batch, HQ, D))
    o = torch.empty((batch, HQ, D), dtype=torch.float16, device="cuda")
    slot = torch.arange(batch, dtype=torch.int32, device="cuda")
    nctx = torch.full((batch,), length, dtype=torch.int32, device="cuda")
    kvs = sm.kv_layers
    aws = torch.zeros(qd.qkdec_attn_workspace_size(batch, HQ, kvs[0]), dtype=torch.uint8, device="cuda")
    fa = lambda kv: qd.qkdec_attn_decode(kv, slot, nctx, batch, q, HQ, D ** -0.5, o16=o, workspace=aws,
                                         stream=stream)
    ms = _timed([lambda kv=kv: fa(kv) for kv in kvs], stream)
    kind_of = {v: k for k, v in qd.KV_KINDS.items()}
    kv_bytes = KV_BYTES_PER_TOKEN[kind_of[kvs[0].type]] / NL
    out["attention (split + merge)"] = {"launches_per_step": len(kvs), "avg_ms": ms,
                                        "bytes_per_launch": batch * length * kv_bytes,
                                        "note": "same kernels as the step's attention (n_ctx = L here, L + 1 "
                                                "in the step)"}

    # the same attention over paged pools (pages of 256 tokens, every
    # sequence's pages scattered by a random permutation of the pool); not part
    # of the step (launches_per_step 0), timed for the comparison
    P = 256
    npp = (length + P - 1) // P
    kind = kind_of[kvs[0].type]
    pools, keep = [], []
    for _ in range(len(kvs)):
        k, v, ks, vs = sd.kv_cache(g, kind, batch * npp, HKV, P, D, P)
        keep.append((k, v, ks, vs))
        pools.append(qd.kv_layer(kvs[0].type, HKV, D, P, batch * npp, k, v, ks, vs))
    table = torch.randperm(batch * npp, device="cuda", generator=g).to(torch.int32).reshape(batch, npp).contiguous()
    pws = torch.zeros(qd.qkdec_attn_paged_workspace_size(batch, HQ, pools[0], npp), dtype=torch.uint8, device="cuda")
    fp = lambda kv: qd.qkdec_attn_decode_paged(kv, table, npp, nctx, batch, q, HQ, D ** -0.5, o16=o, workspace=pws,
                                               stream=stream)
    ms = _timed([lambda kv=kv: fp(kv) for kv in pools], stream)
    out[f"attention, paged pool (pages of {P})"] = {
        "launches_per_step": 0, "avg_ms": ms, "bytes_per_launch": batch * length * kv_bytes,
        "note": "qkdec_attn_decode_paged over 36 pools of the same size; not in the step"}
    del pools, keep

    tok = torch.empty(batch, dtype=torch.int32, device="cuda")
    lws = torch.zeros(qd.qkdec_lm_head_workspace_size(VOCAB, batch), dtype=torch.uint8, device="cuda")
    flm = lambda: qd.qkdec_lm_head_argmax(lm_head, VOCAB, H, x16, batch, tok, workspace=lws, stream=stream)
    ms = _timed([flm] * 4, stream)
    out["lm_head_argmax"] = {"launches_per_step": 1, "avg_ms": ms, "bytes_per_launch": VOCAB * H * 2}
    for v in out.values():
        v["GBps"] = v["bytes_per_launch"] / (v["avg_ms"] * 1e-3) / 1e9
        v["ms_per_step"] = v["avg_ms"] * v["launches_per_step"]
    return out


def gemm_pass(qd, sd, dev_model, batches, seed, replays=5):
    """The standalone batched Q4_K GEMM workload: one pass = the four
    projections of all 36 layers (QKV 6144x4096, O 4096x4096, gate|up
    24576x4096, down 4096x12288), each a qkdec_gemm_q4k call with fp16 N(0,1)
    activations of B rows and fp32 outputs, over every layer's own weights
    (3.9 GB, far beyond the last-level cache).  Captured in one HIP graph and
    replayed between HIP events on the launching stream."""
    import torch
    embed, lm_head, norm, layers = dev_model
    g = sd.generator(seed)
    shapes = [("w_qkv", (HQ + 2 * HKV) * D, H), ("w_o", H, HQ * D), ("w_gate_up", 2 * FFN, H), ("w_down", H, FFN)]
    wbytes = sum(q4k_bytes(n, k) for _, n, k in shapes) * len(layers)
    stream = torch.cuda.Stream()
    rows = []
    for bsz in batches:
        xs = {k: sd.f16_normal(g, (bsz, k)) for k in {k for _, _, k in shapes}}
        ys = {n: torch.empty((bsz, n), dtype=torch.float32, device="cuda") for n in {n for _, n, _ in shapes}}
        wsz = max(qd.qkdec_gemm_q4k_workspace_size(n, k, bsz) for _, n, k in shapes)
        ws = torch.zeros(wsz, dtype=torch.uint8, device="cuda")
        engines = [("mfma", qd.GEMM_MFMA)] + ([("matvec", qd.GEMM_MATVEC)] if bsz <= qd.MATVEC_MAX_B else [])
        nbytes = wbytes + len(layers) * sum(bsz * (2 * k + 4 * n) for _, n, k in shapes)
        for ename, eng in engines:
            calls = [lambda ly=ly, nm=nm, n=n, k=k, eng=eng: qd.qkdec_gemm_q4k_engine(
                         ly[nm], n, k, xs[k], bsz, ys[n], eng, workspace=ws, stream=stream)
                     for ly in layers for nm, n, k in shapes]
            ms = _timed(calls, stream, replays=replays) * len(calls)
            rows.append({"batch": bsz, "engine": ename, "ms_per_pass": ms, "bytes_per_pass": nbytes,
                         "GBps": nbytes / (ms * 1e-3) / 1e9,
                         "frac_of_8TBps": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                         "weight_GBps": wbytes / (ms * 1e-3) / 1e9})
            log(f"  GEMM pass B={bsz} {ename}: {ms:.3f} ms, {rows[-1]['GBps']:.0f} GB/s")
        del xs, ys, ws
    # the largest batch at which the matvec pass is faster than the MFMA pass
    best = {}
    for r in rows:
        best.setdefault(r["batch"], {})[r["engine"]] = r["ms_per_pass"]
    wins = [bb for bb, e in sorted(best.items()) if "matvec" in e and e["matvec"] < e["mfma"]]
    crossover = max(wins) if wins else 0
    return {"workload": "36 layers x {QKV 6144x4096, O 4096x4096, gate|up 24576x4096, down 4096x12288} Q4_K, "
                        "fp16 activations, fp32 out (qkdec_gemm_q4k_engine, MFMA tiles and vector-ALU matvec)",
            "weight_bytes_per_pass": wbytes, "matvec_faster_up_to_batch": crossover,
            "library_auto_max_batch": qd.MATVEC_AUTO_MAX_B, "points": rows}


def attention_pass(qd, sd, batch, contexts, ragged_seed, seed, kind="f16", replays=5):
    """The standalone flash-decode workload: one pass = qkdec_attn_decode over
    36 per-layer caches (32 query / 8 KV heads of 128, fp16 q, K, V N(0,1),
    scale 1/sqrt(128)), B sequences of L cached tokens each, or of ragged
    lengths uniform in 512..8192 (seeded); graph-timed like gemm_pass."""
    import numpy as np
    import torch
    from quantized_decode_amd import KV_KINDS, kv_layer
    g = sd.generator(seed)
    stream = torch.cuda.Stream()
    kvb = KV_BYTES_PER_TOKEN[kind] / NL
    rows = []
    cases = [("L=%d" % L, [L] * batch) for L in contexts]
    if ragged_seed is not None:
        lens = np.random.default_rng(ragged_seed).integers(512, 8193, size=batch)
        cases.append(("ragged U{512..8192}", [int(x) for x in lens]))
    for label, lens in cases:
        cap = (max(lens) + 31) // 32 * 32
        kvs, keep = [], []
        for _ in range(NL):
            k, v, ks, vs = sd.kv_cache(g, kind, batch, HKV, cap, D, cap)
            keep.append((k, v, ks, vs))
            kvs.append(kv_layer(KV_KINDS[kind], HKV, D, cap, batch, k, v, ks, vs))
        q = sd.f16_normal(g, (batch, HQ, D))
        o = torch.empty((batch, HQ, D), dtype=torch.float16, device="cuda")
        slot = torch.arange(batch, dtype=torch.int32, device="cuda")
        nctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
        aws = torch.zeros(qd.qkdec_attn_workspace_size(batch, HQ, kvs[0]), dtype=torch.uint8, device="cuda")
        calls = [lambda kv=kv: qd.qkdec_attn_decode(kv, slot, nctx, batch, q, HQ, D ** -0.5, o16=o, workspace=aws,
                                                    stream=stream) for kv in kvs]
        ms = _timed(calls, stream, replays=replays) * len(calls)
        nbytes = sum(lens) * kvb * NL
        rows.append({"case": label, "batch": batch, "lengths": lens, "ms_per_pass": ms, "bytes_per_pass": nbytes,
                     "GBps": nbytes / (ms * 1e-3) / 1e9, "frac_of_8TBps": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS})
        log(f"  attention pass {label}: {ms:.3f} ms, {rows[-1]['GBps']:.0f} GB/s")
        del kvs, keep, aws
        torch.cuda.empty_cache()
    return {"workload": f"36 layers x qkdec_attn_decode, 32/8 heads x 128, {kind} KV, B={batch}", "points": rows}


def prefill_point(qd, sd, dims, dev_model, n_prompt, seed, kind="f16"):
    """Prompt ingestion (qkdec_prefill): n_prompt tokens into an empty slot of
    the Qwen-shaped model (all 36 layers, keys and values appended, the first
    generated token taken after the last prompt token); one warm-up call, then
    the median of three calls timed with HIP events on the launching stream.
    weight_bytes_read: the Q4_K weights once per pass of the layers."""
    import torch
    from quantized_decode_amd import KV_KINDS, kv_layer
    g = sd.generator(seed)
    cap = (n_prompt + 31) // 32 * 32
    kvs, keep = [], []
    for _ in range(dims.n_layers):
        k, v, ks, vs = sd.kv_cache(g, kind, 1, dims.n_kv_heads, cap, dims.head_dim, 0)
        keep.append((k, v, ks, vs))
        kvs.append(kv_layer(KV_KINDS[kind], dims.n_kv_heads, dims.head_dim, cap, 1, k, v, ks, vs))
    embed, lm_head, norm, layers = dev_model
    sm = qd.StepModel(dims, embed, lm_head, norm, layers, kvs)
    prompt = torch.randint(0, dims.vocab, (n_prompt,), dtype=torch.int32, device="cuda", generator=g)
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(qd.qkdec_prefill_workspace_size(sm), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    times = []
    for i in range(4):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        qd.qkdec_prefill(sm, 0, 0, prompt, n_prompt, tok, ws, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        if i:
            times.append(a.elapsed_time(b))
    ms = sorted(times)[1]
    wbytes = W_BYTES * ((n_prompt + 2047) // 2048)
    del kvs, keep
    return {"prompt_tokens": n_prompt, "kv": kind, "ms": ms, "tok_per_s": n_prompt / (ms * 1e-3),
            "weight_bytes_read": wbytes, "note": "passes of up to 2048 prompt tokens through the layers: MFMA "
                                                  "projections over 64-row tiles, flash attention over the cache "
                                                  "(64 query columns per work-group, causal masks); LM head for "
                                                  "the last token"}


def record_traffic(qd, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mb, batch, context, kv, command):
    """Write profiles/counted_traffic.json from four rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE of the bench, and of `--copy-probe-mb copy_mb`
    for the calibration), stamped with the loaded library's build id."""
    import csv
    import glob
    import re
    import subprocess

    def load(d):
        paths = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if len(paths) != 1:
            raise SystemExit(f"expected one counter CSV under {d}, found {paths}")
        agg = {}
        with open(paths[0]) as fh:
            for r in csv.DictReader(fh):
                agg.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        names = list(agg)
        out = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True).stdout.split("\n")

        def readable(nm, dm):
            # symbols whose parameters c++filt cannot read (_Float16, "DF16_")
            # come back mangled: keep their qualified name
            m = re.match(r"_ZN2qk(\d+)", dm or nm)
            if m:
                n = int(m.group(1))
                return "qk::" + (dm or nm)[m.end():m.end() + n]
            return dm or nm
        return {readable(nm, dm): sum(v) / len(v) for nm, dm, v in zip(names, out, agg.values())}

    def copy_kib(d):
        vals = [v for k, v in load(d).items() if "copyBuffer" in k]
        if not vals:
            raise SystemExit(f"no copy kernel in {d}")
        return max(vals)

    nbytes = copy_mb << 20
    f_cal = nbytes / (copy_kib(copy_fetch_dir) * 1024)
    w_cal = nbytes / (copy_kib(copy_write_dir) * 1024)
    fetch, write = load(fetch_dir), load(write_dir)
    kernels = {}
    for name, kib in fetch.items():
        if not name.startswith(("qk::", "void qk::")):
            continue
        kernels[name] = {"fetched_bytes": kib * 1024 * f_cal, "written_bytes": write.get(name, 0.0) * 1024 * w_cal,
                         "fetch_size_kib": kib, "write_size_kib": write.get(name, 0.0)}
    rec = {"build_id": qd.qkdec_build_id(), "config": {"batch": batch, "context": context, "kv": kv},
           "calibration": {"copy_bytes": nbytes, "fetched_per_fetch_size_byte": f_cal,
                           "written_per_write_size_byte": w_cal},
           "command": command, "kernels": kernels}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
    print(json.dumps({"wrote": TRAFFIC_FILE, "build_id": rec["build_id"], "kernels": len(kernels),
                      "calibration": rec["calibration"]}))


def read_ceiling(gib=4):
    """The box's practical streaming-read rate: a device-wide sum over `gib`
    GiB (torch's reduction kernel, not part of the decode path), best of 3."""
    import torch
    n = gib << 30
    buf = torch.ones(n // 8, dtype=torch.int64, device="cuda")
    buf.sum()
    best = None
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        buf.sum()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del buf
    torch.cuda.empty_cache()
    return {"bytes": n, "ms": best, "GBps": n / (best * 1e-3) / 1e9, "kernel": "torch int64 sum"}


def clocks():
    """Current shader and memory clocks as rocm-smi reports them (None if it
    is not available)."""
    import subprocess
    try:
        out = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=30)
        card = next(iter(json.loads(out.stdout).values()))
        return {k: v for k, v in card.items() if "sclk" in k or "mclk" in k or "fclk" in k}
    except Exception:
        return None


def cpu_baseline(dims, dev_model, batch, length, seed, min_seconds=10.0):
    """The fp64 oracle on the host, on a bounded sample of the step: whole
    layers (four Q4_K GEMMs for all sequences, RoPE, KV append and attention
    over `length` cached tokens) until at least `min_seconds` of work, plus the
    same fraction of the LM head rows; the step estimate scales the sample by
    36 / (layers done)."""
    import numpy as np

    import synth
    from oracle import formats as OF
    from oracle import ops as OO
    from oracle import step as OS
    embed, lm_head, norm, layers = dev_model
    rng = np.random.default_rng(seed)
    kv = synth.kv_cache_f16(rng, rng, batch, dims.n_kv_heads, length + 32, dims.head_dim, [length] * batch)
    x = synth.f16_normal(rng, (batch, H)).astype(np.float64)
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = None
    elapsed, done = 0.0, 0
    while done < len(layers) and elapsed < min_seconds:
        ly = {k: v.cpu().numpy() for k, v in layers[done].items()}
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
        elapsed += time.perf_counter() - t0
        done += 1
    rows = VOCAB * done // NL // 16 * 16
    lm = lm_head[:rows].cpu().numpy()
    t0 = time.perf_counter()
    OO.dense_gemm(lm, OF.round_f16(OO.rmsnorm(x, np.ones(H), dims.rms_eps)))
    elapsed += time.perf_counter() - t0
    step_s = elapsed * NL / done
    return {"value": batch / step_s, "unit": "tok/s", "cores": threads if threads else 1, "kind": "oracle",
            "sample": f"{done} of {NL} layers (4 Q4_K GEMMs, RoPE, KV append, attention over {length} tokens, "
                      f"B={batch}) + {rows} of {VOCAB} LM-head rows, fp64 numpy; step = {NL}/{done} x the "
                      f"{elapsed:.1f} s sample",
            "sample_seconds": elapsed, "host_cpus": os.cpu_count()}


def sweep(args, qd, sd, dims, dev_model):
    """Step time over batch x context x cache kind (graph replays, inputs
    resident), with the planner's predictions beside each point."""
    import torch
    from quantized_decode_amd import planner as P
    kinds = args.sweep_kv.split(",")
    batches = [int(x) for x in args.sweep_batches.split(",")]
    contexts = [int(x) for x in args.sweep_contexts.split(",")]
    vram = torch.cuda.get_device_properties(0).total_memory
    log("streaming-read ceiling (4 GiB)")
    ceiling = read_ceiling()
    bw = ceiling["GBps"] * 1e9
    rows = []
    i = 0
    for kind in kinds:
        k = P.kv_bytes_per_token(dims.n_layers, dims.n_kv_heads, dims.head_dim, kind)
        plan = P.plan_capacity(vram, W_BYTES, k)
        for L in contexts:
            one = None
            for bsz in batches:
                i += 1
                cap = P.slot_capacity(L, args.warmup + args.steps + 2)
                if not plan.fits([cap] * bsz):
                    log(f"B={bsz} L={L} kv={kind}: over the 0.85 budget, skipped")
                    continue
                sm = build_point(qd, sd, dims, dev_model, bsz, L, kind, cap, 6000 + i)
                torch.cuda.synchronize()
                per, _ = time_point(qd, sm, bsz, L, args.steps, args.warmup, dims.vocab, 7000 + i)
                del sm
                torch.cuda.empty_cache()
                ms = sum(per) / len(per)
                tps = bsz / (ms * 1e-3)
                if bsz == 1:
                    one = tps
                l_mean = L + args.warmup + (args.steps - 1) / 2
                by = P.step_bytes(W_BYTES, [l_mean] * bsz, k)
                row = {"kv": kind, "batch": bsz, "context": L, "ms_per_step": ms, "tok_per_s": tps,
                       "bytes_per_step": by, "achieved_GBps": by / (ms * 1e-3) / 1e9,
                       "frac_of_8TBps": by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                       "speedup_vs_b1": tps / one if one else None,
                       "speedup_model": P.speedup(bsz, l_mean, W_BYTES, k),
                       "ceiling_tok_s_at_read_rate": P.ceiling_tok_s(bw, W_BYTES, bsz, l_mean, k),
                       "kv_traffic_bytes": P.kv_traffic_bytes([l_mean] * bsz, k),
                       "context_per_seq_at_085": plan.context_per_sequence(bsz)}
                rows.append(row)
                print(json.dumps(row), flush=True)
                log(f"B={bsz} L={L} kv={kind}: {ms:.3f} ms, {tps:.1f} tok/s, speedup "
                    f"{row['speedup_vs_b1'] or 0:.2f} (model {row['speedup_model']:.2f})")
    summary = {"sweep": "decode step, Qwen-shaped synthetic decoder, Q4_K weights", "steps": args.steps,
               "warmup": args.warmup, "vram_bytes": vram, "weight_bytes": W_BYTES, "read_ceiling": ceiling,
               "crossover_b8": {kind: P.crossover_context(W_BYTES, 8, P.kv_bytes_per_token(
                   dims.n_layers, dims.n_kv_heads, dims.head_dim, kind)) for kind in kinds},
               "points": len(rows)}
    print(json.dumps(summary), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--batch", type=int, default=8)
    ap.add_argument("--context", type=int, default=2400)
    ap.add_argument("--kv", choices=["f16", "q8_0", "q8k_f16v", "f16k_q8v", "fp8"], default="f16")
    ap.add_argument("--points", choices=["all", "main"], default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-paged", action="store_true", help="skip the paged-pool step beside the main point")
    ap.add_argument("--no-clocks", action="store_true",
                    help="do not query rocm-smi (for runs under a profiler, whose preload the child would inherit)")
    ap.add_argument("--sweep", action="store_true", help="context x batch x cache sweep (see above)")
    ap.add_argument("--sweep-kv", default="f16,q8_0,fp8")
    ap.add_argument("--sweep-batches", default="1,2,4,8,16")
    ap.add_argument("--sweep-contexts", default="32,2400,4700,6900,16000,32000")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="only run 3 plain device copies of this many MiB (calibrates the HBM byte counters)")
    ap.add_argument("--no-passes", action="store_true",
                    help="skip the standalone GEMM-pass and attention-pass measurements")
    ap.add_argument("--prefill-only", type=int, default=0, metavar="N",
                    help="only time the prefill of an N-token prompt and print its JSON line")
    ap.add_argument("--prefill-kv", choices=["f16", "q8_0", "q8k_f16v", "f16k_q8v", "fp8"], default="f16",
                    help="cache format of --prefill-only")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write profiles/counted_traffic.json from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of "
                         "this bench (--points main at --batch/--context/--kv) and of --copy-probe-mb; no GPU work")
    ap.add_argument("--traffic-command", default="", help="the profiled command, recorded with --traffic-from")
    args = ap.parse_args()
    if args.traffic_from:
        import quantized_decode_amd as qd
        record_traffic(qd, *args.traffic_from, args.copy_probe_mb or 1024, args.batch, args.context, args.kv,
                       args.traffic_command)
        return
    if args.copy_probe_mb:
        import torch
        n = args.copy_probe_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 3}))
        return
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
    if args.sweep:
        sweep(args, qd, sd, dims, dev_model)
        return
    if args.prefill_only:
        log(f"prefill of a {args.prefill_only}-token prompt")
        print(json.dumps({"prefill": prefill_point(qd, sd, dims, dev_model, args.prefill_only, 9200,
                                                   args.prefill_kv)}))
        return

    points = [(args.batch, args.context, args.kv)]
    if args.points == "all":
        for p in [(8, 2400, "f16"), (8, 6900, "f16"), (8, 2400, "q8_0"), (8, 6900, "q8_0"), (8, 2400, "q8k_f16v"),
                  (8, 2400, "f16k_q8v"), (8, 2400, "fp8"), (8, 6900, "fp8"), (1, 2400, "f16"), (2, 2400, "f16"),
                  (4, 2400, "f16"), (16, 3400, "f16"), (16, 3400, "q8_0"), (8, 8192, "q8_0"), (8, 19000, "q8_0")]:
            if p not in points:
                points.append(p)
    results = []
    kernels = None
    paged = None
    for i, (bsz, L, kind) in enumerate(points):
        cap = (L + args.warmup + args.steps + 2 + 31) // 32 * 32
        log(f"point B={bsz} L={L} kv={kind}: building caches (capacity {cap})")
        sm = build_point(qd, sd, dims, dev_model, bsz, L, kind, cap, 2000 + i)
        torch.cuda.synchronize()
        per, wall = time_point(qd, sm, bsz, L, args.steps, args.warmup, dims.vocab, 3000 + i)
        ms = sum(per) / len(per)
        srt = sorted(per)
        l_mean = L + args.warmup + (args.steps - 1) / 2
        step_bytes = W_BYTES + bsz * l_mean * KV_BYTES_PER_TOKEN[kind]
        gbps = step_bytes / (ms * 1e-3) / 1e9
        results.append({"batch": bsz, "context": L, "kv": kind, "ms_per_step": ms,
                        "ms_p10": srt[len(srt) // 10], "ms_p50": srt[len(srt) // 2],
                        "ms_p90": srt[min(len(srt) - 1, (9 * len(srt)) // 10)],
                        "tok_per_s": bsz / (ms * 1e-3), "bytes_per_step": step_bytes, "achieved_GBps": gbps,
                        "frac_of_8TBps": gbps / PEAK_HBM_GBPS, "wall_s": wall})
        log(f"  {ms:.3f} ms/step, {bsz / (ms * 1e-3):.1f} tok/s, {gbps:.0f} GB/s on the byte model")
        if i == 0 and not args.no_paged:
            log("the same point's step over paged pools (pages of 256)")
            pper = time_paged_step(qd, sd, dims, dev_model, bsz, L, kind, min(args.steps, 16), args.warmup, 8000)
            pms = sum(pper) / len(pper)
            paged = {"batch": bsz, "context": L, "kv": kind, "page_tokens": 256, "ms_per_step": pms,
                     "tok_per_s": bsz / (pms * 1e-3), "vs_arena_step": pms / ms,
                     "note": "qkdec_step_paged, each sequence's pages scattered over the pool; graph replays, "
                             "timed right after the arena step of the same point"}
            log(f"  paged: {pms:.3f} ms/step ({pms / ms:.3f} x the arena step)")
            torch.cuda.empty_cache()
        if i == 0:
            log("per-kernel timing (HIP events on the launching stream)")
            kernels = kernel_timing(qd, sd, dev_model, sm, bsz, L, 4000)
        del sm
        torch.cuda.empty_cache()

    main_pt = results[0]
    dom_name, dom = max(kernels.items(), key=lambda kv: kv[1]["ms_per_step"])
    achieved = dom["bytes_per_launch"] / (dom["avg_ms"] * 1e-3) / 1e9
    traffic = counted_traffic(qd, dom_name, main_pt["batch"], main_pt["context"], main_pt["kv"])
    roofline = {"kernel": dom_name, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic, "avg_launch_ms": dom["avg_ms"],
                "algorithmic_bytes_per_launch": dom["bytes_per_launch"],
                "launches_per_step": dom["launches_per_step"]}

    passes = None
    if not args.no_passes:
        log("standalone GEMM pass (fp16 activations, B = 1, 2, 4, 8, 16)")
        passes = {"gemm": gemm_pass(qd, sd, dev_model, [1, 2, 4, 8, 16], 9000)}
        log("standalone attention pass (B = 8, L = 2400 / 4700 / 6900 and ragged)")
        passes["attention"] = attention_pass(qd, sd, 8, [2400, 4700, 6900], 4242, 9100)
        torch.cuda.empty_cache()
        log("prefill of a 2048-token prompt")
        passes["prefill"] = prefill_point(qd, sd, dims, dev_model, 2048, 9200)
        log(f"  prefill: {passes['prefill']['ms']:.1f} ms, {passes['prefill']['tok_per_s']:.0f} tok/s")
        torch.cuda.empty_cache()

    log("streaming-read ceiling (4 GiB) and clocks")
    ceiling = read_ceiling()
    for pt in results:
        pt["frac_of_read_ceiling"] = pt["achieved_GBps"] / ceiling["GBps"]

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: fp64 oracle on a bounded sample")
        cpu = cpu_baseline(dims, dev_model, args.batch, args.context, 5000)

    out = {
        "metric": "aggregate decode tok/s at B=8, L=2.4k/6.9k; achieved HBM GB/s vs peak",
        "value": main_pt["tok_per_s"], "unit": "tok/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": main_pt["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": compute_dtype(main_pt["kv"]), "data": "synthetic",
        "config": {"workload": f"batched decode step, Qwen-shaped synthetic decoder (36 layers, hidden 4096, "
                               f"32/8 heads x 128, FFN 12288, vocab 151936), Q4_K weights, {main_pt['kv']} KV, "
                               f"B={main_pt['batch']}, L={main_pt['context']}",
                   "batch": main_pt["batch"], "context": main_pt["context"], "kv": main_pt["kv"]},
        "achieved_GBps": main_pt["achieved_GBps"], "frac_of_8TBps": main_pt["frac_of_8TBps"],
        "frac_of_read_ceiling": main_pt["frac_of_read_ceiling"], "read_ceiling": ceiling,
        "clocks": None if args.no_clocks else clocks(),
        "roofline": roofline, "kernels": kernels, "points": results, "paged_step": paged, "passes": passes,
        "cpu_baseline": cpu, "library_build_id": qd.qkdec_build_id(),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
