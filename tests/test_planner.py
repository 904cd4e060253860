"""Capacity planner (host arithmetic) against the oracle's byte model and the
numbers the pages print (tests/golden/pages_numbers.json)."""
import json
import os

import pytest

import synth
from oracle import bytes_model as M
from quantized_decode_amd import planner as P

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))
D = synth.QWEN_SHAPED


def _k(kind):
    return P.kv_bytes_per_token(D.n_layers, D.n_kv_heads, D.head_dim, kind)


def test_bytes_match_the_oracle_byte_model():
    for kind in ("f16", "q8_0", "fp8"):
        assert _k(kind) == M.kv_bytes_per_token(D, kind)
    assert _k("q8k_f16v") == _k("f16k_q8v") == (_k("f16") + _k("q8_0")) / 2
    w = P.model_weight_bytes(D.n_layers, D.hidden, D.n_q_heads, D.n_kv_heads, D.head_dim, D.ffn, D.vocab)
    assert w == M.weight_bytes(D) == 5152849920
    for lengths in ([2400] * 8, [512, 8192, 3000], []):
        assert P.step_bytes(w, lengths, _k("f16")) == M.step_bytes(w, lengths, _k("f16"))
    with pytest.raises(ValueError):
        P.kv_bytes_per_token(36, 8, 128, "q4_0")


def test_speedup_crossover_and_ceiling_match_the_oracle():
    w, k = M.weight_bytes(D), _k("f16")
    for b in (1, 2, 8, 16):
        assert P.crossover_context(w, b, k) == pytest.approx(M.crossover(w, b, k), rel=1e-15)
        for L in (0, 100, 2400, 6900, 55000):
            assert P.speedup(b, L, w, k) == pytest.approx(M.speedup(b, L, w, k), rel=1e-15)
    # the ceiling is B / time and time = bytes / bandwidth
    assert P.ceiling_tok_s(8e12, w, 8, 2400, k) == pytest.approx(8 * 8e12 / M.step_bytes(w, [2400] * 8, k))


def test_speedup_table_of_the_pages():
    g = GOLD["speedup_b8"]
    for L, s in g["rows"]:
        assert P.speedup(g["batch"], L, g["w_bytes"], g["k_bytes"]) == pytest.approx(s, rel=0.05)


def test_capacity_table_of_the_pages():
    # 0.85 of VRAM minus 5.5 GB of weights, at 147 KB per token
    g = GOLD["tab1_capacity"]
    for row in g["rows"]:
        plan = P.plan_capacity(row["vram_gb"] * 1e9, 5.5e9, 147e3, g["frac"])
        assert plan.budget_bytes == pytest.approx(row["budget_gb"] * 1e9, rel=1e-9)
        assert plan.total_tokens == pytest.approx(row["tokens"], rel=0.02)
        assert plan.context_per_sequence(8) == pytest.approx(row["per8"], rel=0.03)
        assert plan.context_per_sequence(16) == pytest.approx(row["per16"], rel=0.03)


def test_capacity_plan_edges():
    plan = P.plan_capacity(16e9, 5.5e9, 147e3)
    n = plan.total_tokens
    assert plan.fits([n]) and not plan.fits([n, 1])
    assert plan.max_batch(n // 3) == 3
    assert plan.context_per_sequence(1) == n
    assert P.plan_capacity(4e9, 5.5e9, 147e3).total_tokens == 0      # the weights alone overflow
    for bad in (lambda: plan.context_per_sequence(0), lambda: plan.max_batch(0),
                lambda: P.plan_capacity(16e9, 5.5e9, 0.0), lambda: P.plan_capacity(16e9, 5.5e9, 1.0, 1.5)):
        with pytest.raises(ValueError):
            bad()
    assert P.slot_capacity(2400, 40) == 2464 and P.slot_capacity(0, 0) == 32 and P.slot_capacity(32, 0) == 32


def test_fp8_doubles_the_crossover():
    # P2 "What a long-running swarm should actually tune": an 8-bit cache halves
    # the per-token bytes and so doubles the crossover context
    w = M.weight_bytes(D)
    assert P.crossover_context(w, 8, _k("fp8")) == pytest.approx(2 * P.crossover_context(w, 8, _k("f16")))


def test_bench_uses_the_planner_byte_model():
    # the bench's per-step bytes (W and k per cache kind) are the planner's and
    # the oracle's: 5,152,849,920 B of weights, 147,456 / 78,336 / 73,728 B per token
    import bench
    assert bench.W_BYTES == M.weight_bytes(D) == 5152849920
    assert bench.KV_BYTES_PER_TOKEN["f16"] == 147456
    assert bench.KV_BYTES_PER_TOKEN["q8_0"] == 78336
    assert bench.KV_BYTES_PER_TOKEN["fp8"] == 73728
    for kind in ("f16", "q8_0", "fp8"):
        assert bench.KV_BYTES_PER_TOKEN[kind] == M.kv_bytes_per_token(D, kind)
