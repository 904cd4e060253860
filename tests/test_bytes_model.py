"""The byte model against the numbers the pages print (tests/golden/pages_numbers.json)."""
import json
import os

import pytest

import synth
from oracle import bytes_model as M

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def test_kv_bytes_per_token_matches_pages():
    # 36 layers x 8 KV heads x 128 x (K, V) x 2 bytes
    k = M.kv_bytes_per_token(synth.QWEN_SHAPED, "f16")
    assert k == 147456
    assert abs(k / 1000 - GOLD["kv_kb_per_token_f16"]["value"]) < 0.5
    kq = M.kv_bytes_per_token(synth.QWEN_SHAPED, "q8_0")
    assert kq == 78336                     # 34 bytes per 32 elements
    # the pages count one byte per element for int8 ("74 KB"): 73,728 B
    assert abs(k / 2 / 1000 - GOLD["kv_kb_per_token_int8"]["value"]) < 0.5
    # an 8-bit float cache has no scales: exactly half of fp16, the pages' 74 KB
    kf = M.kv_bytes_per_token(synth.QWEN_SHAPED, "fp8")
    assert kf == 73728 and 2 * kf == k
    assert abs(kf / 1000 - GOLD["kv_kb_per_token_int8"]["value"]) < 0.5
    # about a gigabyte per agent at 6,900 tokens
    assert abs(6900 * 147e3 / 1e9 - GOLD["kv_gb_at_6900_tokens"]["value"]) < 0.05


def test_weight_bytes_of_the_synthetic_model():
    dims = synth.QWEN_SHAPED
    assert M.layer_weight_bytes(dims) == 108527616
    assert M.weight_bytes(dims) == 5152849920
    assert M.weight_bytes(dims) - dims.vocab * dims.hidden * 2 - 73 * 4096 * 4 == 3906994176
    # same order as the pages' 5.5 GB
    assert abs(M.weight_bytes(dims) / 1e9 - GOLD["weights_gb"]["value"]) / 5.5 < 0.07
    assert M.weight_bytes(synth.TOY) - synth.TOY.vocab * 512 * 2 - 5 * 512 * 4 == 3391488


def test_speedup_table():
    g = GOLD["speedup_b8"]
    for length, printed in g["rows"]:
        s = M.speedup(g["batch"], length, g["w_bytes"], g["k_bytes"])
        assert abs(s - printed) <= 0.05 * printed + 0.05, (length, s, printed)
    assert M.speedup(8, 0, 5.5e9, 147e3) == 8.0
    # exact values of the formula at the printed contexts
    exact = [M.speedup(8, L, 5.5e9, 147e3) for L in (2400, 4700, 6900, 16000, 55000)]
    assert [round(x, 3) for x in exact] == [5.626, 4.491, 3.828, 2.583, 1.549]


def test_crossovers():
    g = GOLD["crossover_p2"]
    x = M.crossover(g["w_bytes"], g["batch"], g["k_bytes"])
    assert round(x) == 4677 and abs(x - g["value"]) / g["value"] < 0.01
    g = GOLD["crossover_p3_f16"]
    x = M.crossover(g["w_mb"], g["batch"], g["k_mb"])
    assert round(x) == 5029 and abs(x - g["value"]) / g["value"] < 0.01
    g = GOLD["crossover_p3_q8"]
    x = M.crossover(g["w_mb"], g["batch"], g["k_mb"])
    assert abs(x - g["value"]) / g["value"] < 0.01
    # with the per-token crossover the per-token KV bytes equal the per-token weight bytes
    assert abs(M.bytes_per_token(5.5e9, 8, 4677.0, 147e3) - 2 * 5.5e9 / 8) / (5.5e9 / 4) < 1e-3
    # the synthetic model's own crossovers at B=8
    w = M.weight_bytes(synth.QWEN_SHAPED)
    assert round(M.crossover(w, 8, 147456)) == 4368
    assert round(M.crossover(w, 8, 78336)) == 8222


def test_fig1_step_model():
    g = GOLD["fig1_step_ms"]
    for b, ms, agg, per in zip(g["batch"], g["ms"], g["agg_tok_s"], g["per_seq_tok_s"]):
        t = M.fitted_step_ms(b, 0, 0.0)
        assert abs(t - ms) < 0.051
        assert abs(1000 * b / t - agg) <= 1.0
        assert abs(1000 / t - per) <= 0.06
    br = GOLD["fig1_breakdown_b1_ms"]
    assert abs(sum(v for k, v in br.items() if k not in ("total", "cite")) - br["total"]) < 1e-9


def test_tab1_capacity():
    g = GOLD["tab1_capacity"]
    for row in g["rows"]:
        budget = M.kv_budget_bytes(row["vram_gb"] * 1e9, 5.5e9, g["frac"])
        assert abs(budget / 1e9 - row["budget_gb"]) < 0.05
        toks = M.kv_capacity_tokens(row["vram_gb"] * 1e9, 5.5e9, 147e3, g["frac"])
        assert abs(toks - row["tokens"]) / row["tokens"] < 0.01
        assert abs(toks / 8 - row["per8"]) / row["per8"] < 0.03
        assert abs(toks / 16 - row["per16"]) / row["per16"] < 0.02


def test_tab3_ceilings_follow_the_step_fit():
    g = GOLD["tab3_ceilings"]
    b = g["batch"]
    # back k out of the 4k fp16 ceiling, then every other printed ceiling follows
    k = ((b / 205 * 1000 - 16.9) / b - 1.1) / 4000
    assert 4.1e-4 < k < 4.2e-4
    for ctx, c16, c8 in g["rows"]:
        if c16 is not None:
            t = M.fitted_step_ms(b, ctx, k)
            assert abs(1000 * b / t - c16) / c16 < 0.02, (ctx, 1000 * b / t, c16)
        t8 = M.fitted_step_ms(b, ctx, k / 2)
        assert abs(1000 * b / t8 - c8) / c8 < 0.02, (ctx, 1000 * b / t8, c8)
    assert abs(1000 * b / M.fitted_step_ms(b, 0, k) - g["short_ceiling"]) <= 1.0
    # the printed KV gigabytes use about 0.137 MB per token: half for Q8
    for ctx, gb16, gb8 in g["kv_gb"]:
        assert abs(gb16 / gb8 - 2.0) < 0.015   # printed to one decimal
        assert abs(gb16 * 1e9 / (8 * ctx) - 0.137e6) / 0.137e6 < 0.03


@pytest.mark.parametrize("batch,length,kind,gb", [
    (8, 2400, "f16", 7.984), (8, 6900, "f16", 13.292), (8, 2400, "q8_0", 6.657), (8, 6900, "q8_0", 9.477)])
def test_metric_points(batch, length, kind, gb):
    dims = synth.QWEN_SHAPED
    by = M.step_bytes(M.weight_bytes(dims), [length] * batch, M.kv_bytes_per_token(dims, kind))
    assert abs(by / 1e9 - gb) < 0.0006
