"""Pins of oracle/bytes.py to the values the pages print (tests/golden/)."""
import json
import math
import os

import pytest

from oracle import bytes as ob

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


BC = _load("bytecross_printed.json")
DJ = _load("dejavu_tables.json")


def _model(name):
    m = BC["models"][name]
    allp, ff = ob.llama_layer_proj_params(m["d"], m["n_q_heads"], m["n_kv_heads"], m["d_h"], m["d_ff"])
    return m, 2 * allp, 2 * ff, ob.kv_bytes_per_token(m["n_kv_heads"], m["d_h"])


def _lm_head_other(m):
    # LM head (vocab x d), one embedding row, 2 norms per layer + final norm, fp16
    return 2 * (m["vocab"] * m["d"] + m["d"] + (2 * m["layers"] + 1) * m["d"])


def test_llama8b_layer_bytes():
    m, b_proj, _, b_kv = _model("Llama-3.1-8B")
    case = BC["layer_bytes"][0]
    assert round(b_proj / 1e6) == case["proj_bytes_MB"]
    assert b_kv == case["kv_bytes_per_token"]


@pytest.mark.parametrize("case", BC["crossovers"], ids=lambda c: f'{c["model"]}-{c["scope"]}-{c["r_P"]}-{c["r_KV"]}')
def test_crossover_values(case):
    _, b_all, b_ff, b_kv = _model(case["model"])
    b_sav = b_all if case["scope"] == "all" else b_ff
    n_star = ob.crossover(b_sav, case["r_P"], b_kv, case["r_KV"])
    assert round(n_star) == case["n_star"]


@pytest.mark.parametrize("case", BC["crossovers_in_K"], ids=lambda c: c["model"])
def test_crossover_in_thousands_of_1024(case):
    _, b_all, b_ff, b_kv = _model(case["model"])
    b_sav = b_all if case["scope"] == "all" else b_ff
    assert round(ob.crossover(b_sav, case["r_P"], b_kv, case["r_KV"]) / 1024, 1) == case["K"]


def test_layer_count_cancels():
    _, b_all, _, b_kv = _model("Llama-3.1-8B")
    for L in (1, 16, 32, 80):
        # equal savings per stack <=> equal savings per layer
        n = ob.crossover(b_all, 0.5, b_kv, 0.3)
        assert math.isclose(ob.saved_proj(b_all, 0.5, L), ob.saved_kv(b_kv, n, 0.3, L), rel_tol=1e-12)


def test_qwen_shares():
    m, b_all, b_ff, b_kv = _model("Qwen3-8B")
    L, oth = m["layers"], _lm_head_other(m)
    for case in BC["shares"]:
        n = case["n"]
        T = ob.step_bytes(b_all, b_kv, n, oth, L)
        if case["what"] == "ff_share_of_reads":
            val = 100 * L * b_ff / T
        elif case["what"] == "cache_share_of_reads":
            val = 100 * L * b_kv * n / T
        else:
            val = 100 * ob.saved_kv(b_kv, n, case["r_KV"], L) / ob.saved_proj(b_ff, case["r_P"], L)
        digits = 0 if float(case["percent"]).is_integer() else 1
        assert round(val, digits) == case["percent"], case


def test_kv_bound_at_128k_needs_lm_head():
    m, b_all, _, b_kv = _model("Llama-3.1-8B")
    case = BC["bounds"][0]
    L, n = m["layers"], case["n"]
    T = ob.step_bytes(b_all, b_kv, n, _lm_head_other(m), L)
    s = ob.speedup(T, ob.saved_kv(b_kv, n, case["r_KV"], L))
    assert round(s, 2) == case["speedup"]
    T0 = ob.step_bytes(b_all, b_kv, n, 0, L)
    assert round(ob.speedup(T0, ob.saved_kv(b_kv, n, case["r_KV"], L)), 2) != case["speedup"]


def test_bounds_monotone_in_context():
    # ByteCross §3: the projection bound falls with context, the KV bound rises
    _, b_all, _, b_kv = _model("Llama-3.1-8B")
    prev_p, prev_kv = math.inf, 0.0
    for n in (2048, 8192, 32768, 131072):
        T = ob.step_bytes(b_all, b_kv, n, 0, 32)
        sp = ob.speedup(T, ob.saved_proj(b_all, 0.5, 32))
        skv = ob.speedup(T, ob.saved_kv(b_kv, n, 0.3, 32))
        assert sp < prev_p and skv > prev_kv
        prev_p, prev_kv = sp, skv
    # at n* the two single-branch bounds coincide
    n_star = ob.crossover(b_all, 0.5, b_kv, 0.3)
    T = ob.step_bytes(b_all, b_kv, n_star, 0, 32)
    assert math.isclose(ob.speedup(T, ob.saved_proj(b_all, 0.5, 32)),
                        ob.speedup(T, ob.saved_kv(b_kv, n_star, 0.3, 32)), rel_tol=1e-12)


def test_fixed_budget_and_batch():
    _, b_all, _, b_kv = _model("Llama-3.1-8B")
    assert ob.kv_keep_for_budget(3276, 32768) == pytest.approx(0.1, abs=1e-4)
    assert ob.kv_keep_for_budget(10, 5) == 1.0
    n1 = ob.batch_crossover(b_all, 0.5, b_kv, 0.3, 1)
    assert n1 == pytest.approx(ob.crossover(b_all, 0.5, b_kv, 0.3))
    # a larger union keep and more caches both pull the crossover in
    assert ob.batch_crossover(b_all, 0.52, b_kv, 0.3, 1) < n1
    assert ob.batch_crossover(b_all, 0.5, b_kv, 0.3, 8) == pytest.approx(n1 / 8)


def _within_last_digit(value, printed):
    s = repr(printed)
    dec = len(s.split(".")[1]) if "." in s and "e" not in s else 0
    return abs(value - printed) <= 10.0 ** (-dec) + 1e-12


def test_dejavu_table2():
    d, g = DJ["d"], DJ["gpus"]
    attn, mlp = ob.opt_layer_params(d)
    assert mlp == DJ["mlp_to_attention_params"] * attn
    for row, params in zip(DJ["table2"], (attn, mlp)):
        flops = 2 * params
        io = 2 * params
        assert _within_last_digit(flops / 1e9, row["gflops"]), row
        assert _within_last_digit(io / 2 ** 30, row["io_gb"]), row
        assert _within_last_digit(1e3 * flops / (g * DJ["flops_per_gpu"]), row["compute_ms"]), row
        assert _within_last_digit(1e3 * (io / 2 ** 30) * 1e9 / (g * DJ["bytes_per_s_per_gpu"]), row["io_ms"]), row


def test_dejavu_table1():
    t, g = DJ["table1"], DJ["gpus"]
    # compute latency of the printed TFLOPs on 8 x 312 TFLOP/s
    assert round(1e3 * t["tflops"] * 1e12 / (g * DJ["flops_per_gpu"]), 2) == t["compute_ms"]
    # 2 flops per parameter per token
    assert abs(2 * t["params"] * t["tokens"] / 1e12 - t["tflops"]) / t["tflops"] < 0.01
    # prompting reads the fp16 weights once, generation once per token
    assert round(2 * t["params"] / 2 ** 30, -1) == t["prompt_io_gb"]
    assert round(2 * t["params"] * t["tokens"] / 2 ** 40) == t["gen_io_tb"]
    bw = g * DJ["bytes_per_s_per_gpu"]
    assert round(1e3 * t["prompt_io_gb"] * 1e9 / bw, 1) == t["prompt_io_ms"]
    assert float(f'{1e3 * t["gen_io_tb"] * 1e12 / bw:.2g}') == t["gen_io_ms"]


def test_dejavu_sparsity_arithmetic():
    s = DJ["sparsity_speedup"]
    assert round(1 / (1 - s["total_sparsity"])) == s["speedup"]
    w = DJ["weighted_sparsity"]
    attn, mlp = ob.opt_layer_params(DJ["d"])
    combined = (mlp * w["mlp"] + attn * w["attention"]) / (mlp + attn)
    assert round(combined, 3) == w["combined"]
    assert abs(combined - w["reported"]) < 0.02


def test_decode_layer_bytes_dense_is_12d2():
    d = 12288
    dense = ob.decode_layer_bytes(d, 96, 128, 4 * d, n_att=0, k_heads=96, k_neurons=4 * d, wbytes=2)
    attn, mlp = ob.opt_layer_params(d)
    biases = 2 * (3 * d + d + 4 * d + d)
    assert dense == 2 * (attn + mlp) + biases
    # selecting everything with the predictors costs exactly the predictor bytes more
    withp = ob.decode_layer_bytes(d, 96, 128, 4 * d, 0, 96, 4 * d, 2, r_attn=128, r_mlp=128)
    assert withp - dense == 2 * 128 * (d + 96 + d + 4 * d)
