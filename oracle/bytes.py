"""Byte account of a decode step, the byte crossover and ideal speedups.

ByteCross ("Where Activation Sparsity and KV-Cache Sparsity Cross in LLM
Decoding") prints no formula, only what they produce; these are the plainest
formulas consistent with its statements, and they reproduce every value it
prints (pinned in tests/test_bytes_pins.py):

  §3.1  a step reads the projection weights once (B_proj bytes per layer),
        the KV cache (b_kv bytes per cached token per layer, so b_kv * n),
        and other reads (LM head, one embedding row, norm weights: B_oth).
  §3.2  the projection branch keeps a fraction r_P of its channels, the KV
        branch reads a fraction r_KV of the cached entries.
  §3.3  the crossover n* is the context where the bytes the two branches
        remove are equal; ideal speedups are total bytes / bytes left; a
        fixed token budget b means r_KV = b / n; in a batch the projection
        reads are shared (union keep ratio) while KV reads scale with B.
  App. C  the layer count cancels from n*.

DejaVu §2.2 (Tables 1 and 2) accounts one OPT-175B layer as 4 d^2 attention
and 8 d^2 MLP parameters, 2 flops per parameter per token, 2 bytes per
parameter (fp16).
"""
from __future__ import annotations


def crossover(b_sav: float, r_p: float, b_kv: float, r_kv: float) -> float:
    """n* with (1 - r_P) * B_sav = (1 - r_KV) * b_kv * n*  (per layer)."""
    return (1.0 - r_p) * b_sav / ((1.0 - r_kv) * b_kv)


def batch_crossover(b_sav: float, r_union: float, b_kv: float, r_kv: float, batch: int) -> float:
    """Per-sequence crossover in a batch: shared projection savings at the
    union keep ratio against KV savings of ``batch`` caches."""
    return (1.0 - r_union) * b_sav / (batch * (1.0 - r_kv) * b_kv)


def step_bytes(b_proj: float, b_kv: float, n: float, b_other: float, layers: int,
               batch: int = 1) -> float:
    """T = L (B_proj + B b_kv n) + B_oth: bytes one dense decode step reads."""
    return layers * (b_proj + batch * b_kv * n) + b_other


def saved_proj(b_sav: float, r_p: float, layers: int) -> float:
    return layers * (1.0 - r_p) * b_sav


def saved_kv(b_kv: float, n: float, r_kv: float, layers: int, batch: int = 1) -> float:
    return layers * batch * (1.0 - r_kv) * b_kv * n


def speedup(total: float, saved: float) -> float:
    """Ideal speedup when ``saved`` of ``total`` bytes are not read."""
    return total / (total - saved)


def kv_keep_for_budget(budget: int, n: int) -> float:
    """Fixed token budget b: r_KV = b / n (capped at 1)."""
    return min(1.0, budget / n)


# ---- model shapes -----------------------------------------------------------

def llama_layer_proj_params(d: int, n_q_heads: int, n_kv_heads: int, d_h: int, d_ff: int):
    """(all projection params, FF params) of a Llama-style layer: Q, O are
    d x (n_q d_h); K, V are d x (n_kv d_h); gate, up, down are d x d_ff."""
    attn = d * (2 * n_q_heads * d_h + 2 * n_kv_heads * d_h)
    ff = 3 * d * d_ff
    return attn + ff, ff


def kv_bytes_per_token(n_kv_heads: int, d_h: int, elem_bytes: int = 2) -> int:
    """K and V of one token of one layer."""
    return 2 * n_kv_heads * d_h * elem_bytes


def opt_layer_params(d: int):
    """(attention, MLP) parameters of an OPT layer: 4 d^2 and 8 d^2
    (DejaVu §2.2: MLP parameters are twice the attention's)."""
    return 4 * d * d, 8 * d * d


def decode_layer_bytes(d: int, h: int, d_h: int, N: int, n_att: float, k_heads: int,
                       k_neurons: int, wbytes: int, r_attn: int = 0, r_mlp: int = 0,
                       fc2_rows: float | None = None, kv_bytes: int = 2) -> float:
    """Bytes one decode step of one layer must read: the selected heads' Q, K,
    V and O blocks and biases, their K/V over ``n_att`` positions, the
    selected fc1 rows and b1 entries, ``fc2_rows`` fc2 rows (default: all
    selected), b_O, b2 and the two predictors (DejaVu §2.3 Eqs. 1-2, §4.1-4.2).
    With k_heads = h, k_neurons = N and no predictors this is the dense step.
    """
    fc2_rows = k_neurons if fc2_rows is None else fc2_rows
    attn_w = 4 * k_heads * d_h * d * wbytes + 3 * k_heads * d_h * wbytes + d * wbytes
    kv = 2 * k_heads * n_att * d_h * kv_bytes
    mlp_w = (k_neurons + fc2_rows) * d * wbytes + k_neurons * wbytes + d * wbytes
    pred = (r_attn * d + r_attn * h + r_mlp * d + r_mlp * N) * wbytes
    return attn_w + kv + mlp_w + pred
