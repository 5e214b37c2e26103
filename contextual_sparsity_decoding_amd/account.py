"""Algorithmic bytes of one sparse decode step of one layer, per kernel.

"Algorithmic" means what the method must move at least once: the selected
weight rows and head blocks, the KV entries attended to, the predictor
weights, biases and the small activation vectors.  Dense bytes the method
avoids are not counted.  Pages: DejaVu (arXiv 2310.17157) §2.3 Eqs. 1-2 and
§4.1-4.2 define what is read; ByteCross (arXiv 2609.33889v1) §3.1 splits a
step into projection-weight bytes and KV bytes that grow with context.

Used by bench.py to turn measured times into effective bandwidth.
"""
from __future__ import annotations

from dataclasses import dataclass

from .configs import LayerDims

KV_BYTES = 2           # fp16 cache
ACT_BYTES = 4          # fp32 activations


@dataclass
class StepBytes:
    head_pred: float
    qkv: float
    attn: float
    out_proj: float
    neuron_pred: float
    fc1: float
    fc2: float
    other: float

    @property
    def total(self) -> float:
        return (self.head_pred + self.qkv + self.attn + self.out_proj + self.neuron_pred + self.fc1 + self.fc2
                + self.other)


def step_bytes(dims: LayerDims, k_heads: int, k_neurons: int, n_att: float, fc2_rows: float,
               holes: float = 0.0, head_pred: bool = True, neuron_pred: bool = True, B: int = 1) -> StepBytes:
    """Bytes of one decode step of one layer.

    k_heads / k_neurons  selected heads / neurons (h / N for the dense path)
    n_att                KV positions each selected head attends to
    fc2_rows             fc2 rows read (survivors of the ReLU, <= k_neurons)
    holes                recomputed K/V positions summed over heads (each
                         re-reads one stored fp32 input row and writes K and V)
    """
    d, h, dh, N, wb = dims.d, dims.h, dims.d_h, dims.N, dims.wbytes
    act = ACT_BYTES * d * B
    hp = (dims.r_attn * d + h * dims.r_attn) * wb + act if head_pred else 0.0
    npd = (dims.r_mlp * d + N * dims.r_mlp) * wb + act if neuron_pred else 0.0
    qkv = (3 * k_heads * dh * d + 3 * k_heads * dh) * wb + act \
        + 2 * k_heads * dh * KV_BYTES * B + holes * (ACT_BYTES * d + 2 * dh * KV_BYTES)
    attn = 2 * k_heads * n_att * dh * KV_BYTES * B
    wo = (k_heads * dh * d + d) * wb + act * 2
    fc1 = (k_neurons * d + k_neurons) * wb + act
    fc2 = (fc2_rows * d + d) * wb + act * 2
    other = 2 * act + 4 * ACT_BYTES * d      # two LayerNorms: x in, y out, gamma and beta
    return StepBytes(hp, qkv, attn, wo, npd, fc1, fc2, other)
