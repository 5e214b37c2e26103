"""Workload shapes for the contextual-sparsity decode step.

Each shape follows a model size the pages evaluate on:

* "Deja Vu: Contextual Sparsity for Efficient LLMs at Inference Time"
  (arXiv 2310.17157) -- OPT-style ReLU decoder layers; §2.3 defines the
  sparsified MLP (Eq. 1) and attention (Eq. 2); §5 / App. C.1 use OPT-66B and
  OPT-175B, batch 1, and batches whose neuron sets are united.
* "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding"
  (arXiv 2609.33889v1) -- §4.1: batch-1 decoding from 2K to 128K context with
  attention-scored KV selection composed with activation sparsity.

Nothing here computes; these are sizes only.  Keep counts are integers, rounded
down from the percentage by the caller (floor(p * total)).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class LayerDims:
    d: int                 # model width (d_model)
    N: int                 # MLP width (d_ffn, "4d" on the DejaVu page)
    h: int = 0             # attention heads (0 = MLP block only)
    d_h: int = 128         # head width
    r_attn: int = 128      # head-predictor rank
    r_mlp: int = 128       # neuron-predictor rank
    wdt: str = "f16"       # weight storage type: "f16" or "f32"

    @property
    def wbytes(self) -> int:
        return 2 if self.wdt == "f16" else 4


@dataclass(frozen=True)
class Workload:
    name: str
    dims: LayerDims
    layers: int = 1
    n_ctx: int = 0                       # tokens already in the KV cache
    k_heads: int = 0                     # selected heads per step (0 = no attention)
    k_neurons: int = 0                   # selected neurons per step
    batch: Tuple[int, ...] = (1,)
    steps: int = 1
    kv_keep: float = 1.0                 # fraction of cached positions kept (KV branch)
    neuron_keep_sweep: Tuple[float, ...] = field(default_factory=tuple)
    ctx_sweep: Tuple[int, ...] = field(default_factory=tuple)


# A single OPT-style ReLU MLP block in fp32 with a d -> 64 -> d_ffn predictor;
# keep 256 of 1024 neurons.  Small enough for brute-force checking.
MLP_BLOCK_FP32 = Workload(
    name="opt-style-mlp-block-d256-ffn1024-fp32",
    dims=LayerDims(d=256, N=1024, h=0, r_attn=0, r_mlp=64, wdt="f32"),
    k_neurons=256,
)

# One OPT-13B-shaped decoder layer, fp16 weights, fp32 accumulate, batch 1,
# 2048 cached tokens, 10% of neurons and 50% of heads kept.
OPT13B_LAYER = Workload(
    name="opt13b-layer-d5120-h40-ffn20480-fp16-ctx2048",
    dims=LayerDims(d=5120, N=20480, h=40, d_h=128, r_attn=128, r_mlp=128, wdt="f16"),
    n_ctx=2048, k_heads=20, k_neurons=2048,
)

# A 64-layer OPT-66B-shaped stack; 1024 cached tokens; neuron keep sweep with
# half of the heads; 128 decoded tokens.
OPT66B_STACK = Workload(
    name="opt66b-stack-64L-d9216-h72-ffn36864-fp16-ctx1024",
    dims=LayerDims(d=9216, N=36864, h=72, d_h=128, r_attn=128, r_mlp=128, wdt="f16"),
    layers=64, n_ctx=1024, k_heads=36, k_neurons=3686, steps=128,
    neuron_keep_sweep=(0.05, 0.10, 0.25, 0.50, 1.00),
)

# 48 OPT-175B-shaped layers, batched decode over the union of per-sequence
# neuron sets; heads dense; 512 cached tokens; 10% neurons.
OPT175B_SHARE = Workload(
    name="opt175b-48L-d12288-h96-ffn49152-fp16-ctx512",
    dims=LayerDims(d=12288, N=49152, h=96, d_h=128, r_attn=128, r_mlp=128, wdt="f16"),
    layers=48, n_ctx=512, k_heads=96, k_neurons=4915, batch=(1, 2, 4, 8, 16),
)

# 32 layers at d=4096, long context; 10% neurons, 10% of KV positions per head.
LONGCTX_STACK = Workload(
    name="longctx-32L-d4096-h32-ffn16384-fp16",
    dims=LayerDims(d=4096, N=16384, h=32, d_h=128, r_attn=128, r_mlp=128, wdt="f16"),
    layers=32, k_heads=32, k_neurons=1638, kv_keep=0.10,
    ctx_sweep=(2048, 8192, 16384, 32768, 131072),
)

ALL = (MLP_BLOCK_FP32, OPT13B_LAYER, OPT66B_STACK, OPT175B_SHARE, LONGCTX_STACK)


def scaled(w: Workload, **dims) -> Workload:
    """A copy of ``w`` with some layer dimensions replaced (reduced test shapes)."""
    return replace(w, dims=replace(w.dims, **dims))
