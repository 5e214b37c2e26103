"""Seeded synthetic inputs for the decode step (no method arithmetic here).

The same bytes feed the HIP library and the CPU oracle.  Every tensor is drawn
from its own stream keyed by ``(seed, layer, tensor id, chunk)``, in fixed
chunks of ``_CHUNK`` elements, so the result does not depend on the number of
threads and any single tensor of any layer can be regenerated alone.

Distributions stand in for trained weights and real text (the pages measure
trained OPT / Llama models on C4 and WikiText, which are not available):
weights and biases ~ N(0, 0.02^2), layer inputs and cached K/V ~ N(0, 1),
LayerNorm gain 1 and bias 0.  Values are drawn in fp32 and rounded to fp16
(round-to-nearest-even) for fp16 storage.

Storage layouts (row-major), chosen so that each selected unit is one
contiguous run of memory, as the DejaVu page's §4.4 "Memory coalescing"
prescribes (the transposed fc2 and output projection):

    w1_t   [N][d]          row j = input weights of neuron j   (W1 transposed)
    w2_t   [N][d]          row j = output weights of neuron j  (W2 transposed)
    b1 [N], b2 [d]
    w_qkv_t[3][h][d_h][d]  Q, K, V projections, one [d_h][d] block per head
    b_qkv  [3][h][d_h]
    w_o_t  [h*d_h][d]      rows i*d_h .. i*d_h+d_h-1 = head i's output block
    b_o [d]
    pa1_t [r_attn][d], pa2_t [h][r_attn]   head predictor (P1 and P2 transposed)
    pm1_t [r_mlp][d],  pm2_t [N][r_mlp]    neuron predictor
    ln1_g, ln1_b, ln2_g, ln2_b  fp32 [d]
    K, V   fp16 [B][h][max_len][d_h]
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Sequence

import numpy as np

from .configs import LayerDims

_CHUNK = 1 << 22
_TENSOR_IDS = {
    "w1_t": 1, "b1": 2, "w2_t": 3, "b2": 4,
    "w_qkv_t": 5, "b_qkv": 6, "w_o_t": 7, "b_o": 8,
    "pa1_t": 9, "pa2_t": 10, "pm1_t": 11, "pm2_t": 12,
    "K": 20, "V": 21, "x": 30, "q_obs": 31, "x_cal": 32, "scores": 40,
}
WEIGHT_STD = 0.02


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal(shape: Sequence[int], seed: int, layer: int, tensor: str | int,
           std: float = 1.0, dtype=np.float32) -> np.ndarray:
    """N(0, std^2) samples of ``shape``, rounded to ``dtype`` (fp16 or fp32)."""
    tid = _TENSOR_IDS[tensor] if isinstance(tensor, str) else int(tensor)
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float32)
    nch = max(1, (n + _CHUNK - 1) // _CHUNK)

    def fill(c: int) -> None:
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = np.random.default_rng([seed, layer, tid, c])
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    if nch == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nch)))
    if std != 1.0:
        out *= np.float32(std)
    out = out.reshape(shape)
    if dtype == np.float16:
        return _to_f16(out)
    return out.astype(dtype, copy=False)


def _to_f16(a: np.ndarray) -> np.ndarray:
    """fp32 -> fp16 round-to-nearest-even (torch's vectorised cast when present)."""
    try:
        import torch
        return torch.from_numpy(np.ascontiguousarray(a)).half().numpy()
    except ImportError:  # pragma: no cover
        return a.astype(np.float16)


def _wdt(dims: LayerDims):
    return np.float16 if dims.wdt == "f16" else np.float32


def mlp_weights(dims: LayerDims, seed: int, layer: int = 0) -> Dict[str, np.ndarray]:
    """fc1/fc2 weights and biases plus the neuron predictor, ~N(0, 0.02^2)."""
    wd, s = _wdt(dims), WEIGHT_STD
    d, N, r = dims.d, dims.N, dims.r_mlp
    return {
        "w1_t": normal((N, d), seed, layer, "w1_t", s, wd),
        "b1": normal((N,), seed, layer, "b1", s, wd),
        "w2_t": normal((N, d), seed, layer, "w2_t", s, wd),
        "b2": normal((d,), seed, layer, "b2", s, wd),
        "pm1_t": normal((r, d), seed, layer, "pm1_t", s, wd),
        "pm2_t": normal((N, r), seed, layer, "pm2_t", s, wd),
    }


def attn_weights(dims: LayerDims, seed: int, layer: int = 0) -> Dict[str, np.ndarray]:
    """Q/K/V/O projections, biases and the head predictor, ~N(0, 0.02^2)."""
    wd, s = _wdt(dims), WEIGHT_STD
    d, h, dh, r = dims.d, dims.h, dims.d_h, dims.r_attn
    return {
        "w_qkv_t": normal((3, h, dh, d), seed, layer, "w_qkv_t", s, wd),
        "b_qkv": normal((3, h, dh), seed, layer, "b_qkv", s, wd),
        "w_o_t": normal((h * dh, d), seed, layer, "w_o_t", s, wd),
        "b_o": normal((d,), seed, layer, "b_o", s, wd),
        "pa1_t": normal((r, d), seed, layer, "pa1_t", s, wd),
        "pa2_t": normal((h, r), seed, layer, "pa2_t", s, wd),
    }


def layer_weights(dims: LayerDims, seed: int, layer: int = 0) -> Dict[str, np.ndarray]:
    """All weights of one decoder layer (LayerNorm gain 1, bias 0)."""
    w = {}
    w.update(attn_weights(dims, seed, layer))
    w.update(mlp_weights(dims, seed, layer))
    one = np.ones(dims.d, np.float32)
    zero = np.zeros(dims.d, np.float32)
    w.update(ln1_g=one, ln1_b=zero, ln2_g=one.copy(), ln2_b=zero.copy())
    return w


def kv_cache(h: int, d_h: int, n_filled: int, max_len: int, seed: int,
             layer: int = 0, batch: int = 1):
    """fp16 K, V of shape [batch][h][max_len][d_h]; positions < n_filled ~N(0,1), rest 0."""
    K = np.zeros((batch, h, max_len, d_h), np.float16)
    V = np.zeros((batch, h, max_len, d_h), np.float16)
    if n_filled > 0:
        K[:, :, :n_filled] = normal((batch, h, n_filled, d_h), seed, layer, "K", 1.0, np.float16)
        V[:, :, :n_filled] = normal((batch, h, n_filled, d_h), seed, layer, "V", 1.0, np.float16)
    return K, V


def layer_inputs(d: int, steps: int, batch: int, seed: int, layer: int = 0) -> np.ndarray:
    """Teacher-forced layer inputs x_t ~ N(0,1), fp32 [steps][batch][d]."""
    return normal((steps, batch, d), seed, layer, "x", 1.0, np.float32)


def observation_queries(h: int, n_obs: int, d_h: int, seed: int, layer: int = 0,
                        batch: int = 1) -> np.ndarray:
    """fp16 queries of the last ``n_obs`` prompt tokens, [batch][h][n_obs][d_h] ~N(0,1)."""
    return normal((batch, h, n_obs, d_h), seed, layer, "q_obs", 1.0, np.float16)


def tied_scores(rows: int, n: int, seed: int, levels: int = 0) -> np.ndarray:
    """fp32 scores [rows][n] for selection tests.

    ``levels > 0`` draws from only that many distinct values (many exact ties);
    ``levels == 0`` draws N(0,1) fp32 values.
    """
    g = np.random.default_rng([seed, 0, _TENSOR_IDS["scores"]])
    if levels > 0:
        return (g.integers(0, levels, size=(rows, n)).astype(np.float32) - levels / 2) * np.float32(0.25)
    return g.standard_normal((rows, n), dtype=np.float32)


# ---- counter-based stream (the large workloads) ------------------------------
# Stacks of 100+ GB are generated on the device by the HIP library's
# dv_fill_normal; libsynth.so (synth_philox.c, built with gcc) is the host
# side of the same generator, written separately from the same definition
# (Philox-4x32-10 with Box-Muller; see synth_philox.c), so that any tensor,
# or any range of one, can be regenerated on the host for the oracle.

_SYNTH_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynth.so")
_synth = None


def _lib():
    global _synth
    if _synth is None:
        if not os.path.exists(_SYNTH_LIB):
            raise ImportError(f"{_SYNTH_LIB} is missing: build it with "
                              "`python -m contextual_sparsity_decoding_amd.build`")
        lib = ctypes.CDLL(_SYNTH_LIB)
        u64, u32p = ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint32)
        lib.synth_philox_block.argtypes = [u32p, u32p, u32p]
        lib.synth_philox_words.argtypes = [u32p, u64, u64, u64, u64, ctypes.c_int]
        lib.synth_philox_normal.argtypes = [ctypes.POINTER(ctypes.c_float), u64, u64, u64, u64, ctypes.c_float,
                                            ctypes.c_float, ctypes.c_int]
        _synth = lib
    return _synth


def philox_block(counter, key) -> np.ndarray:
    """Philox-4x32-10 of one counter (4 words) under one key (2 words)."""
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.empty(4, np.uint32)
    p = ctypes.POINTER(ctypes.c_uint32)
    _lib().synth_philox_block(c.ctypes.data_as(p), k.ctypes.data_as(p), out.ctypes.data_as(p))
    return out


def stream_id(layer: int, tensor: str | int) -> int:
    """Stream of one tensor of one layer under a workload seed."""
    tid = _TENSOR_IDS[tensor] if isinstance(tensor, str) else int(tensor)
    return (int(layer) << 16) | tid


def philox_words(n: int, seed: int, stream: int, offset: int = 0) -> np.ndarray:
    out = np.empty(int(n), np.uint32)
    _lib().synth_philox_words(out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)), int(n), int(offset), int(seed),
                              int(stream), _threads())
    return out


def philox_normal(n: int, seed: int, stream: int, offset: int = 0, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """Elements [offset, offset + n) of the normal stream, fp32."""
    out = np.empty(int(n), np.float32)
    _lib().synth_philox_normal(out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), int(n), int(offset), int(seed),
                               int(stream), float(mean), float(std), _threads())
    return out


def philox_tensor(shape: Sequence[int], seed: int, layer: int, tensor: str, std: float = 1.0,
                  dtype=np.float32) -> np.ndarray:
    """The host copy of what dv_fill_normal writes for (seed, layer, tensor)."""
    n = int(np.prod(shape)) if len(shape) else 1
    a = philox_normal(n, seed, stream_id(layer, tensor), 0, 0.0, std).reshape(shape)
    return _to_f16(a) if dtype == np.float16 else a


# Shapes of one decoder layer's generated tensors (storage layouts above);
# LayerNorm gain and bias are the constants 1 and 0.
def stack_tensor_shapes(dims: LayerDims) -> Dict[str, tuple]:
    d, h, dh, N = dims.d, dims.h, dims.d_h, dims.N
    return {
        "w_qkv_t": (3, h, dh, d), "b_qkv": (3, h, dh), "w_o_t": (h * dh, d), "b_o": (d,),
        "w1_t": (N, d), "b1": (N,), "w2_t": (N, d), "b2": (d,),
        "pa1_t": (dims.r_attn, d), "pa2_t": (h, dims.r_attn), "pm1_t": (dims.r_mlp, d), "pm2_t": (N, dims.r_mlp),
    }


def stack_layer_weights(dims: LayerDims, seed: int, layer: int, names: Sequence[str] | None = None) -> Dict[str, np.ndarray]:
    """Host copy of one generated stack layer's weights (all, or ``names``)."""
    wd = _wdt(dims)
    shapes = stack_tensor_shapes(dims)
    out = {}
    for k in (names if names is not None else list(shapes) + ["ln1_g", "ln1_b", "ln2_g", "ln2_b"]):
        if k in shapes:
            out[k] = philox_tensor(shapes[k], seed, layer, k, WEIGHT_STD, wd)
        elif k.endswith("_g"):
            out[k] = np.ones(dims.d, np.float32)
        else:
            out[k] = np.zeros(dims.d, np.float32)
    return out
