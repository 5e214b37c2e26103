"""The GPU tests' comparators reject the mistakes they exist to catch (CPU:
the mistakes are planted in the oracle's output)."""
import math

import numpy as np
import pytest

from contextual_sparsity_decoding_amd import synth
from contextual_sparsity_decoding_amd.configs import LayerDims
from oracle import ref
from tests.gpu_helpers import assert_selection_close, check_close


def _layer(dims, seed, drop_b2=False, drop_rows=0):
    W = synth.layer_weights(dims, seed)
    if drop_b2:
        W["b2"] = np.zeros_like(W["b2"])
    K, V = synth.kv_cache(dims.h, dims.d_h, 64, 66, seed)
    kv = ref.KVState(K, V, np.zeros((1, 66, dims.d)), np.full((1, dims.h), 63))
    x = synth.layer_inputs(dims.d, 1, 1, seed)[0]
    out, rec = ref.decode_layer(x, W, kv, 64, k_heads=4, k_neurons=400, scale=1 / math.sqrt(dims.d_h))
    if drop_rows:
        idx, a = rec["neuron_idx"], rec["a"][0]
        live = np.nonzero(a > 0)[0][:drop_rows]
        out = out - a[live][:, None].T @ W["w2_t"][idx[live]].astype(np.float64)
    return out


DIMS = LayerDims(d=1024, N=4096, h=8, d_h=128, r_attn=32, r_mlp=64, wdt="f16")


def test_fp16_comparator_rejects_a_dropped_b2():
    want = _layer(DIMS, 3)
    bad = _layer(DIMS, 3, drop_b2=True)
    assert np.abs(bad - want).max() / np.abs(want).max() < 2e-2      # the contract's bound alone misses it
    with pytest.raises(AssertionError):
        check_close(bad, want, "f16", "b2 dropped")
    check_close(want + 1e-7 * np.abs(want).max(), want, "f16", "rounding-sized error")


def test_fp16_comparator_rejects_missing_fc2_rows():
    want = _layer(DIMS, 4)
    with pytest.raises(AssertionError):
        check_close(_layer(DIMS, 4, drop_rows=3), want, "f16", "three fc2 rows missing")


def test_selection_comparator():
    s = np.array([5.0, 4.0, 3.0, 3.0 + 1e-9, 1.0, 0.0])
    assert assert_selection_close([0, 1, 3], [0, 1, 3], s, 3, 1e-6) == 0
    assert assert_selection_close([0, 1, 2], [0, 1, 3], s, 3, 1e-6) == 2      # a swap at the boundary
    with pytest.raises(AssertionError):
        assert_selection_close([0, 2, 3], [0, 1, 3], s, 3, 1e-6)             # 1 is far above the k-th score
    with pytest.raises(AssertionError):
        assert_selection_close([0, 1], [0, 1, 3], s, 3, 1e-6)
