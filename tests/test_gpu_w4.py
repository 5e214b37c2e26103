"""Parity of the 4-bit-weight sparse MLP (W4A16; DejaVu §5, Table 7) with
the oracle (GPU): the device quantizer's codes and scales bit for bit, and
dv_sparse_mlp_w4 against ref.sparse_mlp_w4 on the oracle's own quantization
of the same fp16 weights, at widths that span one to five 2048-column
slices, ragged row counts and the OPT-66B width."""
import numpy as np
import pytest
import torch

from contextual_sparsity_decoding_amd import synth
from contextual_sparsity_decoding_amd.configs import LayerDims
from oracle import ref
from tests.gpu_helpers import check_close, dev, host

pytestmark = pytest.mark.gpu


def quantize_on_device(dv, w_host):
    w = dev(w_host)
    rows, cols = w_host.shape
    q = torch.empty(rows, cols // 2, dtype=torch.uint8, device="cuda")
    s = torch.empty(rows, cols // 128, dtype=torch.float16, device="cuda")
    dv.dv_quantize_w4(w, q, s)
    return q, s


@pytest.mark.parametrize("rows,cols", [(37, 640), (5, 9216), (1, 128)])
def test_quantizer_bit_exact(dvlib, rows, cols):
    g = np.random.default_rng(rows + cols)
    w = (g.standard_normal((rows, cols)) * 0.02).astype(np.float16)
    w[0, :128] = 0                                            # a group of zeros
    if cols >= 256:                                           # exact ties at half a step
        s = 2.0 ** -8
        w[-1, 128:256] = (g.integers(-14, 15, 128) * 0.5 * s).astype(np.float16)
        w[-1, 128] = np.float16(7 * s)
    q, s_dev = quantize_on_device(dvlib, w)
    v, s_ref = ref.quantize_w4(w)
    assert np.array_equal(host(s_dev), s_ref)
    assert np.array_equal(host(q), ref.pack_w4(v))


W4_CASES = [
    # d, N, k: one partial slice; three slices; the OPT-66B width (4.5 slices) at 10%; every row
    (1024, 4096, 333),
    (5120, 20480, 2048),
    (9216, 36864, 3686),
    (512, 700, 700),
]


@pytest.mark.parametrize("skip", [False, True])
@pytest.mark.parametrize("d,N,k", W4_CASES)
def test_sparse_mlp_w4(dvlib, d, N, k, skip):
    dims = LayerDims(d=d, N=N, h=0, r_mlp=16, wdt="f16")
    W = synth.mlp_weights(dims, seed=d + k)
    y = synth.layer_inputs(d, 1, 1, seed=d + k)[0]
    res = synth.normal((1, d), 9, 0, "x")
    full = k == N
    idx = np.arange(N, dtype=np.int32) if full else \
        np.sort(np.random.default_rng(d).choice(N, k, replace=False)).astype(np.int32)
    q1, s1 = quantize_on_device(dvlib, W["w1_t"])
    q2, s2 = quantize_on_device(dvlib, W["w2_t"])
    out = torch.empty(1, d, device="cuda")
    a = torch.empty(1, k, device="cuda")
    rows = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = dvlib.workspace(dvlib.lib.dv_sparse_mlp_w4_workspace_bytes(d, k))
    dvlib.dv_sparse_mlp_w4(dev(y), N, q1, s1, dev(W["b1"]), q2, s2, dev(W["b2"]), None if full else dev(idx), out, ws,
                           n_idx_max=k, residual=dev(res), act_out=a, fc2_rows=rows,
                           flags=dvlib.DV_SKIP_NONPOS_FC2 if skip else 0)
    v1, r1 = ref.quantize_w4(W["w1_t"][idx])
    v2, r2 = ref.quantize_w4(W["w2_t"][idx])
    want, wa = ref.sparse_mlp_w4(y, v1, r1, W["b1"][idx], v2, r2, W["b2"], np.arange(k), residual=res,
                                 skip_nonpos=skip)
    check_close(host(out), want, "f16", "W4 out")
    check_close(host(a), wa, "f16", "W4 a")
    live = int(np.sum(wa > 0))
    near = int(np.sum(np.abs(wa) < 1e-6))                   # a sign decided within rounding
    assert abs(int(host(rows)[0]) - (live if skip else k)) <= (near if skip else 0)
    assert 0 < live < k


def test_sparse_mlp_w4_device_count(dvlib):
    """The count read at run time: rows past it are neither computed nor read."""
    d, N, k = 2048, 4096, 500
    dims = LayerDims(d=d, N=N, h=0, r_mlp=16, wdt="f16")
    W = synth.mlp_weights(dims, seed=77)
    y = synth.layer_inputs(d, 1, 1, seed=77)[0]
    idx = np.sort(np.random.default_rng(77).choice(N, k, replace=False)).astype(np.int32)
    q1, s1 = quantize_on_device(dvlib, W["w1_t"])
    q2, s2 = quantize_on_device(dvlib, W["w2_t"])
    n_dev = torch.tensor([300], dtype=torch.int32, device="cuda")
    out = torch.empty(1, d, device="cuda")
    rows = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = dvlib.workspace(dvlib.lib.dv_sparse_mlp_w4_workspace_bytes(d, k))
    dvlib.dv_sparse_mlp_w4(dev(y), N, q1, s1, dev(W["b1"]), q2, s2, dev(W["b2"]), dev(idx), out, ws, n_idx_max=k,
                           n_idx_dev=n_dev, fc2_rows=rows)
    sel = idx[:300]
    v1, r1 = ref.quantize_w4(W["w1_t"][sel])
    v2, r2 = ref.quantize_w4(W["w2_t"][sel])
    want, _ = ref.sparse_mlp_w4(y, v1, r1, W["b1"][sel], v2, r2, W["b2"], np.arange(300))
    check_close(host(out), want, "f16", "W4 out, device count")
    assert int(host(rows)[0]) == 300
