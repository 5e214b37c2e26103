"""dv_sparse_mlp_noalloc (the entry point that allocates nothing) against
dv_sparse_mlp on the same inputs, through the C ABI (GPU): two calls in a
row, the second smaller, so the built-in scratch keeps the first call's
contents when the second runs."""
import numpy as np
import pytest
import torch

from contextual_sparsity_decoding_amd import synth
from contextual_sparsity_decoding_amd.configs import LayerDims
from tests.gpu_helpers import dev, host

pytestmark = pytest.mark.gpu


def _case(dims, k, seed, B=1):
    W = synth.mlp_weights(dims, seed)
    g = np.random.default_rng(seed)
    idx = np.sort(g.choice(dims.N, k, replace=False)).astype(np.int32)
    y = synth.normal((B, dims.d), seed, 0, "x")
    res = synth.normal((B, dims.d), seed, 1, "x")
    return {k_: dev(v) for k_, v in W.items()}, dev(idx), dev(y), dev(res)


def _run(dv, Wd, idx, y, res, k, noalloc):
    B, d = y.shape
    out = torch.full((B, d), float("nan"), device="cuda")
    act = torch.full((B, k), float("nan"), device="cuda")
    rows = torch.zeros(1, dtype=torch.int32, device="cuda")
    kw = dict(residual=res, act_out=act, fc2_rows=rows, flags=dv.DV_SKIP_NONPOS_FC2)
    if noalloc:
        dv.dv_sparse_mlp_noalloc(y, Wd["w1_t"], Wd["b1"], Wd["w2_t"], Wd["b2"], idx, k, out, **kw)
    else:
        ws = dv.workspace(dv.dv_sparse_mlp_workspace_bytes(B, d, k, dv.wdt_of(Wd["w1_t"])))
        dv.dv_sparse_mlp(y, Wd["w1_t"], Wd["b1"], Wd["w2_t"], Wd["b2"], idx, k, out, ws, **kw)
    return host(out), host(act), int(host(rows)[0])


def test_noalloc_matches_the_workspace_entry_point(dvlib):
    # OPT-66B width at 10% of neurons, then a smaller layer and batch
    cases = [(LayerDims(d=9216, N=36864, h=0, r_mlp=128, wdt="f16"), 3686, 11, 1),
             (LayerDims(d=1024, N=4096, h=0, r_mlp=32, wdt="f16"), 300, 12, 2)]
    prepared = [_case(dims, k, seed, B) + (k,) for dims, k, seed, B in cases]
    for Wd, idx, y, res, k in prepared:
        assert dvlib.dv_sparse_mlp_workspace_bytes(y.shape[0], y.shape[1], k, dvlib.DV_F16) <= dvlib.NOALLOC_SCRATCH_BYTES
        got = _run(dvlib, Wd, idx, y, res, k, noalloc=True)
        want = _run(dvlib, Wd, idx, y, res, k, noalloc=False)
        # the same kernels in the same order: bit for bit
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1]) and got[2] == want[2]
        assert np.isfinite(got[0]).all() and got[2] > 0


def test_noalloc_refuses_shapes_past_its_scratch(dvlib):
    """A batch of 16 over every neuron of an OPT-66B-shaped layer needs about
    21 MB of scratch: refused before anything is enqueued."""
    t = torch.zeros(1 << 16, device="cuda")
    p = t.data_ptr()
    st = dvlib.lib.dv_sparse_mlp_noalloc(p, 16, 9216, 36864, p, p, p, p, dvlib.DV_F16, p, 36864, 0, 0, p + 4096,
                                         0, 0, 0, 0)
    assert st == 6 and "scratch" in dvlib.lib.dv_last_error().decode()
