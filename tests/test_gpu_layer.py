"""Parity of dv_decode_layer with the oracle's decode_layer (GPU), including
the full OPT-13B-shaped layer in the configuration bench.py times.

Selected sets are compared where they are unique: when the gap between the
k-th and (k+1)-th oracle score exceeds the fp32 score error, the GPU's set
must equal the oracle's exactly (it then decides every later value too)."""
import math

import numpy as np
import pytest
import torch

from contextual_sparsity_decoding_amd import configs, synth
from contextual_sparsity_decoding_amd.configs import LayerDims
from oracle import ref
from tests.gpu_helpers import check_close, dev, f16_kv_ok, host, normwise, selection_margin, upload

pytestmark = pytest.mark.gpu

MARGIN = 1e-6


class Layer:
    """One layer's weights and decode state on the device and in the oracle."""

    def __init__(self, dvlib, dims: LayerDims, n0: int, max_len: int, seed: int, B: int = 1):
        self.dv, self.dims, self.B = dvlib, dims, B
        self.W = synth.layer_weights(dims, seed)
        K, V = synth.kv_cache(dims.h, dims.d_h, n0, max_len, seed, batch=B)
        self.okv = ref.KVState(K.copy(), V.copy(), np.zeros((B, max_len, dims.d)), np.full((B, dims.h), n0 - 1))
        self.Wd = upload(self.W)
        self.K, self.V = dev(K), dev(V)
        self.y_buf = torch.zeros(B, max_len, dims.d, device="cuda")
        self.valid = dev(np.full((B, dims.h), n0 - 1, np.int32))
        self.max_len = max_len

    def cfg(self, k_heads, k_neurons, flags):
        d = self.dims
        return self.dv.decode_cfg(B=self.B, d=d.d, h=d.h, d_h=d.d_h, N=d.N, r_attn=d.r_attn, r_mlp=d.r_mlp,
                                  k_heads=k_heads, k_neurons=k_neurons, wdt=self.dv.DV_F16 if d.wdt == "f16" else 0,
                                  pred_act=self.dv.DV_ACT_RELU, eps=1e-5, scale=1 / math.sqrt(d.d_h), flags=flags)

    def step(self, x, pos, k_heads, k_neurons, flags, sel=None):
        dv = self.dv
        cfg = self.cfg(k_heads, k_neurons, flags)
        st = dv.LayerState()
        st.kv = dv.kv_state(self.K, self.V, pos, self.y_buf, self.valid)
        hi = torch.full((max(1, k_heads),), -1, dtype=torch.int32, device="cuda")
        nmax = min(self.dims.N, self.B * max(1, k_neurons))
        ni = torch.full((nmax,), -1, dtype=torch.int32, device="cuda")
        nc = torch.zeros(1, dtype=torch.int32, device="cuda")
        rows = torch.zeros(1, dtype=torch.int32, device="cuda")
        st.head_idx_out, st.neuron_idx_out, st.neuron_count_out, st.fc2_rows_out = (
            hi.data_ptr(), ni.data_ptr(), nc.data_ptr(), rows.data_ptr())
        keep = []
        if sel is not None:
            sidx, slen, send = dev(sel[0]), dev(sel[1]), sel[2]
            keep += [sidx, slen]
            st.sel_idx, st.sel_len, st.sel_cap, st.sel_end = sidx.data_ptr(), slen.data_ptr(), sel[0].shape[-1], send
        ws = dv.workspace(dv.dv_decode_workspace_bytes(cfg, self.max_len))
        out = torch.empty(self.B, self.dims.d, device="cuda")
        dv.dv_decode_layer(dv.layer_weights(self.Wd), cfg, st, dev(x), out, ws)
        return host(out), host(hi), host(ni)[:int(host(nc)[0])], int(host(rows)[0])

    def oracle(self, x, pos, k_heads, k_neurons, flags, sel=None):
        dv = self.dv
        kw = {}
        if sel is not None:
            kw = dict(sel_idx=sel[0], sel_len=sel[1], sel_end=sel[2])
        return ref.decode_layer(x, self.W, self.okv, pos, k_heads=k_heads, k_neurons=k_neurons,
                                scale=1 / math.sqrt(self.dims.d_h), dense_attn=bool(flags & dv.DV_DENSE_ATTN),
                                dense_mlp=bool(flags & dv.DV_DENSE_MLP),
                                skip_nonpos=bool(flags & dv.DV_SKIP_NONPOS_FC2),
                                hole_fill=bool(flags & dv.DV_HOLE_FILL), **kw)


def _compare_step(L, got, want, rec, k_heads, k_neurons, flags, what):
    dv = L.dv
    out, hi, ni, rows = got
    unique = True
    if not flags & dv.DV_DENSE_ATTN:
        if selection_margin(rec["head_scores"][0], k_heads) > MARGIN:
            assert np.array_equal(hi[:k_heads], rec["head_idx"]), f"{what}: head set"
        else:
            unique = False
    if not flags & dv.DV_DENSE_MLP and L.B == 1:
        if selection_margin(rec["neuron_scores"][0], k_neurons) > MARGIN:
            assert np.array_equal(ni, rec["neuron_idx"]), f"{what}: neuron set"
        else:
            unique = False
    if unique:
        e = check_close(out, want, L.dims.wdt, what)
        if flags & dv.DV_SKIP_NONPOS_FC2 and not flags & dv.DV_DENSE_MLP:
            assert rows == int(np.sum(np.any(rec["a"] > 0, axis=0)))
        return e
    return None


def test_opt13b_layer_full_size(dvlib):
    """One OPT-13B-shaped layer, 2048 cached tokens, 20 of 40 heads, 2048 of
    20480 neurons: the launch configuration the benchmark times."""
    w = configs.OPT13B_LAYER
    L = Layer(dvlib, w.dims, w.n_ctx, w.n_ctx + 8, seed=1)
    x = synth.layer_inputs(w.dims.d, 1, 1, seed=1)[0]
    flags = dvlib.DV_HOLE_FILL | dvlib.DV_SKIP_NONPOS_FC2
    got = L.step(x, w.n_ctx, w.k_heads, w.k_neurons, flags)
    want, rec = L.oracle(x, w.n_ctx, w.k_heads, w.k_neurons, flags)
    e = _compare_step(L, got, want, rec, w.k_heads, w.k_neurons, flags, "opt13b sparse")
    assert e is not None, "choose a seed whose selections are unique"
    print(f"opt13b sparse layer normwise error {e:.2e}")
    ok, nbad = f16_kv_ok(host(L.K)[0, :, w.n_ctx], L.okv.K[0, :, w.n_ctx])
    assert ok, f"{nbad} appended K entries off"


def test_opt13b_layer_dense_path(dvlib):
    w = configs.OPT13B_LAYER
    L = Layer(dvlib, w.dims, w.n_ctx, w.n_ctx + 8, seed=2)
    x = synth.layer_inputs(w.dims.d, 1, 1, seed=2)[0]
    flags = dvlib.DV_DENSE_ATTN | dvlib.DV_DENSE_MLP | dvlib.DV_HOLE_FILL
    got = L.step(x, w.n_ctx, w.dims.h, w.dims.N, flags)
    want, rec = L.oracle(x, w.n_ctx, w.dims.h, w.dims.N, flags)
    e = _compare_step(L, got, want, rec, w.dims.h, w.dims.N, flags, "opt13b dense")
    print(f"opt13b dense layer normwise error {e:.2e}")


def test_multistep_decode_with_holes(dvlib):
    dims = LayerDims(d=512, N=2048, h=8, d_h=64, r_attn=16, r_mlp=32, wdt="f16")
    n0, T = 20, 7
    L = Layer(dvlib, dims, n0, 40, seed=3)
    X = synth.layer_inputs(dims.d, T, 1, seed=3)
    flags = dvlib.DV_HOLE_FILL | dvlib.DV_SKIP_NONPOS_FC2
    checked = 0
    for t in range(T):
        got = L.step(X[t], n0 + t, 3, 200, flags)
        want, rec = L.oracle(X[t], n0 + t, 3, 200, flags)
        if _compare_step(L, got, want, rec, 3, 200, flags, f"step {t}") is not None:
            checked += 1
        # keep both sides on the same head sets: stop if they diverge
        if not np.array_equal(got[1][:3], rec["head_idx"]):
            break
    assert checked >= T - 1
    assert np.array_equal(host(L.valid), L.okv.valid_upto)
    ok_k, nk = f16_kv_ok(host(L.K), L.okv.K)
    ok_v, nv = f16_kv_ok(host(L.V), L.okv.V)
    assert ok_k and ok_v, f"K entries off: {nk}, V entries off: {nv}"


def test_batch_union_decode(dvlib):
    dims = LayerDims(d=512, N=2048, h=8, d_h=64, r_attn=16, r_mlp=32, wdt="f16")
    B = 3
    L = Layer(dvlib, dims, 30, 36, seed=4, B=B)
    x = synth.layer_inputs(dims.d, 1, B, seed=4)[0]
    flags = dvlib.DV_DENSE_ATTN | dvlib.DV_HOLE_FILL | dvlib.DV_SKIP_NONPOS_FC2
    out, _, ni, rows = L.step(x, 30, 8, 150, flags)
    want, rec = L.oracle(x, 30, 8, 150, flags)
    margins = [selection_margin(rec["neuron_scores"][b], 150) for b in range(B)]
    assert min(margins) > MARGIN
    assert np.array_equal(ni, rec["neuron_idx"])
    assert 150 < len(ni) < B * 150
    check_close(out, want, "f16", "batch union")
    assert rows == int(np.sum(np.any(rec["a"] > 0, axis=0)))


@pytest.mark.parametrize("B", [8, 13, 16])
def test_batch_union_decode_matrix_cores(dvlib, B):
    """Batches of 8-16 with every head (no stored inputs): Q/K/V and fc1 run
    on the matrix cores; every sequence's output, K/V entry and the union
    against the oracle."""
    from tests.test_gpu_stack import _union_follow
    dims = LayerDims(d=1024, N=4096, h=8, d_h=128, r_attn=16, r_mlp=32, wdt="f16")
    L = Layer(dvlib, dims, 30, 36, seed=40 + B, B=B)
    x = synth.layer_inputs(dims.d, 1, B, seed=40 + B)[0]
    flags = dvlib.DV_DENSE_ATTN | dvlib.DV_SKIP_NONPOS_FC2
    out, _, ni, rows = L.step(x, 30, 8, 300, flags)
    want, rec = L.oracle(x, 30, 8, 300, flags)
    used = _union_follow(ni, rec, 300, f"batch {B}")
    if used is not rec["neuron_idx"]:
        want, _ = ref.sparse_mlp(rec["y2"], L.W["w1_t"], L.W["b1"], L.W["w2_t"], L.W["b2"], used,
                                 residual=rec["h"], skip_nonpos=True)
    e = check_close(out, want, "f16", f"batch {B}")
    ok_k, nk = f16_kv_ok(host(L.K), L.okv.K)
    ok_v, nv = f16_kv_ok(host(L.V), L.okv.V)
    assert ok_k and ok_v, f"K entries off: {nk}, V entries off: {nv}"
    print(f"batch {B}: |U| = {len(ni)}, normwise {e:.2e}")


def test_kv_selected_decode(dvlib):
    dims = LayerDims(d=512, N=2048, h=8, d_h=128, r_attn=16, r_mlp=32, wdt="f16")
    n, budget = 400, 100
    L = Layer(dvlib, dims, n, n + 4, seed=5)
    Q = synth.observation_queries(dims.h, 64, dims.d_h, seed=5)
    sel = np.zeros((1, dims.h, budget), np.int32)
    for i in range(dims.h):
        sel[0, i] = ref.kv_select(Q[0, i], L.okv.K[0, i], n, 1 / math.sqrt(dims.d_h), budget)[0]
    lens = np.full((1, dims.h), budget, np.int32)
    x = synth.layer_inputs(dims.d, 2, 1, seed=5)
    flags = dvlib.DV_HOLE_FILL | dvlib.DV_SKIP_NONPOS_FC2 | dvlib.DV_KV_SELECT
    for t in range(2):
        s = (sel, lens, n)
        got = L.step(x[t], n + t, 4, 300, flags, sel=s)
        want, rec = L.oracle(x[t], n + t, 4, 300, flags, sel=s)
        assert _compare_step(L, got, want, rec, 4, 300, flags, f"kv-select step {t}") is not None


def test_decode_is_deterministic(dvlib):
    dims = LayerDims(d=1024, N=4096, h=8, d_h=128, r_attn=16, r_mlp=32, wdt="f16")
    outs = []
    for _ in range(2):
        L = Layer(dvlib, dims, 64, 70, seed=6)
        x = synth.layer_inputs(dims.d, 1, 1, seed=6)[0]
        outs.append(L.step(x, 64, 4, 400, dvlib.DV_HOLE_FILL | dvlib.DV_SKIP_NONPOS_FC2)[0])
    assert np.array_equal(outs[0], outs[1])


def test_graph_replay_with_device_position(dvlib):
    """One decode step captured in a HIP graph with the position on the
    device (DV_ADVANCE_POS) and replayed step after step, with eager input
    copies and synchronisations in between, matches eager steps driven by
    host positions, replay by replay."""
    dims = LayerDims(d=512, N=2048, h=8, d_h=64, r_attn=16, r_mlp=32, wdt="f16")
    n0, T, L = 20, 6, 40
    eager = Layer(dvlib, dims, n0, L, seed=7)
    graph = Layer(dvlib, dims, n0, L, seed=7)
    X = synth.layer_inputs(dims.d, T, 1, seed=7)
    flags = dvlib.DV_HOLE_FILL | dvlib.DV_SKIP_NONPOS_FC2
    pos_dev = torch.full((1,), n0, dtype=torch.int32, device="cuda")
    cfg = graph.cfg(3, 200, flags | dvlib.DV_ADVANCE_POS)
    st = dvlib.LayerState()
    st.kv = dvlib.kv_state(graph.K, graph.V, L - 1, graph.y_buf, graph.valid, pos_dev)
    ws = dvlib.workspace(dvlib.dv_decode_workspace_bytes(cfg, L))
    wts = dvlib.layer_weights(graph.Wd)
    x_in = torch.zeros(1, dims.d, device="cuda")
    out = torch.zeros(1, dims.d, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dvlib.dv_decode_layer(wts, cfg, st, x_in, out, ws)
    for t in range(T):
        want = eager.step(X[t], n0 + t, 3, 200, flags)[0]
        x_in.copy_(dev(X[t]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = host(out)
        e = normwise(got, want)
        assert e < 1e-5, f"replay {t}: normwise {e:.2e}"
    assert int(host(pos_dev)[0]) == n0 + T
    assert np.array_equal(host(graph.valid), host(eager.valid))
    ok_k, nk = f16_kv_ok(host(graph.K), host(eager.K))
    ok_v, nv = f16_kv_ok(host(graph.V), host(eager.V))
    assert ok_k and ok_v, f"K entries off: {nk}, V entries off: {nv}"
