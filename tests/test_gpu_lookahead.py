"""Parity of dv_decode_layer with DV_LOOKAHEAD (DejaVu §4.3, the parallel
form) against the oracle's decode_layer_lookahead (GPU): the layer runs with
given sets while the next layer's predictors read its normalised input,
either on a second stream or as extra workgroups of the layer's own
launches; also inside captured HIP graphs."""
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


def _sync_objects():
    """An auxiliary stream and two events whose handles exist (torch creates
    events on first record)."""
    aux = torch.cuda.Stream()
    evs = [torch.cuda.Event(), torch.cuda.Event()]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    return aux, evs


class Ahead:
    """One layer's device and oracle state, the next layer's predictors, and
    the index buffers that carry sets from one step to the next."""

    def __init__(self, dv, dims: LayerDims, n0: int, max_len: int, seed: int, k_heads: int, k_neurons: int):
        self.dv, self.dims, self.k_h, self.k_m, self.max_len = dv, dims, k_heads, k_neurons, max_len
        self.W = synth.layer_weights(dims, seed)
        self.Wn = synth.layer_weights(dims, seed + 1000)
        K, V = synth.kv_cache(dims.h, dims.d_h, n0, max_len, seed)
        self.okv = ref.KVState(K.copy(), V.copy(), np.zeros((1, max_len, dims.d)), np.full((1, dims.h), n0 - 1))
        self.Wd, self.Wnd = upload(self.W), upload(self.Wn)
        self.K, self.V = dev(K), dev(V)
        self.y_buf = torch.zeros(1, max_len, dims.d, device="cuda")
        self.valid = dev(np.full((1, dims.h), n0 - 1, np.int32))
        self.wts = dv.layer_weights(self.Wd)

    def cfg(self, flags):
        d = self.dims
        return self.dv.decode_cfg(B=1, d=d.d, h=d.h, d_h=d.d_h, N=d.N, r_attn=d.r_attn, r_mlp=d.r_mlp,
                                  k_heads=self.k_h, k_neurons=self.k_m, wdt=self.dv.DV_F16, pred_act=self.dv.DV_ACT_RELU,
                                  eps=1e-5, scale=1 / math.sqrt(d.d_h), flags=flags)

    def state(self, pos, hi_in, ni_in, hi_next, ni_next, sync=None, pos_dev=None, max_pos=None):
        dv = self.dv
        st = dv.LayerState()
        st.kv = dv.kv_state(self.K, self.V, pos if max_pos is None else max_pos, self.y_buf, self.valid, pos_dev)
        st.head_idx_in, st.neuron_idx_in = hi_in.data_ptr(), ni_in.data_ptr()
        st.next_pa1_t, st.next_pa2_t = self.Wnd["pa1_t"].data_ptr(), self.Wnd["pa2_t"].data_ptr()
        st.next_pm1_t, st.next_pm2_t = self.Wnd["pm1_t"].data_ptr(), self.Wnd["pm2_t"].data_ptr()
        st.next_head_idx, st.next_neuron_idx = hi_next.data_ptr(), ni_next.data_ptr()
        if sync is not None:
            aux, evs = sync
            st.aux_stream, st.ev_fork, st.ev_join = aux.cuda_stream, evs[0].cuda_event, evs[1].cuda_event
        return st

    def oracle(self, x, pos, hi, ni):
        return ref.decode_layer_lookahead(x, self.W, self.Wn, self.okv, pos, head_idx=hi, neuron_idx=ni,
                                          k_heads=self.k_h, k_neurons=self.k_m, scale=1 / math.sqrt(self.dims.d_h))


def _run_steps(dvlib, A: Ahead, n0, X, sync):
    """Eager steps: each step's predicted sets feed the next step."""
    flags = dvlib.DV_LOOKAHEAD | dvlib.DV_HOLE_FILL | dvlib.DV_SKIP_NONPOS_FC2
    cfg = A.cfg(flags)
    ws = dvlib.workspace(dvlib.dv_decode_workspace_bytes(cfg, A.max_len))
    g = np.random.default_rng(7)
    hi = np.sort(g.choice(A.dims.h, A.k_h, replace=False)).astype(np.int32)
    ni = np.sort(g.choice(A.dims.N, A.k_m, replace=False)).astype(np.int32)
    checked = 0
    for t in range(len(X)):
        hi_d, ni_d = dev(hi), dev(ni)
        hn = torch.full((A.k_h,), -1, dtype=torch.int32, device="cuda")
        nn = torch.full((A.k_m,), -1, dtype=torch.int32, device="cuda")
        out = torch.empty(1, A.dims.d, device="cuda")
        st = A.state(n0 + t, hi_d, ni_d, hn, nn, sync)
        dvlib.dv_decode_layer(A.wts, cfg, st, dev(X[t]), out, ws)
        torch.cuda.synchronize()
        want, rec = A.oracle(X[t], n0 + t, hi, ni)
        e = check_close(host(out), want, "f16", f"look-ahead step {t}")
        ok_h = selection_margin(rec["next_head_scores"][0], A.k_h) > MARGIN
        ok_n = selection_margin(rec["next_neuron_scores"][0], A.k_m) > MARGIN
        if ok_h:
            assert np.array_equal(host(hn), rec["next_head_idx"]), f"step {t}: next heads"
        if ok_n:
            assert np.array_equal(host(nn), rec["next_neuron_idx"]), f"step {t}: next neurons"
        if not (ok_h and ok_n):
            break                      # the two sides would continue on different sets
        checked += 1
        hi, ni = rec["next_head_idx"].astype(np.int32), rec["next_neuron_idx"].astype(np.int32)
        print(f"look-ahead step {t}: normwise {e:.2e}")
    return checked


@pytest.mark.parametrize("aux", [True, False])
def test_lookahead_steps_match_oracle(dvlib, aux):
    dims = LayerDims(d=1024, N=4096, h=8, d_h=128, r_attn=32, r_mlp=64, wdt="f16")
    n0, T = 30, 4
    A = Ahead(dvlib, dims, n0, n0 + T + 2, seed=41, k_heads=3, k_neurons=400)
    X = synth.layer_inputs(dims.d, T, 1, seed=41)
    checked = _run_steps(dvlib, A, n0, X, _sync_objects() if aux else None)
    assert checked == T
    assert np.array_equal(host(A.valid), A.okv.valid_upto)
    ok_k, nk = f16_kv_ok(host(A.K), A.okv.K)
    ok_v, nv = f16_kv_ok(host(A.V), A.okv.V)
    assert ok_k and ok_v, f"K entries off: {nk}, V entries off: {nv}"


@pytest.mark.parametrize("N,k_m", [(24576, 2400), (1000, 100), (4100, 4100), (2048, 1)])
def test_lookahead_selection_shapes(dvlib, N, k_m):
    """The neuron selection of the single-stream schedule at budgets its
    split form does not take (more than 20480 scores; a count that is not a
    multiple of 4), at k = n (every neuron kept) and at k = 1: the same sets
    as the oracle either way."""
    dims = LayerDims(d=512, N=N, h=8, d_h=64, r_attn=16, r_mlp=32, wdt="f16")
    n0, T = 12, 2
    A = Ahead(dvlib, dims, n0, n0 + T + 2, seed=47, k_heads=3, k_neurons=k_m)
    X = synth.layer_inputs(dims.d, T, 1, seed=47)
    assert _run_steps(dvlib, A, n0, X, None) == T


@pytest.mark.parametrize("protos", [1, 5])
def test_lookahead_selection_ties(dvlib, protos):
    """Exact ties among the next layer's neuron scores: the rows of its second
    predictor layer repeat `protos` distinct rows, so equal scores are equal on
    both sides.  The selection split over the layer's launches must take the
    lower indices among equal scores at the threshold, as the oracle does,
    also across its 1024-score slices."""
    dims = LayerDims(d=512, N=4096, h=8, d_h=64, r_attn=16, r_mlp=32, wdt="f16")
    n0, k_h, k_m = 12, 3, 1000
    A = Ahead(dvlib, dims, n0, n0 + 3, seed=49, k_heads=k_h, k_neurons=k_m)
    A.Wn["pm2_t"] = A.Wn["pm2_t"][:protos].copy()[np.arange(dims.N) % protos]
    A.Wnd = upload(A.Wn)
    X = synth.layer_inputs(dims.d, 1, 1, seed=49)
    cfg = A.cfg(dvlib.DV_LOOKAHEAD | dvlib.DV_HOLE_FILL | dvlib.DV_SKIP_NONPOS_FC2)
    ws = dvlib.workspace(dvlib.dv_decode_workspace_bytes(cfg, A.max_len))
    g = np.random.default_rng(7)
    hi = np.sort(g.choice(dims.h, k_h, replace=False)).astype(np.int32)
    ni = np.sort(g.choice(dims.N, k_m, replace=False)).astype(np.int32)
    hn = torch.full((k_h,), -1, dtype=torch.int32, device="cuda")
    nn = torch.full((k_m,), -1, dtype=torch.int32, device="cuda")
    out = torch.empty(1, dims.d, device="cuda")
    hi_d, ni_d, x_d = dev(hi), dev(ni), dev(X[0])     # alive until the launches have run
    st = A.state(n0, hi_d, ni_d, hn, nn)
    dvlib.dv_decode_layer(A.wts, cfg, st, x_d, out, ws)
    torch.cuda.synchronize()
    want, rec = A.oracle(X[0], n0, hi, ni)
    check_close(host(out), want, "f16", "tied selection step")
    vals = np.unique(rec["next_neuron_scores"][0])
    assert vals.size == protos
    if protos > 1:
        assert np.min(np.diff(vals)) > MARGIN
    assert np.array_equal(host(nn), rec["next_neuron_idx"])


@pytest.mark.parametrize("aux", [True, False])
def test_lookahead_opt13b_layer_full_size(dvlib, aux):
    """The OPT-13B-shaped layer in the parallel form: 20 given heads, 2048
    given neurons, the next layer's 20 heads and 2048 neurons predicted
    alongside (on a second stream, or inside the layer's launches)."""
    w = configs.OPT13B_LAYER
    A = Ahead(dvlib, w.dims, w.n_ctx, w.n_ctx + 4, seed=43, k_heads=w.k_heads, k_neurons=w.k_neurons)
    X = synth.layer_inputs(w.dims.d, 2, 1, seed=43)
    assert _run_steps(dvlib, A, w.n_ctx, X, _sync_objects() if aux else None) == 2


@pytest.mark.parametrize("aux", [True, False])
def test_lookahead_graph(dvlib, aux):
    """T steps captured in one HIP graph, the predictions on a second stream
    (a fork and a join per step) or inside the layer's launches, the position
    on the device: replayed with eager work in between, every replay equals
    the eager steps."""
    dims = LayerDims(d=512, N=2048, h=8, d_h=64, r_attn=16, r_mlp=32, wdt="f16")
    n0, T, L = 20, 5, 40
    k_h, k_m = 3, 200
    flags = dvlib.DV_LOOKAHEAD | dvlib.DV_HOLE_FILL | dvlib.DV_SKIP_NONPOS_FC2
    eager = Ahead(dvlib, dims, n0, L, seed=45, k_heads=k_h, k_neurons=k_m)
    graph = Ahead(dvlib, dims, n0, L, seed=45, k_heads=k_h, k_neurons=k_m)
    X = synth.layer_inputs(dims.d, T, 1, seed=45)
    g0 = np.random.default_rng(9)
    hi0 = np.sort(g0.choice(dims.h, k_h, replace=False)).astype(np.int32)
    ni0 = np.sort(g0.choice(dims.N, k_m, replace=False)).astype(np.int32)
    # eager reference: sets carried step to step
    cfg = eager.cfg(flags)
    ws_e = dvlib.workspace(dvlib.dv_decode_workspace_bytes(cfg, L))
    hi_b = [dev(hi0), torch.empty(k_h, dtype=torch.int32, device="cuda")]
    ni_b = [dev(ni0), torch.empty(k_m, dtype=torch.int32, device="cuda")]
    want = []
    for t in range(T):
        out = torch.empty(1, dims.d, device="cuda")
        st = eager.state(n0 + t, hi_b[t % 2], ni_b[t % 2], hi_b[(t + 1) % 2], ni_b[(t + 1) % 2])
        dvlib.dv_decode_layer(eager.wts, cfg, st, dev(X[t]), out, ws_e)
        want.append(host(out))
    # graph: one step captured, ping-pong buffers swapped between two captured steps
    sync = _sync_objects() if aux else None
    pos_dev = torch.full((1,), n0, dtype=torch.int32, device="cuda")
    cfg_g = graph.cfg(flags | dvlib.DV_ADVANCE_POS)
    ws_g = dvlib.workspace(dvlib.dv_decode_workspace_bytes(cfg_g, L))
    hg = [dev(hi0), torch.empty(k_h, dtype=torch.int32, device="cuda")]
    ng = [dev(ni0), torch.empty(k_m, dtype=torch.int32, device="cuda")]
    x_in = [torch.zeros(1, dims.d, device="cuda") for _ in range(2)]
    outs = [torch.zeros(1, dims.d, device="cuda") for _ in range(2)]
    states = [graph.state(0, hg[p], ng[p], hg[1 - p], ng[1 - p], sync, pos_dev, L - 1) for p in range(2)]
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for p in range(2):
            dvlib.dv_decode_layer(graph.wts, cfg_g, states[p], x_in[p], outs[p], ws_g)
    replays = 0
    for t0 in range(0, T - 1, 2):
        replays += 1
        for p in range(2):
            x_in[p].copy_(dev(X[t0 + p]))
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for p in range(2):
            e = normwise(host(outs[p]), want[t0 + p])
            assert e < 1e-5, f"replay step {t0 + p}: normwise {e:.2e}"
    assert int(host(pos_dev)[0]) == n0 + 2 * replays


@pytest.mark.parametrize("d,N,k_m", [(1024, 4096, 400), (4096, 16384, 1638)])
def test_lookahead_neuron_predictor_alone(dvlib, d, N, k_m):
    """Every head (no head predictor) and the neuron set predicted one layer
    ahead: the neuron predictor alone rides in the layer's launches."""
    dims = LayerDims(d=d, N=N, h=8, d_h=128, r_attn=32, r_mlp=64, wdt="f16")
    n0, T = 30, 3
    A = Ahead(dvlib, dims, n0, n0 + T + 2, seed=43, k_heads=dims.h, k_neurons=k_m)
    X = synth.layer_inputs(dims.d, T, 1, seed=43)
    flags = dvlib.DV_LOOKAHEAD | dvlib.DV_DENSE_ATTN | dvlib.DV_SKIP_NONPOS_FC2
    cfg = A.cfg(flags)
    ws = dvlib.workspace(dvlib.dv_decode_workspace_bytes(cfg, A.max_len))
    g = np.random.default_rng(8)
    ni = np.sort(g.choice(N, k_m, replace=False)).astype(np.int32)
    dummy = torch.zeros(dims.h, dtype=torch.int32, device="cuda")
    for t in range(T):
        ni_d = dev(ni)
        nn = torch.full((k_m,), -1, dtype=torch.int32, device="cuda")
        out = torch.empty(1, dims.d, device="cuda")
        st = A.state(n0 + t, dummy, ni_d, dummy, nn)
        st.next_pa1_t = st.next_pa2_t = 0                      # no head predictor
        dvlib.dv_decode_layer(A.wts, cfg, st, dev(X[t]), out, ws)
        torch.cuda.synchronize()
        want, rec = ref.decode_layer_lookahead(X[t], A.W, A.Wn, A.okv, n0 + t, head_idx=None, neuron_idx=ni,
                                               k_heads=dims.h, k_neurons=k_m, scale=1 / math.sqrt(dims.d_h))
        e = check_close(host(out), want, "f16", f"neuron-only look-ahead step {t}")
        if selection_margin(rec["next_neuron_scores"][0], k_m) <= MARGIN:
            break
        assert np.array_equal(host(nn), rec["next_neuron_idx"]), f"step {t}: next neurons"
        ni = rec["next_neuron_idx"].astype(np.int32)
        print(f"neuron-only look-ahead step {t}: normwise {e:.2e}")
