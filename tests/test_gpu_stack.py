"""The device generator and the layer stack (GPU).

* dv_fill_normal against the host side of the same generator
  (synth_philox.c, pinned to the generator's known-answer vectors);
* dv_decode_stack in DejaVu §4.3's parallel form against the oracle, chained
  over layers and tokens at a small shape, and at the full 64-layer
  OPT-66B-shaped stack on sampled layers and tokens (the oracle reruns
  layer l of token t from the state the device held before it: its input,
  the sets it was given, its KV cache, stored inputs and valid positions,
  with weights regenerated on the host from the same seeded streams).
"""
import math

import numpy as np
import pytest
import torch

from contextual_sparsity_decoding_amd import configs, synth
from contextual_sparsity_decoding_amd.configs import LayerDims
from oracle import ref
from tests.gpu_helpers import assert_selection_close, check_close, dev, f16_kv_ok, host, selection_margin

pytestmark = pytest.mark.gpu

MARGIN = 1e-6


# ---------------------------------------------------------------- generator --

@pytest.mark.parametrize("n,offset", [(10007, 0), (4096, 13), (1000, 4 * ((1 << 32) + 3))])
def test_fill_normal_matches_host_generator(dvlib, n, offset):
    seed, sid = (5 << 32) | 77, synth.stream_id(31, "w2_t")
    w = torch.empty(n, dtype=torch.int32, device="cuda")
    dvlib.dv_fill_normal(w, seed, sid, offset=offset, raw=True)
    want_w = synth.philox_words(n, seed, sid, offset)
    assert np.array_equal(host(w).view(np.uint32), want_w)
    f = torch.empty(n, device="cuda")
    dvlib.dv_fill_normal(f, seed, sid, offset=offset, std=0.02)
    want_f = synth.philox_normal(n, seed, sid, offset, std=0.02)
    got_f = host(f)
    # both sides evaluate log, cos and sin in double: the float results agree
    # to the last bit except where the two libraries' last double bits
    # straddle a float rounding boundary
    ulp = np.spacing(np.abs(want_f))
    assert np.all(np.abs(got_f - want_f) <= ulp)
    assert np.mean(got_f == want_f) > 0.9999
    h = torch.empty(n, dtype=torch.float16, device="cuda")
    dvlib.dv_fill_normal(h, seed, sid, offset=offset, std=0.02)
    assert np.sum(host(h) != want_f.astype(np.float16)) <= 1


def test_fill_normal_layout_of_a_tensor(dvlib):
    """A tensor is one stream in row-major order: element [i, j] is stream element i * cols + j."""
    t = torch.empty(3, 1, 40, 16, dtype=torch.float16, device="cuda")
    dvlib.dv_fill_normal(t, 9, synth.stream_id(2, "K"))
    want = synth.philox_tensor((3, 1, 40, 16), 9, 2, "K", 1.0, np.float16)
    assert np.sum(host(t) != want) <= 1


# ---------------------------------------------------------------- the stack --

class DeviceStack:
    """A Stack plus the buffers a look-ahead decode carries."""

    def __init__(self, dv, dims, L, n0, max_len, seed, k_heads, k_neurons, window=None, n_dense_prefix=0):
        from contextual_sparsity_decoding_amd.stack import Stack
        self.dv, self.dims, self.L, self.kA, self.kM = dv, dims, L, k_heads, k_neurons
        self.S = Stack(dims, L, n0, max_len, seed)
        flags = dv.DV_LOOKAHEAD | dv.DV_HOLE_FILL | dv.DV_SKIP_NONPOS_FC2 | dv.DV_ADVANCE_POS
        if window is not None:
            flags |= dv.DV_KV_WINDOW
        self.cfg = self.S.cfg(k_heads, k_neurons, flags, 1 / math.sqrt(dims.d_h))
        if window is not None:
            self.cfg.win_sink, self.cfg.win_len = window
        self.cfg.n_dense_prefix = n_dense_prefix
        self.ws = dv.workspace(dv.dv_stack_workspace_bytes(self.cfg, max_len))
        self.head_sets = torch.full((L, k_heads), -1, dtype=torch.int32, device="cuda")
        self.neuron_sets = torch.full((L, k_neurons), -1, dtype=torch.int32, device="cuda")
        self.x_trace = torch.empty(max(1, L - 1), 1, dims.d, device="cuda")
        self.x_out = torch.empty(1, dims.d, device="cuda")

    def token(self, x):
        self.dv.dv_decode_stack(self.S.layers_array(), self.cfg, x, self.x_out, self.ws, head_sets=self.head_sets,
                                neuron_sets=self.neuron_sets, x_trace=self.x_trace)


def _follow(got, want, scores, k, what):
    """The set the oracle continues with: the device's set must equal the
    oracle's bit for bit, except for swaps at the k-th score that fp32
    rounding of the scores allows (then the oracle follows the device's
    choice, so both sides keep computing the same thing)."""
    if np.array_equal(got, want):
        return want
    assert selection_margin(scores, k) <= MARGIN, f"{what}: sets differ with a clear margin"
    assert_selection_close(got, want, scores, k, MARGIN * max(1.0, float(np.abs(scores).max())), what)
    return np.asarray(got, np.int64)


@pytest.mark.parametrize("window,P", [(None, 0), ((4, 16), 0), (None, 1)])
def test_stack_chained_small(dvlib, window, P):
    """3 layers x 4 tokens: every layer's sets, output, K/V and valid
    positions follow the oracle's chain (layer l's input is layer l-1's
    output; its sets were predicted by layer l-1).  With ``window`` every
    layer reads its 4 sink and 16 most recent positions, a window that
    slides one position per token; with P = 1 layer 0 runs dense and
    predicts layer 1's sets."""
    dims = LayerDims(d=1024, N=4096, h=8, d_h=128, r_attn=32, r_mlp=64, wdt="f16")
    L, n0, T, kA, kM = 3, 40, 4, 3, 400
    seed = 17 + (window is not None) + 2 * P
    D = DeviceStack(dvlib, dims, L, n0, n0 + T + 2, seed, kA, kM, window, P)
    Ws = [synth.stack_layer_weights(dims, seed, l) for l in range(L)]
    kvs = []
    for l in range(L):
        K = synth.philox_tensor((1, dims.h, n0 + T + 2, dims.d_h), seed, l, "K", 1.0, np.float16)
        V = synth.philox_tensor((1, dims.h, n0 + T + 2, dims.d_h), seed, l, "V", 1.0, np.float16)
        kvs.append(ref.KVState(K, V, np.zeros((1, n0 + T + 2, dims.d)), np.full((1, dims.h), n0 - 1)))
    X = synth.philox_tensor((T, 1, dims.d), seed, 0, "x")
    scale = 1 / math.sqrt(dims.d_h)
    errs = []
    for t in range(T):
        D.token(dev(X[t]))
        got_h, got_n, got_x, got_tr = host(D.head_sets), host(D.neuron_sets), host(D.x_out), host(D.x_trace)
        heads = neurons = None
        if P == 0:
            heads, neurons, sA, sM = ref.predict_sets(X[t], Ws[0], kA, kM)
            heads = _follow(got_h[0], heads, sA[0], kA, f"token {t} layer 0 heads")
            neurons = _follow(got_n[0], neurons, sM[0], kM, f"token {t} layer 0 neurons")
        x = X[t]
        for l in range(L):
            Wn = Ws[l + 1] if l + 1 < L and l + 1 >= P else None
            x, rec = ref.decode_layer_lookahead(x, Ws[l], Wn, kvs[l], n0 + t, head_idx=heads, neuron_idx=neurons,
                                                k_heads=kA, k_neurons=kM, scale=scale, window=window)
            got = got_tr[l] if l + 1 < L else got_x
            errs.append(check_close(got, x, "f16", f"token {t} layer {l}"))
            if Wn is not None:
                heads = _follow(got_h[l + 1], rec["next_head_idx"], rec["next_head_scores"][0], kA,
                                f"token {t} layer {l + 1} heads")
                neurons = _follow(got_n[l + 1], rec["next_neuron_idx"], rec["next_neuron_scores"][0], kM,
                                  f"token {t} layer {l + 1} neurons")
    for l in range(L):
        assert np.array_equal(host(D.S.valid[l]), kvs[l].valid_upto)
        ok_k, nk = f16_kv_ok(host(D.S.K[l]), kvs[l].K)
        ok_v, nv = f16_kv_ok(host(D.S.V[l]), kvs[l].V)
        assert ok_k and ok_v, f"layer {l}: K entries off {nk}, V entries off {nv}"
    assert int(D.S.pos_dev.item()) == n0 + T           # moved on once per token, not once per layer
    print(f"chained stack: worst normwise {max(errs):.2e}")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_stack_opt66b_sampled_layers(dvlib):
    """The 64-layer OPT-66B-shaped stack (d = 9216, 72 heads, d_ffn = 36864,
    1024 cached tokens, 36 heads and 10% of neurons) decoding 128 tokens in the
    look-ahead form; layers {0, 31, 63} at tokens {0, 1, 127} rerun by the
    oracle from the state the device held before them."""
    wl = configs.OPT66B_STACK
    dims, L, n0, T, seed = wl.dims, wl.layers, wl.n_ctx, 128, 1234
    kA, kM = wl.k_heads, int(math.floor(0.10 * dims.N))
    max_len = n0 + T + 8
    layers, tokens = (0, 31, 63), (0, 1, 127)
    D = DeviceStack(dvlib, dims, L, n0, max_len, seed, kA, kM)
    X = torch.empty(T, 1, dims.d, device="cuda")
    dvlib.dv_fill_normal(X, seed, synth.stream_id(0, "x"))
    snaps = {}
    for t in range(T):
        if t in tokens:
            for l in layers:
                snaps[(l, t)] = {"K": host(D.S.K[l]), "V": host(D.S.V[l]), "y_buf": host(D.S.y_buf[l]),
                                 "valid": host(D.S.valid[l])}
        D.token(X[t])
        if t in tokens:
            hs, ns, tr, xo = host(D.head_sets), host(D.neuron_sets), host(D.x_trace), host(D.x_out)
            for l in layers:
                s = snaps[(l, t)]
                s.update(x_in=host(X[t]) if l == 0 else tr[l - 1], heads=hs[l], neurons=ns[l],
                         x_out=tr[l] if l + 1 < L else xo, next_heads=hs[l + 1] if l + 1 < L else None,
                         next_neurons=ns[l + 1] if l + 1 < L else None,
                         K_after=host(D.S.K[l]), V_after=host(D.S.V[l]), valid_after=host(D.S.valid[l]))
    torch.cuda.synchronize()
    del D
    torch.cuda.empty_cache()
    scale = 1 / math.sqrt(dims.d_h)
    for l in layers:
        W = synth.stack_layer_weights(dims, seed, l)
        Wn = synth.stack_layer_weights(dims, seed, l + 1, names=["pa1_t", "pa2_t", "pm1_t", "pm2_t"]) \
            if l + 1 < L else None
        for t in tokens:
            s = snaps[(l, t)]
            if l == 0:
                h0, n0_, sA, sM = ref.predict_sets(s["x_in"], W, kA, kM)
                _follow(s["heads"], h0, sA[0], kA, f"token {t}: layer 0 heads")
                _follow(s["neurons"], n0_, sM[0], kM, f"token {t}: layer 0 neurons")
            kv = ref.KVState(s["K"], s["V"], s["y_buf"].astype(np.float64), s["valid"].astype(np.int64))
            want, rec = ref.decode_layer_lookahead(s["x_in"], W, Wn, kv, n0 + t, head_idx=s["heads"],
                                                   neuron_idx=s["neurons"], k_heads=kA, k_neurons=kM, scale=scale)
            e = check_close(s["x_out"], want, "f16", f"layer {l} token {t}")
            if Wn is not None:
                _follow(s["next_heads"], rec["next_head_idx"], rec["next_head_scores"][0], kA,
                        f"layer {l} token {t}: next heads")
                _follow(s["next_neurons"], rec["next_neuron_idx"], rec["next_neuron_scores"][0], kM,
                        f"layer {l} token {t}: next neurons")
            assert np.array_equal(s["valid_after"], kv.valid_upto), f"layer {l} token {t}: valid positions"
            ok_k, nk = f16_kv_ok(s["K_after"], kv.K)
            ok_v, nv = f16_kv_ok(s["V_after"], kv.V)
            assert ok_k and ok_v, f"layer {l} token {t}: K off {nk}, V off {nv}"
            print(f"opt66b stack layer {l} token {t}: normwise {e:.2e}")


def _union_follow(got_u, rec, k, what):
    """The device's union of per-sequence neuron sets against the oracle's:
    equal, or differing only in neurons that sit at some sequence's k-th
    score within fp32 rounding.  Returns the union the oracle continues with."""
    want = rec["neuron_idx"]
    got_u = np.asarray(got_u, np.int64)
    if np.array_equal(got_u, want):
        return want
    s = np.asarray(rec["neuron_scores"], np.float64)
    kth = np.sort(s, axis=1)[:, ::-1][:, k - 1]
    for j in set(got_u.tolist()) ^ set(want.tolist()):
        assert np.any(np.abs(s[:, j] - kth) <= MARGIN * max(1.0, np.abs(s).max())), f"{what}: neuron {j}"
    return got_u


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_stack_longctx_composed_sampled(dvlib):
    """The 32-layer long-context stack (d = 4096, 32 heads, d_ffn = 16384) at
    8192 cached tokens in the composed mode: 10% of each head's positions
    chosen by the attention-scored selection (plus the decoded tokens), 10%
    of neurons.  The selection of sampled heads against the oracle's; layers
    {0, 15, 31} at tokens {0, 2} rerun by the oracle from the device's state."""
    from contextual_sparsity_decoding_amd.stack import Stack
    wl = configs.LONGCTX_STACK
    dims, L, n, T, seed = wl.dims, wl.layers, 8192, 3, 515
    b, kM = int(wl.kv_keep * n), wl.k_neurons
    scale = 1 / math.sqrt(dims.d_h)
    S = Stack(dims, L, n, n + T + 4, seed, hole_fill=False)
    S.select_kv(b)
    flags = dvlib.DV_DENSE_ATTN | dvlib.DV_KV_SELECT | dvlib.DV_SKIP_NONPOS_FC2 | dvlib.DV_ADVANCE_POS
    cfg = S.cfg(dims.h, kM, flags, scale)
    ws = dvlib.workspace(dvlib.dv_stack_workspace_bytes(cfg, S.max_len))
    nsets = torch.full((L, kM), -1, dtype=torch.int32, device="cuda")
    x_trace = torch.empty(L - 1, 1, dims.d, device="cuda")
    x_out = torch.empty(1, dims.d, device="cuda")
    X = torch.empty(T, 1, dims.d, device="cuda")
    dvlib.dv_fill_normal(X, seed, synth.stream_id(0, "x"))
    layers, tokens = (0, 15, 31), (0, 2)
    # the selection itself, for two heads of layer 15, against the oracle's
    Kh = synth.philox_tensor((1, dims.h, S.max_len, dims.d_h), seed, 15, "K", 1.0, np.float16)
    assert np.array_equal(host(S.K[15]), Kh)
    Q = synth.philox_tensor((1, dims.h, 64, dims.d_h), seed, 15, "q_obs", 1.0, np.float16)
    sel15 = host(S.sel[15][0])
    for i in (0, 19):
        want_idx, sm = ref.kv_select(Q[0, i], Kh[0, i], n, scale, b, n_sink=4, n_window=64, width=7)
        forced = sm.copy()
        forced[:4] = np.inf
        forced[n - 64:] = np.inf
        assert_selection_close(sel15[0, i], want_idx, forced, b, 1e-5 * max(1.0, np.abs(sm).max()), f"head {i}")
    snaps = {}
    for t in range(T):
        if t in tokens:
            for l in layers:
                snaps[(l, t)] = {"K": host(S.K[l]), "V": host(S.V[l])}
        dvlib.dv_decode_stack(S.layers_array(), cfg, X[t], x_out, ws, neuron_sets=nsets, x_trace=x_trace)
        if t in tokens:
            tr, xo, ns = host(x_trace), host(x_out), host(nsets)
            for l in layers:
                snaps[(l, t)].update(x_in=host(X[t]) if l == 0 else tr[l - 1], x_out=tr[l] if l + 1 < L else xo,
                                     neurons=ns[l], sel=host(S.sel[l][0]), sel_len=host(S.sel[l][1]))
    torch.cuda.synchronize()
    del S, ws
    torch.cuda.empty_cache()
    for l in layers:
        W = synth.stack_layer_weights(dims, seed, l)
        for t in tokens:
            s = snaps[(l, t)]
            kv = ref.KVState(s["K"].copy(), s["V"].copy())
            want, rec = ref.decode_layer(s["x_in"], W, kv, n + t, k_heads=dims.h, k_neurons=kM, scale=scale,
                                         dense_attn=True, skip_nonpos=True, hole_fill=False, sel_idx=s["sel"],
                                         sel_len=s["sel_len"], sel_end=n)
            used = _follow(s["neurons"], rec["neuron_idx"], rec["neuron_scores"][0], kM, f"layer {l} token {t}")
            if used is not rec["neuron_idx"]:
                want, _ = ref.sparse_mlp(rec["y2"], W["w1_t"], W["b1"], W["w2_t"], W["b2"], used, residual=rec["h"],
                                         skip_nonpos=True)
            e = check_close(s["x_out"], want, "f16", f"longctx layer {l} token {t}")
            print(f"longctx stack layer {l} token {t}: normwise {e:.2e}")


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("B", [16, 4])
def test_stack_opt175b_batch_union_sampled(dvlib, B):
    """Four layers at the OPT-175B share's width (d = 12288, 96 heads dense,
    d_ffn = 49152) decoding B sequences with 512 cached tokens each; every
    layer's MLP reads the union of the B top-10% neuron sets.  Both batches
    run Q/K/V and fc1 on the matrix cores (4 rows of 12288 inputs do not fit
    in LDS).  Layers {0, 3} at tokens {0, 1} rerun by the oracle from the
    device's state."""
    from contextual_sparsity_decoding_amd.stack import Stack
    wl = configs.OPT175B_SHARE
    dims, L, n, T, seed = wl.dims, 4, wl.n_ctx, 2, 177
    kM = wl.k_neurons
    scale = 1 / math.sqrt(dims.d_h)
    S = Stack(dims, L, n, n + T + 4, seed, batch=B, hole_fill=False)
    flags = dvlib.DV_DENSE_ATTN | dvlib.DV_SKIP_NONPOS_FC2 | dvlib.DV_ADVANCE_POS
    cfg = S.cfg(dims.h, kM, flags, scale)
    ws = dvlib.workspace(dvlib.dv_stack_workspace_bytes(cfg, S.max_len))
    nmax = min(dims.N, B * kM)
    usets = torch.full((L, nmax), -1, dtype=torch.int32, device="cuda")
    counts = torch.zeros(L, dtype=torch.int32, device="cuda")
    x_trace = torch.empty(L - 1, B, dims.d, device="cuda")
    x_out = torch.empty(B, dims.d, device="cuda")
    X = torch.empty(T, B, dims.d, device="cuda")
    dvlib.dv_fill_normal(X, seed, synth.stream_id(B, "x"))
    layers = (0, 3)
    snaps = {}
    for t in range(T):
        for l in layers:
            snaps[(l, t)] = {"K": host(S.K[l]), "V": host(S.V[l])}
        dvlib.dv_decode_stack(S.layers_array(), cfg, X[t], x_out, ws, neuron_sets=usets, neuron_counts=counts,
                              x_trace=x_trace)
        tr, xo, us, uc = host(x_trace), host(x_out), host(usets), host(counts)
        for l in layers:
            snaps[(l, t)].update(x_in=host(X[t]) if l == 0 else tr[l - 1], x_out=tr[l] if l + 1 < L else xo,
                                 union=us[l, :uc[l]])
    torch.cuda.synchronize()
    del S, ws
    torch.cuda.empty_cache()
    for l in layers:
        W = synth.stack_layer_weights(dims, seed, l)
        for t in range(T):
            s = snaps[(l, t)]
            kv = ref.KVState(s["K"].copy(), s["V"].copy())
            want, rec = ref.decode_layer(s["x_in"], W, kv, n + t, k_heads=dims.h, k_neurons=kM, scale=scale,
                                         dense_attn=True, skip_nonpos=True, hole_fill=False)
            used = _union_follow(s["union"], rec, kM, f"layer {l} token {t}")
            if used is not rec["neuron_idx"]:
                want, _ = ref.sparse_mlp(rec["y2"], W["w1_t"], W["b1"], W["w2_t"], W["b2"], used, residual=rec["h"],
                                         skip_nonpos=True)
            e = check_close(s["x_out"], want, "f16", f"batched layer {l} token {t}")
            print(f"batch-{B} stack layer {l} token {t}: |U| = {len(s['union'])}, normwise {e:.2e}")


def test_launch_timing_marks_each_kernel(dvlib):
    """dv_time_launches: one event pair per launch of the role, each pair
    inside the token's own span, and the decode's results unchanged by it."""
    dims = LayerDims(d=1024, N=4096, h=8, d_h=128, r_attn=32, r_mlp=64, wdt="f16")
    L, n0, kA, kM, seed = 3, 40, 3, 400, 23
    D = DeviceStack(dvlib, dims, L, n0, n0 + 8, seed, kA, kM)
    x = torch.empty(1, dims.d, device="cuda")
    dvlib.dv_fill_normal(x, seed, synth.stream_id(0, "x"))
    D.S.reset()
    D.token(x)
    plain = host(D.x_out)
    for kind in (dvlib.DV_KERNEL_QKV, dvlib.DV_KERNEL_ATTN, dvlib.DV_KERNEL_OUT, dvlib.DV_KERNEL_FC1,
                 dvlib.DV_KERNEL_FC2):
        D.S.reset()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        timer = dvlib.LaunchTimer(kind, L)
        e0.record()
        with timer:
            D.token(x)
        e1.record()
        d_ms = timer.durations_ms()
        span = e0.elapsed_time(e1)
        assert len(d_ms) == L, (kind, len(d_ms))
        assert all(0 < t < span for t in d_ms), (kind, d_ms, span)
        assert np.array_equal(host(D.x_out), plain), kind
