"""Parity of each libdv entry point with the CPU oracle on the same seeded
bytes (GPU).  Index sets must match bit for bit; floating-point outputs meet
max-abs 1e-4 (fp32 weights) or normwise 2e-2 (fp16 weights, fp32 accumulate);
fp16 KV entries may differ by one unit in the last place (both sides round
their own fp32/fp64 value to fp16)."""
import math

import numpy as np
import pytest
import torch

from contextual_sparsity_decoding_amd import synth
from contextual_sparsity_decoding_amd.configs import LayerDims
from oracle import ref
from tests.gpu_helpers import assert_selection_close, check_close, dev, f16_kv_ok, host, maxabs, normwise, selection_margin

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------- LayerNorm ----

@pytest.mark.parametrize("B,d", [(1, 200), (3, 5120), (1, 12288)])
def test_layernorm(dvlib, B, d):
    x = synth.normal((B, d), 1, 0, "x") * 3 + 1
    g = synth.normal((d,), 2, 0, "x")
    b = synth.normal((d,), 3, 0, "x")
    y = torch.empty(B, d, device="cuda")
    dvlib.dv_layernorm(dev(x), dev(g), dev(b), 1e-5, y)
    want = ref.layernorm(x, g, b, 1e-5)
    assert maxabs(host(y), want) < 1e-4


# ------------------------------------------------------------- predictor ----

PRED_CASES = [
    # B, d, r, n_out, wdt   (the fp32 MLP block's predictor, the OPT-13B layer's two, a ragged one)
    (1, 256, 64, 1024, "f32"),
    (1, 5120, 128, 20480, "f16"),
    (1, 5120, 128, 40, "f16"),
    (3, 200, 24, 333, "f16"),
    (2, 96, 8, 70, "f32"),
]


@pytest.mark.parametrize("act", ["relu", "none"])
@pytest.mark.parametrize("B,d,r,n,wdt", PRED_CASES)
def test_predict(dvlib, B, d, r, n, wdt, act):
    dt = np.float16 if wdt == "f16" else np.float32
    p1 = synth.normal((r, d), 4, 0, "pm1_t", 0.02, dt)
    p2 = synth.normal((n, r), 4, 0, "pm2_t", 0.02, dt)
    y = synth.normal((B, d), 4, 0, "x")
    ws = dvlib.workspace(dvlib.dv_predict_workspace_bytes(B, d, r, dvlib.wdt_of(dev(p1))))
    s = torch.empty(B, n, device="cuda")
    dvlib.dv_predict(dev(y), dev(p1), dev(p2), dvlib.DV_ACT_RELU if act == "relu" else dvlib.DV_ACT_NONE, s, ws)
    want = ref.predictor(y, p1, p2, act)
    check_close(host(s), want, wdt, "scores")
    assert normwise(host(s), want) < 1e-5


# ------------------------------------------------------------- top-k --------

def _scores(case, B, n, seed):
    if case == "normal":
        return synth.tied_scores(B, n, seed)
    if case == "ties":
        return synth.tied_scores(B, n, seed, levels=5)
    s = synth.tied_scores(B, n, seed, levels=9)
    g = np.random.default_rng(seed)
    m = g.random((B, n))
    s[m < 0.05] = np.nan
    s[(m >= 0.05) & (m < 0.1)] = -0.0
    s[(m >= 0.1) & (m < 0.12)] = np.inf
    s[(m >= 0.12) & (m < 0.14)] = -np.inf
    return s


TOPK_CASES = [(1, 40, 20), (1, 20480, 2048), (1, 49152, 4915), (1, 65536, 1000), (3, 1000, 77),
              (1, 7, 7), (2, 300, 1), (1, 36864, 1843), (1, 1, 1),
              (1, 257, 100), (1, 20481, 2048), (2, 32768, 3000),      # ragged and full single tiles
              (1, 131072, 13107), (1, 70001, 5000),                   # rows of several tiles
              (16, 49152, 4915), (5, 40001, 777)]                     # batches over one-tile rows of 40-48 per thread


@pytest.mark.parametrize("case", ["normal", "ties", "specials"])
@pytest.mark.parametrize("B,n,k", TOPK_CASES)
def test_topk_bit_exact(dvlib, B, n, k, case):
    s = _scores(case, B, n, seed=n + k)
    idx = torch.full((B, k), -1, dtype=torch.int32, device="cuda")
    u = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    uc = torch.zeros(1, dtype=torch.int32, device="cuda")
    dvlib.dv_topk_select(dev(s), k, idx, u, uc)
    got = host(idx)
    want = ref.topk_rows(s, k)
    for b in range(B):
        assert np.array_equal(got[b], want[b]), (b, case)
    U = ref.union_sorted(want)
    assert int(host(uc)[0]) == len(U)
    assert np.array_equal(host(u)[:len(U)], U)


def test_topk_k_zero_and_full(dvlib):
    s = _scores("ties", 2, 500, 3)
    idx = torch.empty((2, 500), dtype=torch.int32, device="cuda")
    dvlib.dv_topk_select(dev(s), 500, idx)
    assert np.array_equal(host(idx), np.tile(np.arange(500), (2, 1)))
    dvlib.dv_topk_select(dev(s), 0, idx)        # nothing to do, no error


# ------------------------------------------------------------- MLP ----------

def _mlp_inputs(d, N, k, B, wdt, seed):
    dims = LayerDims(d=d, N=N, h=0, r_mlp=16, wdt=wdt)
    W = synth.mlp_weights(dims, seed)
    y = synth.layer_inputs(d, 1, B, seed)[0]
    idx = np.sort(np.random.default_rng(seed).choice(N, k, replace=False)).astype(np.int32)
    return W, y, idx


MLP_CASES = [
    # d, N, k, B, wdt
    (256, 1024, 256, 1, "f32"),       # the fp32 MLP block
    (5120, 20480, 2048, 1, "f16"),    # the OPT-13B layer's MLP at 10% of neurons
    (200, 300, 77, 2, "f16"),         # ragged: 400-byte rows, partial slice
    (9216, 36864, 1843, 1, "f16"),    # OPT-66B width at 5%
    # batches of 8-16: fc1 on the matrix cores (fp32 inputs split into fp16 hi + lo)
    (1024, 4096, 333, 8, "f16"),      # ragged: 333 rows, not a multiple of the 64-row tiles
    (4096, 16384, 1638, 16, "f16"),
    (12288, 49152, 4915, 9, "f16"),   # OPT-175B width, odd batch
    (1280, 5120, 512, 12, "f16"),     # five 256-column slices of the matrix-core gather-AXPY
    (1024, 4096, 400, 2, "f16"),      # a batch of 2 on the matrix-core gather-AXPY, fc1 on the vector path
    (12288, 49152, 4915, 3, "f16"),   # a batch of 3 whose inputs do not fit in LDS: fc1 on the matrix cores
]


@pytest.mark.parametrize("skip", [False, True])
@pytest.mark.parametrize("d,N,k,B,wdt", MLP_CASES)
def test_sparse_mlp(dvlib, d, N, k, B, wdt, skip):
    W, y, idx = _mlp_inputs(d, N, k, B, wdt, seed=d + k)
    res = synth.normal((B, d), 9, 0, "x")
    Wd = {n: dev(v) for n, v in W.items()}
    out = torch.empty(B, d, device="cuda")
    a = torch.empty(B, k, device="cuda")
    rows = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = dvlib.workspace(dvlib.dv_sparse_mlp_workspace_bytes(B, d, k, dvlib.wdt_of(Wd["w1_t"])))
    dvlib.dv_sparse_mlp(dev(y), Wd["w1_t"], Wd["b1"], Wd["w2_t"], Wd["b2"], dev(idx), k, out, ws, residual=dev(res),
                        act_out=a, fc2_rows=rows, flags=dvlib.DV_SKIP_NONPOS_FC2 if skip else 0)
    want, wa = ref.sparse_mlp(y, W["w1_t"], W["b1"], W["w2_t"], W["b2"], idx, residual=res, skip_nonpos=skip)
    check_close(host(out), want, wdt, "out")
    check_close(host(a), wa, wdt, "a")
    live = int(np.sum(np.any(wa > 0, axis=0)))
    assert int(host(rows)[0]) == (live if skip else k)
    # some neuron is dead in every row of a small batch; in a batch of 16
    # nearly every one fires somewhere
    assert 0 < live <= k and (B > 4 or live < k)


@pytest.mark.parametrize("B", [8, 16])
def test_sparse_mlp_matrix_core_edges(dvlib, B):
    """Batches on the matrix-core kernels with nothing to gather: every fc1
    output non-positive (fc2 keeps no row, so out = residual + b2, and the
    rows-read count is 0), and a device-side count of zero selected rows
    (fc1 writes nothing, the finalize adds no group)."""
    d, N, k = 1024, 4096, 333
    W, y, idx = _mlp_inputs(d, N, k, B, "f16", seed=B + 71)
    res = synth.normal((B, d), 72, 0, "x")
    W = dict(W)
    W["b1"] = np.full_like(W["b1"], -1e3)               # the ReLU closes every neuron
    Wd = {n: dev(v) for n, v in W.items()}
    out = torch.empty(B, d, device="cuda")
    rows = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = dvlib.workspace(dvlib.dv_sparse_mlp_workspace_bytes(B, d, k, dvlib.DV_F16))
    dvlib.dv_sparse_mlp(dev(y), Wd["w1_t"], Wd["b1"], Wd["w2_t"], Wd["b2"], dev(idx), k, out, ws, residual=dev(res),
                        fc2_rows=rows, flags=dvlib.DV_SKIP_NONPOS_FC2)
    want, wa = ref.sparse_mlp(y, W["w1_t"], W["b1"], W["w2_t"], W["b2"], idx, residual=res, skip_nonpos=True)
    assert not np.any(wa > 0)
    check_close(host(out), want, "f16", "all neurons closed")
    assert int(host(rows)[0]) == 0
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    out2 = torch.full((B, d), float("nan"), device="cuda")
    dvlib.dv_sparse_mlp(dev(y), Wd["w1_t"], Wd["b1"], Wd["w2_t"], Wd["b2"], dev(idx), k, out2, ws, residual=dev(res),
                        n_idx_dev=zero)
    base = res.astype(np.float64) + W["b2"].astype(np.float64)[None, :]
    check_close(host(out2), base, "f16", "no selected rows")


def test_sparse_mlp_dense_and_union(dvlib):
    d, N, B = 512, 2048, 4
    W, y, _ = _mlp_inputs(d, N, 10, B, "f16", seed=5)
    Wd = {n: dev(v) for n, v in W.items()}
    out = torch.empty(B, d, device="cuda")
    ws = dvlib.workspace(dvlib.dv_sparse_mlp_workspace_bytes(B, d, N, dvlib.DV_F16))
    dvlib.dv_sparse_mlp(dev(y), Wd["w1_t"], Wd["b1"], Wd["w2_t"], Wd["b2"], None, N, out, ws)
    want, _ = ref.dense_mlp(y, W["w1_t"], W["b1"], W["w2_t"], W["b2"])
    check_close(host(out), want, "f16", "dense")
    # union of per-row top-k sets with a device-side count
    s = synth.tied_scores(B, N, 6)
    k = 100
    idx = torch.empty(B, k, dtype=torch.int32, device="cuda")
    u = torch.empty(N, dtype=torch.int32, device="cuda")
    uc = torch.zeros(1, dtype=torch.int32, device="cuda")
    dvlib.dv_topk_select(dev(s), k, idx, u, uc)
    nmax = min(N, B * k)
    dvlib.dv_sparse_mlp(dev(y), Wd["w1_t"], Wd["b1"], Wd["w2_t"], Wd["b2"], u, nmax, out, ws, n_idx_dev=uc,
                        flags=dvlib.DV_SKIP_NONPOS_FC2)
    U = ref.union_sorted(ref.topk_rows(s, k))
    assert int(host(uc)[0]) == len(U) and len(U) < nmax
    want, _ = ref.sparse_mlp(y, W["w1_t"], W["b1"], W["w2_t"], W["b2"], U, skip_nonpos=True)
    check_close(host(out), want, "f16", "union")


def test_mlp_block_fp32_end_to_end(dvlib):
    """The fp32 MLP block: predictor -> top-256 -> sparse MLP, all on the GPU."""
    dims = LayerDims(d=256, N=1024, h=0, r_mlp=64, wdt="f32")
    W = synth.mlp_weights(dims, seed=0)
    x = synth.layer_inputs(256, 1, 1, seed=0)[0]
    Wd = {n: dev(v) for n, v in W.items()}
    s = torch.empty(1, 1024, device="cuda")
    dvlib.dv_predict(dev(x), Wd["pm1_t"], Wd["pm2_t"], dvlib.DV_ACT_RELU, s,
                     dvlib.workspace(dvlib.dv_predict_workspace_bytes(1, 256, 64, dvlib.DV_F32)))
    idx = torch.empty(1, 256, dtype=torch.int32, device="cuda")
    dvlib.dv_topk_select(s, 256, idx)
    out = torch.empty(1, 256, device="cuda")
    dvlib.dv_sparse_mlp(dev(x), Wd["w1_t"], Wd["b1"], Wd["w2_t"], Wd["b2"], idx, 256, out,
                        dvlib.workspace(dvlib.dv_sparse_mlp_workspace_bytes(1, 256, 256, dvlib.DV_F32)),
                        flags=dvlib.DV_SKIP_NONPOS_FC2)
    sc = ref.predictor(x, W["pm1_t"], W["pm2_t"]).astype(np.float32)[0]
    want_idx = ref.topk_select(sc, 256)
    assert selection_margin(sc, 256) > 1e-6      # fp32 score error is ~1e-8 here
    assert np.array_equal(host(idx)[0], want_idx)
    want, _ = ref.sparse_mlp(x, W["w1_t"], W["b1"], W["w2_t"], W["b2"], want_idx, skip_nonpos=True)
    check_close(host(out), want, "f32", "mlp block")


# ------------------------------------------------------------- projections --

def _attn_setup(d, h, dh, max_len, n_filled, seed, wdt="f16", B=1):
    dims = LayerDims(d=d, N=64, h=h, d_h=dh, r_attn=16, r_mlp=16, wdt=wdt)
    W = synth.attn_weights(dims, seed)
    K, V = synth.kv_cache(h, dh, n_filled, max_len, seed, batch=B)
    return W, K, V


@pytest.mark.parametrize("B,h,dh,full,d", [(2, 8, 64, False, 512), (2, 8, 128, False, 512), (1, 8, 64, False, 512),
                                           (1, 8, 128, False, 512), (1, 80, 64, False, 512), (1, 8, 128, True, 512),
                                           (1, 8, 128, False, 6144), (1, 8, 128, False, 9216),
                                           (2, 8, 128, False, 9216)])
def test_qkv_with_holes_over_steps(dvlib, B, h, dh, full, d):
    """Missing K/V positions recomputed from the stored inputs (DejaVu §4.2):
    batch rows of two (each row its own holes), and a batch of one, where
    helper workgroups take the rounds past the first (more items than
    helpers when every head has a long gap; with 80 heads, 40 selected
    and then all 80, past the helpers' 64-head limit).  With `full` the
    cache holds exactly the positions the steps write (the last step writes
    slot max_len - 1).  At d = 6144 one stored input fits beside y in LDS:
    the owner computes one missing position and helpers take one at a time.
    At d = 9216 none does: the owners (wave pairs splitting each row) take
    every missing position, each staged in y's place once y is consumed
    (batch of one) or read from global memory (two batch rows)."""
    n0, T = 10, 9
    L = n0 + T if full else 48
    W, K, V = _attn_setup(d, h, dh, L, n0, seed=dh + h + B, B=B)
    X = synth.layer_inputs(d, T, B, seed=dh + B)
    g = np.random.default_rng(dh + h)
    # oracle state
    okv = ref.KVState(K.copy(), V.copy(), np.zeros((B, L, d)), np.full((B, h), n0 - 1))
    # device state
    Kd, Vd = dev(K), dev(V)
    yb = torch.zeros(B, L, d, device="cuda")
    vu = dev(np.full((B, h), n0 - 1, np.int32))
    wq, bq = dev(W["w_qkv_t"]), dev(W["b_qkv"])
    ws = dvlib.workspace(dvlib.dv_attn_proj_workspace_bytes(0, B, d, h, dh, h, dvlib.DV_F16))
    for t in range(T):
        pos = n0 + t
        if t == T - 1:
            sel = np.arange(h, dtype=np.int32)             # every head: holes of up to 8 steps
        elif t == T - 2 and h > 64:
            sel = np.sort(g.choice(h, 40, replace=False)).astype(np.int32)
        else:
            sel = np.sort(g.choice(h, 3, replace=False)).astype(np.int32)
        sel_d, x_d = dev(sel), dev(X[t])
        q = torch.empty(B, len(sel), dh, device="cuda")
        kv = dvlib.kv_state(Kd, Vd, pos, yb, vu)
        dvlib.dv_sparse_attn_proj(dvlib.DV_PROJ_QKV, h, dh, sel_d, len(sel), wq, bq, x_d, q, ws, kv=kv)
        wq_ = ref.qkv_step(X[t], W["w_qkv_t"], W["b_qkv"], sel, okv, pos)
        check_close(host(q), wq_, "f16", f"q step {t}")
    assert np.array_equal(host(vu), okv.valid_upto)
    Kg, Vg = host(Kd), host(Vd)
    ok_k, nk = f16_kv_ok(Kg, okv.K)
    ok_v, nv = f16_kv_ok(Vg, okv.V)
    assert ok_k and ok_v, f"K entries off: {nk}, V entries off: {nv}"
    same = np.array_equal(host(yb)[:, n0:n0 + T], okv.y_buf[:, n0:n0 + T].astype(np.float32))
    assert same, "stored layer inputs differ"


def test_qkv_without_hole_fill(dvlib):
    d, h, dh, L = 256, 4, 64, 16
    W, K, V = _attn_setup(d, h, dh, L, 5, seed=3)
    x = synth.layer_inputs(d, 1, 1, seed=3)[0]
    Kd, Vd = dev(K), dev(V)
    sel = np.array([1, 3], np.int32)
    q = torch.empty(1, 2, dh, device="cuda")
    dvlib.dv_sparse_attn_proj(0, h, dh, dev(sel), 2, dev(W["w_qkv_t"]), dev(W["b_qkv"]), dev(x), q, None,
                              kv=dvlib.kv_state(Kd, Vd, 8))
    okv = ref.KVState(K.copy(), V.copy())
    wq = ref.qkv_step(x, W["w_qkv_t"], W["b_qkv"], sel, okv, 8, hole_fill=False)
    check_close(host(q), wq, "f16", "q")
    ok_k, nk = f16_kv_ok(host(Kd), okv.K)
    ok_v, nv = f16_kv_ok(host(Vd), okv.V)
    assert ok_k and ok_v, f"K entries off: {nk}, V entries off: {nv}"
    assert np.all(host(Kd)[0, :, 5:8] == 0)          # skipped slots untouched


@pytest.mark.parametrize("B,n_sel,wdt", [(1, 20, "f16"), (2, 3, "f16"), (1, 4, "f32"), (8, 20, "f16"), (13, 20, "f16")])
def test_out_proj(dvlib, B, n_sel, wdt):
    d, h, dh = 5120 if n_sel == 20 else 320, 40 if n_sel == 20 else 6, 128
    W, _, _ = _attn_setup(d, h, dh, 4, 0, seed=n_sel, wdt=wdt)
    heads = np.sort(np.random.default_rng(n_sel).choice(h, n_sel, replace=False)).astype(np.int32)
    o = synth.normal((B, n_sel, dh), 5, 0, "x")
    res = synth.normal((B, d), 6, 0, "x")
    out = torch.empty(B, d, device="cuda")
    ws = dvlib.workspace(dvlib.dv_attn_proj_workspace_bytes(1, B, d, h, dh, n_sel, dvlib.wdt_of(dev(W["w_o_t"]))))
    dvlib.dv_sparse_attn_proj(dvlib.DV_PROJ_OUT, h, dh, dev(heads), n_sel, dev(W["w_o_t"]), dev(W["b_o"]), dev(o),
                              out, ws, residual=dev(res))
    want = ref.out_proj(o, W["w_o_t"], W["b_o"], heads, residual=res)
    check_close(host(out), want, wdt, "out_proj")


# ------------------------------------------------------------- attention ----

@pytest.mark.parametrize("splits", [0, 1, 3, 7])
@pytest.mark.parametrize("dh,n_ctx", [(128, 2049), (64, 1000), (128, 1), (32, 77), (256, 300)])
def test_splitk_dense(dvlib, dh, n_ctx, splits):
    h, L, B = 6, n_ctx + 3, 2
    K, V = synth.kv_cache(h, dh, n_ctx, L, seed=dh + n_ctx, batch=B)
    heads = np.array([0, 2, 5], np.int32)
    q = synth.normal((B, 3, dh), 7, 0, "x")
    scale = 1 / math.sqrt(dh)
    view = dvlib.kv_view(dev(K), dev(V), n_ctx)
    ws = dvlib.workspace(dvlib.dv_splitk_workspace_bytes(B, 3, dh, n_ctx, splits))
    o = torch.empty(B, 3, dh, device="cuda")
    dvlib.dv_splitk_attn(dev(q), dev(heads), 3, view, scale, o, ws, num_splits=splits)
    want = ref.attention(q, ref.KVState(K, V), heads, n_ctx, scale)
    assert maxabs(host(o), want) < 1e-4


@pytest.mark.parametrize("splits", [0, 2, 5])
def test_splitk_selected_positions(dvlib, splits):
    h, dh, n_ctx, sel_end, cap, B = 4, 128, 900, 850, 200, 1
    L = 960
    K, V = synth.kv_cache(h, dh, n_ctx, L, seed=11, batch=B)
    g = np.random.default_rng(11)
    sel = np.zeros((B, h, cap), np.int32)
    lens = np.array([[200, 37, 0, 1]], np.int32)
    for i in range(h):
        sel[0, i, :lens[0, i]] = np.sort(g.choice(sel_end, lens[0, i], replace=False))
    heads = np.arange(h, dtype=np.int32)
    q = synth.normal((B, h, dh), 8, 0, "x")
    view = dvlib.kv_view(dev(K), dev(V), n_ctx, dev(sel), dev(lens), sel_end)
    ws = dvlib.workspace(dvlib.dv_splitk_workspace_bytes(B, h, dh, cap + n_ctx - sel_end, splits))
    o = torch.empty(B, h, dh, device="cuda")
    dvlib.dv_splitk_attn(dev(q), dev(heads), h, view, 0.1, o, ws, num_splits=splits)
    want = ref.attention(q, ref.KVState(K, V), heads, n_ctx, 0.1, sel, lens, sel_end)
    assert maxabs(host(o), want) < 1e-4
    # a head with no positions at all gets zeros
    view = dvlib.kv_view(dev(K), dev(V), n_ctx, dev(sel), dev(np.zeros((B, h), np.int32)), n_ctx)
    dvlib.dv_splitk_attn(dev(q), dev(heads), h, view, 0.1, o, ws, num_splits=splits)
    assert np.all(host(o) == 0)


@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("n_ctx,n_sink,win_len", [(2049, 4, 200), (300, 4, 400), (77, 0, 10), (1000, 50, 3),
                                                  (5000, 4, 496)])
def test_splitk_window(dvlib, n_ctx, n_sink, win_len, splits):
    """The KV window (sinks plus the recent positions), read in place."""
    h, dh, B = 4, 128, 2
    K, V = synth.kv_cache(h, dh, n_ctx, n_ctx + 5, seed=n_ctx + win_len, batch=B)
    heads = np.array([3, 0, 1], np.int32)
    q = synth.normal((B, 3, dh), 9, 0, "x")
    view = dvlib.kv_view(dev(K), dev(V), n_ctx, win_sink=n_sink, win_len=win_len)
    ws = dvlib.workspace(dvlib.dv_splitk_workspace_bytes(B, 3, dh, min(n_ctx, n_sink + win_len), splits))
    o = torch.empty(B, 3, dh, device="cuda")
    dvlib.dv_splitk_attn(dev(q), dev(heads), 3, view, 0.09, o, ws, num_splits=splits)
    want = ref.attention(q, ref.KVState(K, V), heads, n_ctx, 0.09, window=(n_sink, win_len))
    assert maxabs(host(o), want) < 1e-4


def test_splitk_window_with_device_count(dvlib):
    """The count read at run time moves the recent window with it."""
    h, dh, B, bound, n_sink, win_len = 4, 128, 1, 3000, 4, 300
    K, V = synth.kv_cache(h, dh, bound, bound, seed=33, batch=B)
    heads = np.arange(h, dtype=np.int32)
    q = synth.normal((B, h, dh), 10, 0, "x")
    n_dev = torch.zeros(1, dtype=torch.int32, device="cuda")
    view = dvlib.kv_view(dev(K), dev(V), bound, n_ctx_dev=n_dev, win_sink=n_sink, win_len=win_len)
    ws = dvlib.workspace(dvlib.dv_splitk_workspace_bytes(B, h, dh, n_sink + win_len, 0))
    o = torch.empty(B, h, dh, device="cuda")
    for n in (1, 200, 304, 2999, 3000):
        n_dev.fill_(n)
        dvlib.dv_splitk_attn(dev(q), dev(heads), h, view, 0.1, o, ws)
        want = ref.attention(q, ref.KVState(K, V), heads, n, 0.1, window=(n_sink, win_len))
        assert maxabs(host(o), want) < 1e-4, n


def test_kv_score_and_selection(dvlib):
    h, dh, n, n_obs, B = 4, 128, 700, 64, 1
    K, V = synth.kv_cache(h, dh, n, n + 10, seed=21, batch=B)
    Q = synth.observation_queries(h, n_obs, dh, seed=21, batch=B)
    scale = 1 / math.sqrt(dh)
    view = dvlib.kv_view(dev(K), dev(V), n)
    sc = torch.empty(B, h, n, device="cuda")
    ws = dvlib.workspace(dvlib.dv_kv_score_workspace_bytes(B, h, n, n_obs))
    dvlib.dv_kv_score(dev(Q), view, scale, 4, n_obs, 7, sc, ws)
    got = host(sc)
    budget = 70
    idx = torch.empty(B * h, budget, dtype=torch.int32, device="cuda")
    dvlib.dv_topk_select(sc.view(B * h, n), budget, idx)
    gi = host(idx)
    for i in range(h):
        want_idx, sm = ref.kv_select(Q[0, i], K[0, i], n, scale, budget, n_sink=4, n_window=n_obs, width=7)
        free = slice(4, n - n_obs)
        assert np.all(np.isinf(got[0, i, :4])) and np.all(np.isinf(got[0, i, n - n_obs:]))
        assert maxabs(got[0, i, free], sm[free]) < 1e-5 * max(1.0, np.abs(sm).max())
        # top-b of the GPU's own scores is bit-exact (the selection kernel's
        # contract), and the oracle's set differs at most by swaps at the
        # boundary that the score error allows
        assert np.array_equal(gi[i], ref.topk_select(got[0, i], budget))
        forced = sm.copy()
        forced[:4] = np.inf
        forced[n - n_obs:] = np.inf
        assert_selection_close(gi[i], want_idx, forced, budget, 1e-5 * max(1.0, np.abs(sm).max()), f"head {i}")
