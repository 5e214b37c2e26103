"""Parity at the widths and lengths of the larger workloads (GPU).

The OPT-66B-width layer (d=9216, 72 heads, N=36864, 1024 cached tokens), the
OPT-175B share's batched path (d=12288, 96 heads, N=49152, 16 sequences over
the union of their neuron sets, 512 cached tokens) and the long-context
composition (d=4096, 32 heads, up to 131072 cached positions with a 10% KV
budget) each run here at full size, through the same entry points the layer
uses, against the oracle on the same seeded inputs.  Where a selection could
be ambiguous the test feeds both sides the same index set, so every value
compared is unique."""
import math

import numpy as np
import pytest
import torch

from contextual_sparsity_decoding_amd import configs, synth
from contextual_sparsity_decoding_amd.configs import LayerDims
from oracle import ref
from tests.gpu_helpers import assert_selection_close, check_close, dev, f16_kv_ok, host, maxabs, upload
from tests.test_gpu_layer import Layer, _compare_step

pytestmark = pytest.mark.gpu


# ------------------------------------------------------- OPT-66B width -----

def test_opt66b_width_layer_two_steps(dvlib):
    """d=9216: 36 of 72 heads, 1843 of 36864 neurons (5%), 1024 cached tokens,
    two steps so that newly selected heads recompute a missing position (at
    this width the stored inputs are read from global memory)."""
    w = configs.OPT66B_STACK
    L = Layer(dvlib, w.dims, w.n_ctx, w.n_ctx + 4, seed=66)
    X = synth.layer_inputs(w.dims.d, 2, 1, seed=66)
    k_m = int(0.05 * w.dims.N)
    flags = dvlib.DV_HOLE_FILL | dvlib.DV_SKIP_NONPOS_FC2
    checked = 0
    for t in range(2):
        got = L.step(X[t], w.n_ctx + t, w.k_heads, k_m, flags)
        want, rec = L.oracle(X[t], w.n_ctx + t, w.k_heads, k_m, flags)
        e = _compare_step(L, got, want, rec, w.k_heads, k_m, flags, f"opt66b step {t}")
        if e is not None:
            checked += 1
            print(f"opt66b-width step {t}: normwise {e:.2e}")
        if not np.array_equal(got[1][:w.k_heads], rec["head_idx"]):
            break
    assert checked == 2, "choose a seed whose selections are unique"
    assert np.array_equal(host(L.valid), L.okv.valid_upto)
    ok_k, nk = f16_kv_ok(host(L.K), L.okv.K)
    ok_v, nv = f16_kv_ok(host(L.V), L.okv.V)
    assert ok_k and ok_v, f"K entries off: {nk}, V entries off: {nv}"


# ------------------------------------------------------- OPT-175B share ----

C4 = configs.OPT175B_SHARE
B16 = 16


def _c4_union(seed, B=B16):
    s = synth.tied_scores(B, C4.dims.N, seed)
    return s, ref.union_sorted(ref.topk_rows(s, C4.k_neurons))


def test_opt175b_topk_and_union_b16(dvlib):
    s, U = _c4_union(175)
    k = C4.k_neurons
    idx = torch.full((B16, k), -1, dtype=torch.int32, device="cuda")
    u = torch.full((C4.dims.N,), -1, dtype=torch.int32, device="cuda")
    uc = torch.zeros(1, dtype=torch.int32, device="cuda")
    dvlib.dv_topk_select(dev(s), k, idx, u, uc)
    want = ref.topk_rows(s, k)
    got = host(idx)
    for b in range(B16):
        assert np.array_equal(got[b], want[b]), b
    assert int(host(uc)[0]) == len(U)
    assert np.array_equal(host(u)[:len(U)], U)
    print(f"union of 16 sets of {k}: {len(U)} of {C4.dims.N} neurons")


@pytest.mark.parametrize("B", [B16, 4])
def test_opt175b_mlp_over_union(dvlib, B):
    """fc1 over the union for B rows (on the matrix cores: 16 rows, or 4 rows
    of 12288 inputs that do not fit in LDS), fc2 skipping neurons that are
    zero in every row, at d=12288, N=49152."""
    d, N = C4.dims.d, C4.dims.N
    _, U = _c4_union(175, B)
    U = U.astype(np.int32)
    W = synth.mlp_weights(C4.dims, 175)
    y = synth.layer_inputs(d, 1, B, 175)[0]
    res = synth.normal((B, d), 176, 0, "x")
    Wd = {n: dev(v) for n, v in W.items() if n in ("w1_t", "b1", "w2_t", "b2")}
    out = torch.empty(B, d, device="cuda")
    a = torch.empty(B, len(U), device="cuda")
    rows = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = dvlib.workspace(dvlib.dv_sparse_mlp_workspace_bytes(B, d, len(U), dvlib.DV_F16))
    dvlib.dv_sparse_mlp(dev(y), Wd["w1_t"], Wd["b1"], Wd["w2_t"], Wd["b2"], dev(U), len(U), out, ws,
                        residual=dev(res), act_out=a, fc2_rows=rows, flags=dvlib.DV_SKIP_NONPOS_FC2)
    want, wa = ref.sparse_mlp(y, W["w1_t"], W["b1"], W["w2_t"], W["b2"], U, residual=res, skip_nonpos=True)
    check_close(host(a), wa, "f16", "fc1 over the union")
    e = check_close(host(out), want, "f16", "mlp out")
    assert int(host(rows)[0]) == int(np.sum(np.any(wa > 0, axis=0)))
    print(f"opt175b-width union MLP, B={B}: normwise {e:.2e}")


def test_opt175b_attention_b16(dvlib):
    """Dense heads for 16 sequences: Q/K/V with KV append (inputs too wide for
    LDS, read from global memory), split-K over 513 positions, out-projection."""
    dims = C4.dims
    d, h, dh, n0 = dims.d, dims.h, dims.d_h, C4.n_ctx
    W = synth.attn_weights(dims, 177)
    y = synth.layer_inputs(d, 1, B16, 177)[0]
    K, V = synth.kv_cache(h, dh, n0, n0 + 2, 177, batch=B16)
    Wd = {n: dev(v) for n, v in W.items() if n in ("w_qkv_t", "b_qkv", "w_o_t", "b_o")}
    Kd, Vd = dev(K), dev(V)
    q = torch.empty(B16, h, dh, device="cuda")
    kv = dvlib.kv_state(Kd, Vd, n0)
    dvlib.dv_sparse_attn_proj(dvlib.DV_PROJ_QKV, h, dh, None, h, Wd["w_qkv_t"], Wd["b_qkv"], dev(y), q,
                              dvlib.workspace(256), kv=kv)
    okv = ref.KVState(K.copy(), V.copy())
    heads = np.arange(h, dtype=np.int32)
    wq = ref.qkv_step(y, W["w_qkv_t"], W["b_qkv"], heads, okv, n0, hole_fill=False)
    check_close(host(q), wq, "f16", "q")
    ok_k, nk = f16_kv_ok(host(Kd)[:, :, n0], okv.K[:, :, n0])
    ok_v, nv = f16_kv_ok(host(Vd)[:, :, n0], okv.V[:, :, n0])
    assert ok_k and ok_v, f"appended K off: {nk}, V off: {nv}"
    # attention over 513 positions from the GPU's cache (equal to the oracle's within fp16 rounding)
    scale = 1 / math.sqrt(dh)
    view = dvlib.kv_view(Kd, Vd, n0 + 1)
    o = torch.empty(B16, h, dh, device="cuda")
    ws = dvlib.workspace(dvlib.dv_splitk_workspace_bytes(B16, h, dh, n0 + 1, 0))
    dvlib.dv_splitk_attn(q, dev(heads), h, view, scale, o, ws)
    wo = ref.attention(host(q), ref.KVState(host(Kd), host(Vd)), heads, n0 + 1, scale)
    assert maxabs(host(o), wo) < 1e-4
    out = torch.empty(B16, d, device="cuda")
    res = synth.normal((B16, d), 178, 0, "x")
    ws = dvlib.workspace(dvlib.dv_attn_proj_workspace_bytes(dvlib.DV_PROJ_OUT, B16, d, h, dh, h, dvlib.DV_F16))
    dvlib.dv_sparse_attn_proj(dvlib.DV_PROJ_OUT, h, dh, None, h, Wd["w_o_t"], Wd["b_o"], o, out, ws,
                              residual=dev(res))
    want = ref.out_proj(host(o), W["w_o_t"], W["b_o"], heads, residual=res)
    e = check_close(host(out), want, "f16", "out-projection")
    print(f"opt175b-width attention block, B=16: out normwise {e:.2e}")


# ------------------------------------------------------- long context ------

C5 = configs.LONGCTX_STACK


def test_longctx_splitk_131072(dvlib):
    """32 heads over 131072 cached positions: dense, and over 13107 retained
    positions per head plus the entries appended after selection."""
    h, dh, n = C5.dims.h, C5.dims.d_h, 131072
    b = int(C5.kv_keep * n)
    sel_end = n - 8
    K, V = synth.kv_cache(h, dh, n, n, seed=131)
    Kd, Vd = dev(K), dev(V)
    heads = np.arange(h, dtype=np.int32)
    q = synth.normal((1, h, dh), 132, 0, "x")
    scale = 1 / math.sqrt(dh)
    o = torch.empty(1, h, dh, device="cuda")
    ws = dvlib.workspace(dvlib.dv_splitk_workspace_bytes(1, h, dh, n, 0))
    dvlib.dv_splitk_attn(dev(q), dev(heads), h, dvlib.kv_view(Kd, Vd, n), scale, o, ws)
    okv = ref.KVState(K, V)
    assert maxabs(host(o), ref.attention(q, okv, heads, n, scale)) < 1e-4
    g = np.random.default_rng(133)
    sel = np.stack([np.sort(g.choice(sel_end, b, replace=False)) for _ in range(h)])[None].astype(np.int32)
    lens = np.full((1, h), b, np.int32)
    view = dvlib.kv_view(Kd, Vd, n, dev(sel), dev(lens), sel_end)
    dvlib.dv_splitk_attn(dev(q), dev(heads), h, view, scale, o, ws)
    want = ref.attention(q, okv, heads, n, scale, sel, lens, sel_end)
    assert maxabs(host(o), want) < 1e-4


def test_longctx_kv_scores_131072(dvlib):
    """The selection scores of 64 observation queries over 131072 positions
    for all 32 heads (GPU), against the oracle on two sampled heads, and the
    budget's top-b for them."""
    h, dh, n, n_obs = C5.dims.h, C5.dims.d_h, 131072, 64
    b = int(C5.kv_keep * n)
    K, V = synth.kv_cache(h, dh, n, n, seed=134)
    Q = synth.observation_queries(h, n_obs, dh, seed=134)
    scale = 1 / math.sqrt(dh)
    view = dvlib.kv_view(dev(K), dev(V), n)
    sc = torch.empty(1, h, n, device="cuda")
    ws = dvlib.workspace(dvlib.dv_kv_score_workspace_bytes(1, h, n, n_obs))
    dvlib.dv_kv_score(dev(Q), view, scale, 4, n_obs, 7, sc, ws)
    idx = torch.empty(h, b, dtype=torch.int32, device="cuda")
    dvlib.dv_topk_select(sc.view(h, n), b, idx)
    got, gi = host(sc), host(idx)
    for i in (0, 21):
        want_idx, sm = ref.kv_select(Q[0, i], K[0, i], n, scale, b, n_sink=4, n_window=n_obs, width=7)
        free = slice(4, n - n_obs)
        assert np.all(np.isinf(got[0, i, :4])) and np.all(np.isinf(got[0, i, n - n_obs:]))
        assert maxabs(got[0, i, free], sm[free]) < 1e-5 * max(1.0, np.abs(sm).max())
        # top-b of the GPU's own scores is bit-exact (the selection kernel's
        # contract); the oracle's set differs at most by boundary swaps the
        # score error allows
        assert np.array_equal(gi[i], ref.topk_select(got[0, i], b))
        forced = sm.copy()
        forced[:4] = np.inf
        forced[n - n_obs:] = np.inf
        assert_selection_close(gi[i], want_idx, forced, b, 1e-5 * max(1.0, np.abs(sm).max()), f"head {i}")


def test_longctx_layer_kv_select_8192(dvlib):
    """One composed layer at d=4096: dense heads over 819 retained positions
    of 8192 plus the appended entries, 1638 of 16384 neurons."""
    w = C5
    n, b = 8192, int(C5.kv_keep * 8192)
    L = Layer(dvlib, w.dims, n, n + 4, seed=135)
    g = np.random.default_rng(136)
    sel = np.stack([np.sort(g.choice(n, b, replace=False)) for _ in range(w.dims.h)])[None].astype(np.int32)
    lens = np.full((1, w.dims.h), b, np.int32)
    X = synth.layer_inputs(w.dims.d, 2, 1, seed=135)
    flags = dvlib.DV_DENSE_ATTN | dvlib.DV_HOLE_FILL | dvlib.DV_SKIP_NONPOS_FC2 | dvlib.DV_KV_SELECT
    for t in range(2):
        s = (sel, lens, n)
        got = L.step(X[t], n + t, w.dims.h, w.k_neurons, flags, sel=s)
        want, rec = L.oracle(X[t], n + t, w.dims.h, w.k_neurons, flags, sel=s)
        e = _compare_step(L, got, want, rec, w.dims.h, w.k_neurons, flags, f"long-context step {t}")
        assert e is not None, "choose a seed whose neuron selection is unique"
        print(f"long-context layer step {t}: normwise {e:.2e}")
