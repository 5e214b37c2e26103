"""The C-ABI library loads, exports every entry point include/dv.h declares,
and rejects bad arguments on the host before any launch (no GPU needed: every
call here fails validation, so nothing reaches the device)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dv.h")
LIB = os.path.join(ROOT, "contextual_sparsity_decoding_amd", "libdv.so")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dv_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def dv():
    if not os.path.exists(LIB):
        pytest.fail("libdv.so is not built (python -m contextual_sparsity_decoding_amd.build)")
    from contextual_sparsity_decoding_amd import dv as mod
    return mod


def test_every_declared_symbol_is_exported(dv):
    names = declared()
    assert len(names) >= 18
    for n in names:
        assert hasattr(dv.lib, n), n
    assert set(dv.EXPORTS) == set(names)


def test_version_and_status_strings(dv):
    assert dv.lib.dv_api_version() == 1
    for i, s in enumerate(dv.STATUS):
        assert dv.lib.dv_status_str(i).decode() == s


# fake device addresses: validation rejects these calls before touching them
P = 1 << 20          # 16-byte aligned, never dereferenced
Q = (1 << 20) + 8    # misaligned


def err(dv):
    return dv.lib.dv_last_error().decode()


def test_predict_validation(dv):
    L = dv.lib
    s = L.dv_predict(0, 1, 64, P, 16, P, 10, dv.DV_F16, dv.DV_ACT_RELU, P, P, 1 << 20, 0)
    assert s == 1 and "NULL" in err(dv)
    assert L.dv_predict(P, 1, 64, P, 16, P, 10, 7, 1, P, P, 1 << 20, 0) == 3
    assert L.dv_predict(P, 1, 64, P, 16, P, 10, dv.DV_F16, 9, P, P, 1 << 20, 0) == 3
    assert L.dv_predict(P, 0, 64, P, 16, P, 10, dv.DV_F16, 1, P, P, 1 << 20, 0) == 2
    assert L.dv_predict(P, 17, 64, P, 16, P, 10, dv.DV_F16, 1, P, P, 1 << 20, 0) == 2
    assert L.dv_predict(P, 1, 60, P, 16, P, 10, dv.DV_F16, 1, P, P, 1 << 20, 0) == 4   # 120-byte rows
    assert L.dv_predict(P, 1, 64, Q, 16, P, 10, dv.DV_F16, 1, P, P, 1 << 20, 0) == 4
    assert L.dv_predict(P, 1, 64, P, 16, P, 10, dv.DV_F16, 1, P, P, 0, 0) == 6
    assert L.dv_predict_workspace_bytes(1, 5120, 128, dv.DV_F16) > 0


def test_topk_validation(dv):
    L = dv.lib
    assert L.dv_topk_select(P, 1, 10, 11, P, 0, 0, 0, 0, 0) == 5
    assert L.dv_topk_select(P, 1, 10, -1, P, 0, 0, 0, 0, 0) == 5
    assert L.dv_topk_select(0, 1, 10, 3, P, 0, 0, 0, 0, 0) == 1
    assert L.dv_topk_select(P, 1, (1 << 22) + 1, 3, P, 0, 0, 0, 0, 0) == 2
    assert L.dv_topk_select(P, 2, (1 << 18) + 1, 3, P, P, P, 0, 0, 0) == 2   # union bitmap limit
    assert L.dv_topk_select(P, 65, 10, 3, P, 0, 0, 0, 0, 0) == 2
    assert L.dv_topk_select(P, 2, 10, 3, P, P, 0, 0, 0, 0) == 1     # union needs both outputs
    assert L.dv_topk_select(0, 1, 10, 0, 0, 0, 0, 0, 0, 0) == 0     # k = 0 is empty, nothing to launch


def test_sparse_mlp_validation(dv):
    L = dv.lib
    args = dict(y=P, B=1, d=64, N=256, w1=P, b1=P, w2=P, b2=P, wdt=dv.DV_F16, idx=P, nmax=32, ndev=0, res=0,
                out=P + 4096, act=0, rows=0, flags=0, ws=P, wsb=1 << 20)

    def call(**kw):
        a = dict(args, **kw)
        return L.dv_sparse_mlp(a["y"], a["B"], a["d"], a["N"], a["w1"], a["b1"], a["w2"], a["b2"], a["wdt"],
                               a["idx"], a["nmax"], a["ndev"], a["res"], a["out"], a["act"], a["rows"], a["flags"],
                               a["ws"], a["wsb"], 0)
    assert call(y=0) == 1
    assert call(wdt=5) == 3
    assert call(B=0) == 2
    assert call(nmax=257) == 5
    assert call(idx=0) == 2                 # NULL idx means every neuron: n_idx_max must be N
    assert call(flags=0x40) == 3
    assert call(d=60) == 4
    assert call(w2=Q) == 4
    assert call(out=P) == 5                 # out aliases y
    assert call(wsb=16) == 6
    assert L.dv_sparse_mlp_workspace_bytes(1, 5120, 2048, dv.DV_F16) > 0


def test_attn_proj_validation(dv):
    L = dv.lib
    kv = dv.KVState(P, P, 100, 100, 0, 0)          # pos == max_len
    assert L.dv_sparse_attn_proj(0, 1, 64, 4, 16, P, 2, P, P, 1, P, 0, P + 4096, C.byref(kv), P, 1 << 20, 0) == 2
    assert L.dv_sparse_attn_proj(0, 1, 64, 4, 64, P, 2, P, P, 1, P, 0, P + 4096, C.byref(kv), P, 1 << 20, 0) == 5
    assert L.dv_sparse_attn_proj(0, 1, 64, 4, 64, P, 5, P, P, 1, P, 0, P + 4096, None, P, 1 << 20, 0) == 5
    assert L.dv_sparse_attn_proj(0, 1, 64, 4, 64, P, 2, P, P, 1, P, 0, P + 4096, None, P, 1 << 20, 0) == 1
    assert L.dv_sparse_attn_proj(3, 1, 64, 4, 64, P, 2, P, P, 1, P, 0, P + 4096, None, P, 1 << 20, 0) == 3
    assert L.dv_sparse_attn_proj(1, 1, 64, 4, 64, P, 2, P, P, 1, P, 0, P + 4096, None, P, 0, 0) == 6


def test_splitk_and_score_validation(dv):
    L = dv.lib
    v = dv.KVView(P, P, 4, 100, 101, 0, 0, 0, 0)    # n_ctx > max_len
    assert L.dv_splitk_attn(P, 1, 64, P, 2, C.byref(v), 0.1, 0, P, P, 1 << 20, 0) == 5
    v = dv.KVView(P, P, 4, 100, 50, P, P, 40, 30)    # sel_cap > sel_end
    assert L.dv_splitk_attn(P, 1, 64, P, 2, C.byref(v), 0.1, 0, P, P, 1 << 20, 0) == 5
    v = dv.KVView(P, P, 4, 100, 50, 0, 0, 0, 0)
    assert L.dv_splitk_attn(P, 1, 48, P, 2, C.byref(v), 0.1, 0, P, P, 1 << 20, 0) == 2
    assert L.dv_splitk_attn(P, 1, 64, P, 5, C.byref(v), 0.1, 0, P, P, 1 << 20, 0) == 5
    assert L.dv_splitk_attn(P, 1, 64, P, 2, C.byref(v), 0.1, 0, P, P, 0, 0) == 6
    assert L.dv_kv_score(P, 1, 4, 64, 8, C.byref(v), 0.1, 4, 8, 6, P, P, 1 << 20, 0) == 5   # even width
    assert L.dv_kv_score(P, 1, 4, 64, 51, C.byref(v), 0.1, 4, 8, 7, P, P, 1 << 20, 0) == 5  # n_obs > n
    v = dv.KVView(P, P, 4, 100, 50, 0, 0, 0, 0, 0, 4, -1)         # negative window
    assert L.dv_splitk_attn(P, 1, 64, P, 2, C.byref(v), 0.1, 0, P, P, 1 << 20, 0) == 5
    v = dv.KVView(P, P, 4, 100, 50, P, P, 20, 30, 0, 4, 8)         # window and retained set together
    assert L.dv_splitk_attn(P, 1, 64, P, 2, C.byref(v), 0.1, 0, P, P, 1 << 20, 0) == 7
    # the window sizes the workspace: 12 positions need fewer splits than 50
    v = dv.KVView(P, P, 4, 100, 50, 0, 0, 0, 0, 0, 4, 8)
    need = L.dv_splitk_workspace_bytes(1, 2, 64, 12, 0)
    assert L.dv_splitk_attn(P, 1, 64, P, 2, C.byref(v), 0.1, 0, P, P, need - 1, 0) == 6


def test_decode_layer_validation(dv):
    L = dv.lib
    cfg = dv.DecodeCfg(B=2, d=64, h=4, d_h=16, N=256, r_attn=16, r_mlp=16, k_heads=2, k_neurons=32,
                       wdt=dv.DV_F16, pred_act=1, eps=1e-5, scale=0.25, flags=0)
    assert L.dv_decode_workspace_bytes(C.byref(cfg), 32) == 0          # d_h = 16 unsupported
    cfg.d_h = 64
    w = dv.LayerWeights(*([P] * 16))
    st = dv.LayerState()
    st.kv = dv.KVState(P, P, 32, 5, 0, 0)
    assert L.dv_decode_layer(C.byref(w), C.byref(cfg), C.byref(st), P, P + 8192, P, 1 << 30, 0) == 7  # heads, B=2
    cfg.B = 1
    assert L.dv_decode_workspace_bytes(C.byref(cfg), 32) > 0
    cfg.flags = 0x8
    assert L.dv_decode_layer(C.byref(w), C.byref(cfg), C.byref(st), P, P + 8192, P, 1 << 30, 0) == 1  # hole state
    cfg.flags = 0x200
    assert L.dv_decode_layer(C.byref(w), C.byref(cfg), C.byref(st), P, P + 8192, P, 1 << 30, 0) == 3
    cfg.flags = dv.DV_TEAL                                             # needs every head and neuron
    assert L.dv_decode_layer(C.byref(w), C.byref(cfg), C.byref(st), P, P + 8192, P, 1 << 30, 0) == 7
    cfg.flags = dv.DV_TEAL | dv.DV_DENSE_ATTN | dv.DV_DENSE_MLP | dv.DV_HOLE_FILL
    assert L.dv_decode_layer(C.byref(w), C.byref(cfg), C.byref(st), P, P + 8192, P, 1 << 30, 0) == 7
    cfg.flags = dv.DV_TEAL | dv.DV_DENSE_ATTN | dv.DV_DENSE_MLP          # input-major weights missing
    assert L.dv_decode_layer(C.byref(w), C.byref(cfg), C.byref(st), P, P + 8192, P, 1 << 30, 0) == 1
    assert "w_qkv_in" in err(dv)
    w2 = dv.LayerWeights(*([P] * 18))
    st.teal_thr[2] = float("nan")
    assert L.dv_decode_layer(C.byref(w2), C.byref(cfg), C.byref(st), P, P + 8192, P, 1 << 30, 0) == 5
    st.teal_thr[2] = 0.0
    cfg.flags = 0
    cfg.k_neurons = 300
    assert L.dv_decode_layer(C.byref(w), C.byref(cfg), C.byref(st), P, P + 8192, P, 1 << 30, 0) == 5
    cfg.k_neurons = 32
    cfg.flags = dv.DV_KV_WINDOW                                        # win_len 0
    assert L.dv_decode_layer(C.byref(w), C.byref(cfg), C.byref(st), P, P + 8192, P, 1 << 30, 0) == 5
    cfg.flags, cfg.win_sink, cfg.win_len = dv.DV_KV_WINDOW | dv.DV_KV_SELECT, 4, 8
    assert L.dv_decode_layer(C.byref(w), C.byref(cfg), C.byref(st), P, P + 8192, P, 1 << 30, 0) == 5
    assert "DV_KV_WINDOW" in err(dv)
    cfg.flags, cfg.win_sink, cfg.win_len, cfg.n_dense_prefix = 0, 0, 0, -1
    assert L.dv_decode_layer(C.byref(w), C.byref(cfg), C.byref(st), P, P + 8192, P, 1 << 30, 0) == 5
    assert L.dv_stack_workspace_bytes(C.byref(cfg), 32) == 0
    # a dense prefix needs room for the dense layers' workspace
    cfg.n_dense_prefix = 0
    sparse = L.dv_stack_workspace_bytes(C.byref(cfg), 32)
    cfg.n_dense_prefix = 1
    assert L.dv_stack_workspace_bytes(C.byref(cfg), 32) >= sparse


def test_lookahead_sets_must_not_alias(dv):
    L = dv.lib
    cfg = dv.DecodeCfg(B=1, d=64, h=4, d_h=64, N=256, r_attn=16, r_mlp=16, k_heads=2, k_neurons=32,
                       wdt=dv.DV_F16, pred_act=1, eps=1e-5, scale=0.125, flags=dv.DV_LOOKAHEAD)
    w = dv.LayerWeights(*([P] * 16))
    st = dv.LayerState()
    st.kv = dv.KVState(P, P, 32, 5, 0, 0)
    st.head_idx_in, st.neuron_idx_in = P + 4096, P + 8192
    st.next_pa1_t = st.next_pa2_t = st.next_pm1_t = st.next_pm2_t = P
    st.next_head_idx, st.next_neuron_idx = P + 12288, P + 16384
    ok = L.dv_decode_layer(C.byref(w), C.byref(cfg), C.byref(st), P + 20480, P + 24576, 0, 0, 0)
    assert ok == 6                                   # separate buffers: only the workspace is missing
    st.next_neuron_idx = P + 8192 + 64               # inside neuron_idx_in
    assert L.dv_decode_layer(C.byref(w), C.byref(cfg), C.byref(st), P + 20480, P + 24576, P, 1 << 30, 0) == 5
    assert "overlap" in err(dv)
    st.next_neuron_idx = P + 16384
    st.next_head_idx = P + 4096                      # the same buffer as head_idx_in
    assert L.dv_decode_layer(C.byref(w), C.byref(cfg), C.byref(st), P + 20480, P + 24576, P, 1 << 30, 0) == 5


def _stack_cfg(dv, flags):
    return dv.DecodeCfg(B=1, d=64, h=4, d_h=64, N=256, r_attn=16, r_mlp=16, k_heads=2, k_neurons=32,
                        wdt=dv.DV_F16, pred_act=1, eps=1e-5, scale=0.125, flags=flags)


def test_decode_stack_validation(dv):
    L = dv.lib
    cfg = _stack_cfg(dv, dv.DV_LOOKAHEAD | dv.DV_ADVANCE_POS)
    lay = dv.StackLayer()
    lay.w = dv.LayerWeights(*([P] * 16))
    lay.kv = dv.KVState(P, P, 32, 5, 0, 0, P)
    arr = (dv.StackLayer * 3)(lay, lay, lay)
    big = 1 << 30
    assert L.dv_decode_stack(arr, 3, C.byref(cfg), 0, P, 0, 0, P, P + 4096, 0, P, big, 0) == 1     # head_sets
    assert L.dv_decode_stack(arr, 0, C.byref(cfg), P, P, 0, 0, P, P + 4096, 0, P, big, 0) == 2
    assert L.dv_decode_stack(arr, 3, C.byref(cfg), P, P, 0, 0, P, P, 0, P, big, 0) == 5           # x_out = x_in
    assert L.dv_decode_stack(arr, 3, C.byref(cfg), P, P, 0, 0, P, P + 4096, 0, P, 64, 0) == 6
    assert L.dv_stack_workspace_bytes(C.byref(cfg), 32) > L.dv_decode_workspace_bytes(C.byref(cfg), 32)
    assert L.dv_decode_stack(arr, 3, C.byref(cfg), P, P, 0, 0, P, P + 4096, P + 256, P, big, 0) == 5  # x_trace on x_in
    # a bad layer is named, and nothing is enqueued before the check
    bad = dv.StackLayer()
    bad.w = dv.LayerWeights(*([P] * 16))
    bad.kv = dv.KVState(P, P, 32, 40, 0, 0, P)        # pos past max_len
    arr2 = (dv.StackLayer * 3)(lay, lay, bad)
    assert L.dv_decode_stack(arr2, 3, C.byref(cfg), P, P + 65536, 0, 0, P, P + 4096, 0, P + (1 << 20), big, 0) == 5
    assert "layer 2" in err(dv)
    # the next layer's predictor must be there in the look-ahead form
    nopred = dv.StackLayer()
    nopred.w = dv.LayerWeights(*([P] * 12 + [0] * 4))
    nopred.kv = lay.kv
    arr3 = (dv.StackLayer * 2)(lay, nopred)
    assert L.dv_decode_stack(arr3, 2, C.byref(cfg), P, P + 65536, 0, 0, P, P + 4096, 0, P + (1 << 20), big, 0) == 1
    assert "layer 1" in err(dv)


def test_fill_normal_validation(dv):
    L = dv.lib
    assert L.dv_fill_normal(0, 10, dv.DV_F16, 1, 2, 0, 0.0, 1.0, 0) == 1
    assert L.dv_fill_normal(P, 10, 7, 1, 2, 0, 0.0, 1.0, 0) == 3
    assert L.dv_fill_normal(Q, 10, dv.DV_F32, 1, 2, 0, 0.0, 1.0, 0) == 4
    assert L.dv_fill_normal(P, 10, dv.DV_F32, 1, 2, 0, float("nan"), 1.0, 0) == 5
    assert L.dv_fill_normal(P, 10, dv.DV_F32, 1, 2, (1 << 64) - 8, 0.0, 1.0, 0) == 5
    assert L.dv_fill_normal(0, 0, dv.DV_F32, 1, 2, 0, 0.0, 1.0, 0) == 0      # nothing to write


def test_time_launches_validation(dv):
    L = dv.lib
    assert L.dv_time_launches(9, None, 0) == 3
    assert L.dv_time_launches(dv.DV_KERNEL_QKV, None, 4) == 1
    assert L.dv_time_launches(0, None, 0) == 0
    assert L.dv_launch_events_used() == 0


def test_bytes_read_matches_the_oracle_account(dv):
    """The library's byte account of a step (weights and KV read) against
    the oracle's (oracle/bytes.py, pinned to the pages' printed values)."""
    from oracle import bytes as ob
    for (d, h, N, kA, kM, n_att, rows, flags) in (
            (5120, 40, 20480, 20, 2048, 2049, 1023.5, 0),
            (9216, 72, 36864, 36, 3686, 1100, 3686, 0),
            (9216, 72, 36864, 72, 36864, 1100, 36864, dv.DV_DENSE_ATTN | dv.DV_DENSE_MLP),
            (12288, 96, 49152, 96, 4915, 513, 2000, dv.DV_DENSE_ATTN)):
        cfg = dv.DecodeCfg(B=1, d=d, h=h, d_h=128, N=N, r_attn=128, r_mlp=128, k_heads=kA, k_neurons=kM,
                           wdt=dv.DV_F16, pred_act=1, eps=1e-5, scale=0.088, flags=flags)
        b = dv.dv_bytes_read(cfg, n_att, rows, 0.0)
        ra = 0 if flags & dv.DV_DENSE_ATTN else 128
        rm = 0 if flags & dv.DV_DENSE_MLP else 128
        want = ob.decode_layer_bytes(d, h, 128, N, n_att, kA, kM, 2, r_attn=ra, r_mlp=rm, fc2_rows=rows)
        assert b.weights + b.kv_read == pytest.approx(want, rel=1e-12)
        assert b.total > b.weights + b.kv_read
    bad = dv.DecodeCfg(B=1, d=64, h=4, d_h=64, N=256, r_attn=16, r_mlp=16, k_heads=9, k_neurons=32,
                       wdt=dv.DV_F16, pred_act=1, eps=1e-5, scale=0.125, flags=0)
    with pytest.raises(dv.DVError):
        dv.dv_bytes_read(bad, 10, 10)


def test_teal_bytes_match_the_oracle_account(dv):
    """The threshold-sparse account's weight bytes against the oracle's
    (ref.teal_layer_bytes); every channel kept is the dense layer's."""
    from oracle import ref
    d, h, dh, N = 4096, 32, 128, 16384
    flags = dv.DV_DENSE_ATTN | dv.DV_DENSE_MLP | dv.DV_TEAL
    cfg = dv.DecodeCfg(B=1, d=d, h=h, d_h=dh, N=N, r_attn=128, r_mlp=128, k_heads=h, k_neurons=N,
                       wdt=dv.DV_F16, pred_act=1, eps=1e-5, scale=0.088, flags=flags)
    for kept in ((2048, 2100, 1990, 8000), (d, h * dh, d, N), (0, 0, 0, 0)):
        b = dv.dv_bytes_read_teal(cfg, 8193, kept)
        rows = {k: np.arange(int(v)) for k, v in zip(ref.TEAL_INPUTS, kept)}
        assert b.weights == pytest.approx(ref.teal_layer_bytes(d, h, dh, N, rows), rel=1e-12)
    full = dv.dv_bytes_read_teal(cfg, 8193, (d, h * dh, d, N))
    dense = dv.dv_bytes_read(dv.DecodeCfg(B=1, d=d, h=h, d_h=dh, N=N, r_attn=128, r_mlp=128, k_heads=h, k_neurons=N,
                                          wdt=dv.DV_F16, pred_act=1, eps=1e-5, scale=0.088,
                                          flags=dv.DV_DENSE_ATTN | dv.DV_DENSE_MLP), 8193, N)
    assert full.weights == pytest.approx(dense.weights, rel=1e-12) and full.kv_read == dense.kv_read
    with pytest.raises(dv.DVError):
        dv.dv_bytes_read_teal(cfg, 10, (d + 1, 0, 0, 0))
    cfg.flags = dv.DV_DENSE_ATTN | dv.DV_DENSE_MLP
    with pytest.raises(dv.DVError):
        dv.dv_bytes_read_teal(cfg, 10, (1, 1, 1, 1))


def test_sparse_mlp_noalloc_validation(dv):
    """Checked on the host before the built-in scratch is looked up; shapes
    whose scratch would exceed it are refused with a clear error."""
    L = dv.lib
    assert L.dv_sparse_mlp_noalloc(0, 1, 64, 256, P, P, P, P, dv.DV_F16, P, 32, 0, 0, P + 4096, 0, 0, 0, 0) == 1
    assert L.dv_sparse_mlp_noalloc(P, 1, 64, 256, P, P, P, P, 5, P, 32, 0, 0, P + 4096, 0, 0, 0, 0) == 3
    assert L.dv_sparse_mlp_noalloc(P, 1, 64, 256, P, P, P, P, dv.DV_F16, P, 32, 0, 0, P, 0, 0, 0, 0) == 5
    # d = 9216, 36864 rows, batch 16: far past 8 MiB of scratch
    big = L.dv_sparse_mlp_noalloc(P, 16, 9216, 36864, P, P, P, P, dv.DV_F16, P, 36864, 0, 0, P + (1 << 24),
                                  0, 0, 0, 0)
    assert big == 6 and "scratch" in err(dv)
    need = L.dv_sparse_mlp_workspace_bytes(16, 9216, 36864, dv.DV_F16)
    assert need > dv.NOALLOC_SCRATCH_BYTES
