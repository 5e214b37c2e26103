"""ctypes binding of libdv (include/dv.h): argument marshalling only.

Every function takes torch tensors already on the GPU (or None where the C
call accepts NULL), reads sizes from their shapes, passes raw device
pointers and the current HIP stream, and raises DVError on a non-zero
status.  All arithmetic happens in libdv's HIP kernels.

Importing this module fails when libdv.so has not been built; there is no
fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdv.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with "
                      "`python -m contextual_sparsity_decoding_amd.build` (hipcc, gfx950)")
lib = C.CDLL(_LIB_PATH)

DV_F32, DV_F16, DV_U32 = 0, 1, 2
DV_ACT_NONE, DV_ACT_RELU = 0, 1
DV_PROJ_QKV, DV_PROJ_OUT = 0, 1
DV_SKIP_NONPOS_FC2 = 0x1
DV_DENSE_ATTN = 0x2
DV_DENSE_MLP = 0x4
DV_HOLE_FILL = 0x8
DV_KV_SELECT = 0x10
DV_ADVANCE_POS = 0x20
DV_LOOKAHEAD = 0x40
DV_KV_WINDOW = 0x80
DV_TEAL = 0x100
DV_KERNEL_QKV, DV_KERNEL_ATTN, DV_KERNEL_OUT, DV_KERNEL_FC1, DV_KERNEL_FC2 = 1, 2, 3, 4, 5
STATUS = ["DV_OK", "DV_ERR_NULL", "DV_ERR_SHAPE", "DV_ERR_DTYPE", "DV_ERR_ALIGN", "DV_ERR_RANGE",
          "DV_ERR_WORKSPACE", "DV_ERR_UNSUPPORTED", "DV_ERR_HIP"]

vp, ci, cf, cu, sz = C.c_void_p, C.c_int, C.c_float, C.c_uint, C.c_size_t


class KVState(C.Structure):
    _fields_ = [("k_cache", vp), ("v_cache", vp), ("max_len", ci), ("pos", ci),
                ("y_buf", vp), ("valid_upto", vp), ("pos_dev", vp)]


class KVView(C.Structure):
    _fields_ = [("k_cache", vp), ("v_cache", vp), ("h", ci), ("max_len", ci), ("n_ctx", ci),
                ("sel_idx", vp), ("sel_len", vp), ("sel_cap", ci), ("sel_end", ci), ("n_ctx_dev", vp),
                ("win_sink", ci), ("win_len", ci)]


class DecodeCfg(C.Structure):
    _fields_ = [("B", ci), ("d", ci), ("h", ci), ("d_h", ci), ("N", ci), ("r_attn", ci), ("r_mlp", ci),
                ("k_heads", ci), ("k_neurons", ci), ("wdt", ci), ("pred_act", ci), ("eps", cf),
                ("scale", cf), ("flags", cu), ("win_sink", ci), ("win_len", ci), ("n_dense_prefix", ci)]


class LayerWeights(C.Structure):
    _fields_ = [(n, vp) for n in ("ln1_g", "ln1_b", "ln2_g", "ln2_b", "w_qkv_t", "b_qkv", "w_o_t", "b_o",
                                  "w1_t", "b1", "w2_t", "b2", "pa1_t", "pa2_t", "pm1_t", "pm2_t",
                                  "w_qkv_in", "w1_in")]


class LayerState(C.Structure):
    _fields_ = [("kv", KVState), ("sel_idx", vp), ("sel_len", vp), ("sel_cap", ci), ("sel_end", ci),
                ("head_idx_out", vp), ("neuron_idx_out", vp), ("neuron_count_out", vp),
                ("fc2_rows_out", vp),
                # DV_LOOKAHEAD
                ("head_idx_in", vp), ("neuron_idx_in", vp),
                ("next_pa1_t", vp), ("next_pa2_t", vp), ("next_pm1_t", vp), ("next_pm2_t", vp),
                ("next_head_idx", vp), ("next_neuron_idx", vp),
                ("aux_stream", vp), ("ev_fork", vp), ("ev_join", vp),
                # DV_TEAL
                ("teal_thr", cf * 4), ("teal_rows_out", vp), ("teal_rec", vp)]


class StackLayer(C.Structure):
    _fields_ = [("w", LayerWeights), ("kv", KVState), ("sel_idx", vp), ("sel_len", vp), ("sel_cap", ci),
                ("sel_end", ci), ("teal_thr", cf * 4), ("teal_rows_out", vp), ("teal_rec", vp)]


class Bytes(C.Structure):
    _fields_ = [(n, C.c_double) for n in ("head_pred", "neuron_pred", "qkv", "out_proj", "fc1", "fc2", "weights",
                                          "kv_read", "kv_write", "act", "total")]


def _sig(name, restype, *argtypes):
    f = getattr(lib, name)
    f.restype = restype
    f.argtypes = list(argtypes)
    return f


_sig("dv_api_version", ci)
_sig("dv_status_str", C.c_char_p, ci)
_sig("dv_last_error", C.c_char_p)
_sig("dv_layernorm", ci, vp, ci, ci, vp, vp, cf, vp, vp)
_sig("dv_predict_workspace_bytes", sz, ci, ci, ci, ci)
_sig("dv_predict", ci, vp, ci, ci, vp, ci, vp, ci, ci, ci, vp, vp, sz, vp)
_sig("dv_topk_workspace_bytes", sz, ci, ci, ci)
_sig("dv_topk_select", ci, vp, ci, ci, ci, vp, vp, vp, vp, sz, vp)
_sig("dv_sparse_mlp_workspace_bytes", sz, ci, ci, ci, ci)
_sig("dv_sparse_mlp", ci, vp, ci, ci, ci, vp, vp, vp, vp, ci, vp, ci, vp, vp, vp, vp, vp, cu, vp, sz, vp)
_sig("dv_sparse_mlp_noalloc", ci, vp, ci, ci, ci, vp, vp, vp, vp, ci, vp, ci, vp, vp, vp, vp, vp, cu, vp)
_sig("dv_attn_proj_workspace_bytes", sz, ci, ci, ci, ci, ci, ci, ci)
_sig("dv_sparse_attn_proj", ci, ci, ci, ci, ci, ci, vp, ci, vp, vp, ci, vp, vp, vp, C.POINTER(KVState), vp, sz, vp)
_sig("dv_splitk_workspace_bytes", sz, ci, ci, ci, ci, ci)
_sig("dv_splitk_attn", ci, vp, ci, ci, vp, ci, C.POINTER(KVView), cf, ci, vp, vp, sz, vp)
_sig("dv_kv_score_workspace_bytes", sz, ci, ci, ci, ci)
_sig("dv_kv_score", ci, vp, ci, ci, ci, ci, C.POINTER(KVView), cf, ci, ci, ci, vp, vp, sz, vp)
_sig("dv_decode_workspace_bytes", sz, C.POINTER(DecodeCfg), ci)
_sig("dv_decode_layer", ci, C.POINTER(LayerWeights), C.POINTER(DecodeCfg), C.POINTER(LayerState), vp, vp, vp, sz, vp)
_sig("dv_stack_workspace_bytes", sz, C.POINTER(DecodeCfg), ci)
_sig("dv_decode_stack", ci, C.POINTER(StackLayer), ci, C.POINTER(DecodeCfg), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp)
_sig("dv_fill_normal", ci, vp, C.c_uint64, ci, C.c_uint64, C.c_uint64, C.c_uint64, cf, cf, vp)
_sig("dv_bytes_read", ci, C.POINTER(DecodeCfg), C.c_double, C.c_double, C.c_double, C.POINTER(Bytes))
_sig("dv_bytes_read_teal", ci, C.POINTER(DecodeCfg), C.c_double, C.POINTER(C.c_double), C.POINTER(Bytes))
_sig("dv_quantize_w4", ci, vp, ci, ci, vp, vp, vp)
_sig("dv_sparse_mlp_w4_workspace_bytes", sz, ci, ci)
_sig("dv_sparse_mlp_w4", ci, vp, ci, ci, vp, vp, vp, vp, vp, vp, vp, ci, vp, vp, vp, vp, vp, cu, vp, sz, vp)
_sig("dv_time_launches", ci, ci, C.POINTER(vp), ci)
_sig("dv_launch_events_used", ci)

EXPORTS = ("dv_api_version", "dv_status_str", "dv_last_error", "dv_layernorm", "dv_predict_workspace_bytes",
           "dv_predict", "dv_topk_workspace_bytes", "dv_topk_select", "dv_sparse_mlp_workspace_bytes",
           "dv_sparse_mlp", "dv_attn_proj_workspace_bytes", "dv_sparse_attn_proj", "dv_splitk_workspace_bytes",
           "dv_splitk_attn", "dv_kv_score_workspace_bytes", "dv_kv_score", "dv_decode_workspace_bytes",
           "dv_decode_layer", "dv_stack_workspace_bytes", "dv_decode_stack", "dv_fill_normal", "dv_bytes_read",
           "dv_bytes_read_teal", "dv_quantize_w4", "dv_sparse_mlp_w4_workspace_bytes",
           "dv_sparse_mlp_w4", "dv_time_launches", "dv_launch_events_used", "dv_sparse_mlp_noalloc")


class DVError(RuntimeError):
    def __init__(self, name: str, status: int):
        self.status = status
        msg = lib.dv_last_error().decode()
        super().__init__(f"{name}: {STATUS[status] if 0 <= status < len(STATUS) else status}: {msg}")


def _check(name: str, st: int) -> None:
    if st != 0:
        raise DVError(name, st)


def ptr(t: Optional[torch.Tensor]) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError("libdv takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libdv takes contiguous tensors")
    return t.data_ptr()


def stream_handle(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream if hasattr(s, "cuda_stream") else int(s)


def wdt_of(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return DV_F16
    if t.dtype == torch.float32:
        return DV_F32
    raise ValueError(f"weights must be fp16 or fp32, got {t.dtype}")


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace of at least ``nbytes`` (the library keeps it zeroed)."""
    return torch.zeros(max(256, int(nbytes)), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- calls ------

def dv_api_version() -> int:
    return lib.dv_api_version()


def dv_layernorm(x, gamma, beta, eps, y, stream=None):
    B, d = x.shape
    _check("dv_layernorm", lib.dv_layernorm(ptr(x), B, d, ptr(gamma), ptr(beta), eps, ptr(y), stream_handle(stream)))


def dv_predict_workspace_bytes(B, d, r, wdt) -> int:
    return lib.dv_predict_workspace_bytes(B, d, r, wdt)


def dv_predict(y, p1_t, p2_t, act, scores, ws, stream=None):
    B, d = y.shape
    r = p1_t.shape[0]
    n_out = p2_t.shape[0]
    _check("dv_predict", lib.dv_predict(ptr(y), B, d, ptr(p1_t), r, ptr(p2_t), n_out, wdt_of(p1_t), act,
                                        ptr(scores), ptr(ws), ws.numel() if ws is not None else 0,
                                        stream_handle(stream)))


def dv_topk_select(scores, k, idx, union_idx=None, union_count=None, stream=None):
    B, n = scores.shape
    _check("dv_topk_select", lib.dv_topk_select(ptr(scores), B, n, k, ptr(idx), ptr(union_idx), ptr(union_count),
                                                0, 0, stream_handle(stream)))


def dv_sparse_mlp_workspace_bytes(B, d, n_idx_max, wdt) -> int:
    return lib.dv_sparse_mlp_workspace_bytes(B, d, n_idx_max, wdt)


def dv_sparse_mlp(y, w1_t, b1, w2_t, b2, idx, n_idx_max, out, ws, *, n_idx_dev=None, residual=None,
                  act_out=None, fc2_rows=None, flags=0, stream=None):
    B, d = y.shape
    N = w1_t.shape[0]
    _check("dv_sparse_mlp", lib.dv_sparse_mlp(
        ptr(y), B, d, N, ptr(w1_t), ptr(b1), ptr(w2_t), ptr(b2), wdt_of(w1_t), ptr(idx), n_idx_max, ptr(n_idx_dev),
        ptr(residual), ptr(out), ptr(act_out), ptr(fc2_rows), flags, ptr(ws), ws.numel(), stream_handle(stream)))


NOALLOC_SCRATCH_BYTES = 8 << 20


def dv_sparse_mlp_noalloc(y, w1_t, b1, w2_t, b2, idx, n_idx_max, out, *, n_idx_dev=None, residual=None,
                          act_out=None, fc2_rows=None, flags=0, stream=None):
    """dv_sparse_mlp with the library's built-in scratch instead of a workspace."""
    B, d = y.shape
    N = w1_t.shape[0]
    _check("dv_sparse_mlp_noalloc", lib.dv_sparse_mlp_noalloc(
        ptr(y), B, d, N, ptr(w1_t), ptr(b1), ptr(w2_t), ptr(b2), wdt_of(w1_t), ptr(idx), n_idx_max, ptr(n_idx_dev),
        ptr(residual), ptr(out), ptr(act_out), ptr(fc2_rows), flags, stream_handle(stream)))


def kv_state(K, V, pos, y_buf=None, valid_upto=None, pos_dev=None) -> KVState:
    s = KVState(ptr(K), ptr(V), K.shape[2], pos, ptr(y_buf), ptr(valid_upto), ptr(pos_dev))
    s._keep = (K, V, y_buf, valid_upto, pos_dev)   # the struct holds raw pointers: keep the tensors alive
    return s


def kv_view(K, V, n_ctx, sel_idx=None, sel_len=None, sel_end=0, n_ctx_dev=None, win_sink=0,
            win_len=0) -> KVView:
    cap = sel_idx.shape[-1] if sel_idx is not None else 0
    v = KVView(ptr(K), ptr(V), K.shape[1], K.shape[2], n_ctx, ptr(sel_idx), ptr(sel_len), cap, sel_end,
               ptr(n_ctx_dev), win_sink, win_len)
    v._keep = (K, V, sel_idx, sel_len, n_ctx_dev)
    return v


def dv_attn_proj_workspace_bytes(mode, B, d, h, d_h, n_sel, wdt) -> int:
    return lib.dv_attn_proj_workspace_bytes(mode, B, d, h, d_h, n_sel, wdt)


def dv_sparse_attn_proj(mode, h, d_h, head_idx, n_sel, w_t, bias, inp, out, ws, *, residual=None, kv=None,
                        stream=None):
    B = inp.shape[0]
    d = w_t.shape[-1]
    kvp = C.byref(kv) if kv is not None else None
    _check("dv_sparse_attn_proj", lib.dv_sparse_attn_proj(
        mode, B, d, h, d_h, ptr(head_idx), n_sel, ptr(w_t), ptr(bias), wdt_of(w_t), ptr(inp), ptr(residual),
        ptr(out), kvp, ptr(ws), ws.numel() if ws is not None else 0, stream_handle(stream)))


def dv_splitk_workspace_bytes(B, n_sel, d_h, max_positions, num_splits=0) -> int:
    return lib.dv_splitk_workspace_bytes(B, n_sel, d_h, max_positions, num_splits)


def dv_splitk_attn(q, head_idx, n_sel, view: KVView, scale, o, ws, num_splits=0, stream=None):
    B, _, d_h = q.shape
    _check("dv_splitk_attn", lib.dv_splitk_attn(ptr(q), B, d_h, ptr(head_idx), n_sel, C.byref(view), scale,
                                                num_splits, ptr(o), ptr(ws), ws.numel(), stream_handle(stream)))


def dv_kv_score_workspace_bytes(B, h, n, n_obs) -> int:
    return lib.dv_kv_score_workspace_bytes(B, h, n, n_obs)


def dv_kv_score(q_obs, view: KVView, scale, n_sink, n_window, width, scores, ws, stream=None):
    B, h, n_obs, d_h = q_obs.shape
    _check("dv_kv_score", lib.dv_kv_score(ptr(q_obs), B, h, d_h, n_obs, C.byref(view), scale, n_sink, n_window,
                                          width, ptr(scores), ptr(ws), ws.numel(), stream_handle(stream)))


def layer_weights(W: dict) -> LayerWeights:
    """LayerWeights from a dict of device tensors (keys as in synth.layer_weights)."""
    w = LayerWeights(*[ptr(W.get(n)) for n, _ in LayerWeights._fields_])
    w._keep = dict(W)
    return w


def decode_cfg(**kw) -> DecodeCfg:
    return DecodeCfg(**kw)


def dv_decode_workspace_bytes(cfg: DecodeCfg, max_len: int) -> int:
    return lib.dv_decode_workspace_bytes(C.byref(cfg), max_len)


def dv_decode_layer(wts: LayerWeights, cfg: DecodeCfg, st: LayerState, x_in, x_out, ws, stream=None):
    _check("dv_decode_layer", lib.dv_decode_layer(C.byref(wts), C.byref(cfg), C.byref(st), ptr(x_in), ptr(x_out),
                                                  ptr(ws), ws.numel(), stream_handle(stream)))


def dv_stack_workspace_bytes(cfg: DecodeCfg, max_len: int) -> int:
    return lib.dv_stack_workspace_bytes(C.byref(cfg), max_len)


def stack_layers(layers) -> "C.Array":
    """A C array of StackLayer from a sequence of them (kept alive by the array)."""
    arr = (StackLayer * len(layers))(*layers)
    arr._keep = list(layers)
    return arr


def dv_decode_stack(layers, cfg: DecodeCfg, x_in, x_out, ws, *, head_sets=None, neuron_sets=None,
                    neuron_counts=None, fc2_rows=None, x_trace=None, stream=None):
    _check("dv_decode_stack", lib.dv_decode_stack(
        layers, len(layers), C.byref(cfg), ptr(head_sets), ptr(neuron_sets), ptr(neuron_counts), ptr(fc2_rows),
        ptr(x_in), ptr(x_out), ptr(x_trace), ptr(ws), ws.numel(), stream_handle(stream)))


def dv_fill_normal(out, seed: int, stream_id: int, offset: int = 0, mean: float = 0.0, std: float = 1.0,
                   raw: bool = False, stream=None):
    """Fill ``out`` (fp16 or fp32; int32 with ``raw``) with the seeded normal stream (seed, stream_id)."""
    if raw:
        dt = DV_U32
        if out.dtype != torch.int32:
            raise ValueError("raw words go to an int32 tensor")
    else:
        dt = wdt_of(out)
    _check("dv_fill_normal", lib.dv_fill_normal(ptr(out), out.numel(), dt, seed, stream_id, offset, mean, std,
                                                stream_handle(stream)))


def dv_bytes_read(cfg: DecodeCfg, n_att: float, fc2_rows: float, holes: float = 0.0) -> Bytes:
    b = Bytes()
    _check("dv_bytes_read", lib.dv_bytes_read(C.byref(cfg), n_att, fc2_rows, holes, C.byref(b)))
    return b


def dv_bytes_read_teal(cfg: DecodeCfg, n_att: float, kept) -> Bytes:
    b = Bytes()
    k = (C.c_double * 4)(*[float(v) for v in kept])
    _check("dv_bytes_read_teal", lib.dv_bytes_read_teal(C.byref(cfg), n_att, k, C.byref(b)))
    return b


def dv_quantize_w4(w, q, scales, stream=None):
    """w fp16 [rows][cols] -> q uint8 [rows][cols / 2], scales fp16 [rows][cols / 128]."""
    rows, cols = w.shape
    _check("dv_quantize_w4", lib.dv_quantize_w4(ptr(w), rows, cols, ptr(q), ptr(scales), stream_handle(stream)))


def dv_sparse_mlp_w4(y, N, q1, s1, b1, q2, s2, b2, idx, out, ws, *, n_idx_max=None, n_idx_dev=None, residual=None,
                     act_out=None, fc2_rows=None, flags=0, stream=None):
    d = y.shape[-1]
    n = n_idx_max if n_idx_max is not None else (idx.numel() if idx is not None else N)
    _check("dv_sparse_mlp_w4", lib.dv_sparse_mlp_w4(ptr(y), d, N, ptr(q1), ptr(s1), ptr(b1), ptr(q2), ptr(s2), ptr(b2),
                                                    ptr(idx), n, ptr(n_idx_dev), ptr(residual), ptr(out),
                                                    ptr(act_out), ptr(fc2_rows), flags, ptr(ws), ws.numel(),
                                                    stream_handle(stream)))


class LaunchTimer:
    """Events around each launch of one kernel role (dv_time_launches) on this thread.

    Use as a context manager around calls of dv_decode_layer / dv_decode_stack;
    ``durations_ms()`` afterwards (once the work has run) gives one duration
    per timed launch."""

    def __init__(self, kernel: int, max_launches: int):
        self.kernel = kernel
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * max_launches)]
        for e in self.events:          # materialise the HIP events
            e.record()
        torch.cuda.synchronize()
        self._arr = (vp * len(self.events))(*[e.cuda_event for e in self.events])
        self.used = 0

    def __enter__(self):
        _check("dv_time_launches", lib.dv_time_launches(self.kernel, self._arr, len(self.events)))
        return self

    def __exit__(self, *exc):
        self.used = lib.dv_launch_events_used()
        lib.dv_time_launches(0, None, 0)
        return False

    def durations_ms(self):
        torch.cuda.synchronize()
        return [self.events[2 * i].elapsed_time(self.events[2 * i + 1]) for i in range(self.used // 2)]
