"""A decoder stack generated on the device and run one token at a time.

Weights, biases, predictors and the seeded K/V caches of every layer are
written by the library's own generator (dv_fill_normal), so stacks of
100+ GB never pass through host memory; ``synth.stack_layer_weights`` and
``synth.philox_tensor`` regenerate any of them on the host.  Streams: tensor
``name`` of layer ``l`` is ``synth.stream_id(l, name)`` under the stack's
seed.  Weights and biases ~ N(0, 0.02^2), caches ~ N(0, 1) (every slot,
the filled ones being positions < n_ctx), LayerNorm gain 1 and bias 0.

This module allocates device memory and marshals arguments; every step of
the decode runs in libdv (dv_decode_stack).
"""
from __future__ import annotations

import copy
import math
from typing import List, Optional

import torch

from . import dv, synth
from .configs import LayerDims


class Stack:
    """``layers`` decoder layers of shape ``dims`` on the current device.

    One decode position (``pos_dev``) is shared by every layer; it starts at
    ``n_ctx`` and moves on by one per token (DV_ADVANCE_POS).  ``hole_fill``
    allocates each layer's stored inputs and valid positions (DejaVu §4.2).
    """

    def __init__(self, dims: LayerDims, layers: int, n_ctx: int, max_len: int, seed: int, batch: int = 1,
                 hole_fill: bool = True, teal: bool = False):
        self.dims, self.L, self.n_ctx, self.max_len, self.seed, self.B = dims, layers, n_ctx, max_len, seed, batch
        wdt = torch.float16 if dims.wdt == "f16" else torch.float32
        shapes = synth.stack_tensor_shapes(dims)
        self.W: List[dict] = []
        self.K: List[torch.Tensor] = []
        self.V: List[torch.Tensor] = []
        self.y_buf: List[Optional[torch.Tensor]] = []
        self.valid: List[Optional[torch.Tensor]] = []
        one = torch.ones(dims.d, device="cuda")
        zero = torch.zeros(dims.d, device="cuda")
        for l in range(layers):
            w = {}
            for name, shp in shapes.items():
                t = torch.empty(shp, dtype=wdt, device="cuda")
                dv.dv_fill_normal(t, seed, synth.stream_id(l, name), std=synth.WEIGHT_STD)
                w[name] = t
            w.update(ln1_g=one, ln1_b=zero, ln2_g=one, ln2_b=zero)
            if teal:   # input-major copies for threshold sparsity (a layout change, no arithmetic)
                w["w_qkv_in"] = w["w_qkv_t"].reshape(3 * dims.h * dims.d_h, dims.d).t().contiguous()
                w["w1_in"] = w["w1_t"].t().contiguous()
            self.W.append(w)
            for name, lst in (("K", self.K), ("V", self.V)):
                t = torch.empty(batch, dims.h, max_len, dims.d_h, dtype=torch.float16, device="cuda")
                dv.dv_fill_normal(t, seed, synth.stream_id(l, name))
                lst.append(t)
            self.y_buf.append(torch.zeros(batch, max_len, dims.d, device="cuda") if hole_fill else None)
            self.valid.append(torch.full((batch, dims.h), n_ctx - 1, dtype=torch.int32, device="cuda")
                              if hole_fill else None)
        self.hole_fill = hole_fill
        self.pos_dev = torch.full((1,), n_ctx, dtype=torch.int32, device="cuda")
        self.wts = [dv.layer_weights(w) for w in self.W]
        self.sel = [None] * layers          # DV_KV_SELECT: (sel_idx, sel_len, sel_end) per layer
        self.teal_thr = [(-1.0,) * 4] * layers   # DV_TEAL thresholds per layer (-1: every channel)
        self.teal_rows = torch.zeros(4, dtype=torch.int32, device="cuda") if teal else None
        self.teal_rec = None                # DV_TEAL: per-layer records of the projection inputs
        self._arr = None

    def set_context(self, n_ctx: int, max_len: int) -> None:
        """New caches of max_len slots per layer with n_ctx positions filled
        (the weights stay); clears any KV selection."""
        d = self.dims
        self.K, self.V, self._arr = [], [], None
        self.sel = [None] * self.L
        torch.cuda.empty_cache()
        for l in range(self.L):
            for name, lst in (("K", self.K), ("V", self.V)):
                t = torch.empty(self.B, d.h, max_len, d.d_h, dtype=torch.float16, device="cuda")
                dv.dv_fill_normal(t, self.seed, synth.stream_id(l, name))
                lst.append(t)
            if self.hole_fill:
                self.y_buf[l] = torch.zeros(self.B, max_len, d.d, device="cuda")
                self.valid[l] = torch.full((self.B, d.h), n_ctx - 1, dtype=torch.int32, device="cuda")
        self.n_ctx, self.max_len = n_ctx, max_len
        self.reset()

    def select_kv(self, budget: int, n_obs: int = 64, n_sink: int = 4, width: int = 7) -> None:
        """ByteCross §4.1 / App. A, once per layer after the seeded prompt: the
        positions the last n_obs prompt queries (seeded N(0,1) fp16, one set
        per layer) attend to most, smoothed, with the sinks and the
        observation window forced in; the top `budget` per head are kept and
        every position from n_ctx on (the decoded tokens) is always read."""
        d, n = self.dims, self.n_ctx
        scale = 1 / math.sqrt(d.d_h)
        q = torch.empty(self.B, d.h, n_obs, d.d_h, dtype=torch.float16, device="cuda")
        scores = torch.empty(self.B, d.h, n, device="cuda")
        ws = dv.workspace(dv.dv_kv_score_workspace_bytes(self.B, d.h, n, n_obs))
        for l in range(self.L):
            dv.dv_fill_normal(q, self.seed, synth.stream_id(l, "q_obs"))
            view = dv.kv_view(self.K[l], self.V[l], n)
            dv.dv_kv_score(q, view, scale, n_sink, n_obs, width, scores, ws)
            idx = torch.empty(self.B, d.h, budget, dtype=torch.int32, device="cuda")
            dv.dv_topk_select(scores.view(self.B * d.h, n), budget, idx.view(self.B * d.h, budget))
            lens = torch.full((self.B, d.h), budget, dtype=torch.int32, device="cuda")
            self.sel[l] = (idx, lens, n)
        self._arr = None

    def batch_view(self, B: int) -> "Stack":
        """The same layers with the first B sequences' caches (the stack's
        batch is the caches' outermost dimension), sharing the decode position."""
        if not 1 <= B <= self.B:
            raise ValueError(f"batch {B} outside [1, {self.B}]")
        v = copy.copy(self)
        v.B = B
        v.K = [k[:B] for k in self.K]
        v.V = [t[:B] for t in self.V]
        v.y_buf = [y[:B] if y is not None else None for y in self.y_buf]
        v.valid = [t[:B] if t is not None else None for t in self.valid]
        v.sel = [None] * self.L
        v._arr = None
        return v

    def reset(self) -> None:
        """Back to the seeded state: position n_ctx, every head valid up to n_ctx - 1
        (slots past n_ctx - 1 are rewritten before they are read)."""
        self.pos_dev.fill_(self.n_ctx)
        for v in self.valid:
            if v is not None:
                v.fill_(self.n_ctx - 1)

    def set_kv_selection(self, layer: int, sel_idx: torch.Tensor, sel_len: torch.Tensor, sel_end: int) -> None:
        self.sel[layer] = (sel_idx, sel_len, sel_end)
        self._arr = None

    def layers_array(self):
        """The C array of dv_stack_layer (built once, reused by every call)."""
        if self._arr is None:
            items = []
            for l in range(self.L):
                sl = dv.StackLayer()
                sl.w = self.wts[l]
                # kv.pos is only the bound of the device position
                sl.kv = dv.kv_state(self.K[l], self.V[l], self.max_len - 1, self.y_buf[l], self.valid[l], self.pos_dev)
                if self.sel[l] is not None:
                    si, sn, se = self.sel[l]
                    sl.sel_idx, sl.sel_len, sl.sel_cap, sl.sel_end = si.data_ptr(), sn.data_ptr(), si.shape[-1], se
                    sl._keep_sel = (si, sn)
                for i, t in enumerate(self.teal_thr[l]):
                    sl.teal_thr[i] = t
                if self.teal_rows is not None:
                    sl.teal_rows_out = self.teal_rows.data_ptr()
                if self.teal_rec is not None:
                    sl.teal_rec = self.teal_rec[l].data_ptr()
                items.append(sl)
            self._arr = dv.stack_layers(items)
        return self._arr

    def calibrate_teal(self, keep: float, X: torch.Tensor, ws: torch.Tensor, cfg: dv.DecodeCfg) -> None:
        """Threshold sparsity's thresholds from seeded activations: the stack
        decodes the tokens X [T][B][d] with every channel kept (cfg carries
        DV_TEAL; the decode state is reset before and after), recording each
        layer's four projection inputs; each threshold is the (1 - keep)
        quantile of that input's magnitudes over the tokens, so that a
        fraction `keep` of the calibration entries exceeds it."""
        d = self.dims
        width = max(d.d, d.h * d.d_h, d.N)
        T = X.shape[0]
        rec = [torch.zeros(4, self.B, width, device="cuda") for _ in range(self.L)]
        mags = [[[] for _ in range(4)] for _ in range(self.L)]
        widths = (d.d, d.h * d.d_h, d.d, d.N)
        self.teal_thr = [(-1.0,) * 4] * self.L
        self.teal_rec, self._arr = rec, None
        self.reset()
        x_out = torch.empty(self.B, d.d, device="cuda")
        x_trace = torch.empty(max(1, self.L - 1), self.B, d.d, device="cuda")
        for t in range(T):
            dv.dv_decode_stack(self.layers_array(), cfg, X[t], x_out, ws, x_trace=x_trace)
            for l in range(self.L):
                for i in range(4):
                    mags[l][i].append(rec[l][i, :, :widths[i]].abs().flatten().clone())
        torch.cuda.synchronize()
        thr = []
        for l in range(self.L):
            thr.append(tuple(float(torch.quantile(torch.cat(mags[l][i]), 1.0 - keep)) for i in range(4)))
        self.teal_thr, self.teal_rec, self._arr = thr, None, None
        self.reset()

    def cfg(self, k_heads: int, k_neurons: int, flags: int, scale: float, eps: float = 1e-5,
            pred_act: int = dv.DV_ACT_RELU) -> dv.DecodeCfg:
        d = self.dims
        dense_a = bool(flags & dv.DV_DENSE_ATTN)
        dense_m = bool(flags & dv.DV_DENSE_MLP)
        return dv.decode_cfg(B=self.B, d=d.d, h=d.h, d_h=d.d_h, N=d.N, r_attn=d.r_attn, r_mlp=d.r_mlp,
                             k_heads=d.h if dense_a else k_heads, k_neurons=d.N if dense_m else k_neurons,
                             wdt=dv.DV_F16 if d.wdt == "f16" else dv.DV_F32, pred_act=pred_act, eps=eps,
                             scale=scale, flags=flags)
