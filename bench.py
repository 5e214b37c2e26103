"""Benchmark: sparse decode of a 64-layer OPT-66B-shaped stack on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers L]

The workload is the one the metric is quoted on: 64 decoder layers of
OPT-66B shape (d = 9216, 72 heads x 128, d_ffn = 36864 ReLU), fp16 weights
with fp32 accumulation (about 131 GB resident, generated on the device by
the library's seeded generator), batch 1, a 1024-token KV cache per layer,
36 of 72 heads and a neuron keep ratio of 10% selected by rank-128
predictors.  A step is one token through all 64 layers.  The schedule is
DejaVu §4.3's parallel form: layer l runs on the sets layer l-1 predicted
from its input, and predicts layer l+1's sets inside its own launches; the
first layer's sets come from its own predictors.  Hole fill (§4.2) and the
fc2 skip of non-positive neurons are on.

Each configuration decodes from the same seeded state: W untimed warm-up
tokens, then K timed tokens (W + K <= 128, within the 128-token decode),
each one replay of a HIP graph of the whole stack (the next token's input is
copied in before each replay, inside the timed region).

Prints one JSON line: stack tokens/s at 10% neurons, effective HBM
bandwidth on the bytes the step must read, the neuron keep sweep
{5, 10, 25, 50, 100}% with the same library's dense path (every head and
neuron, every fc2 row) and the byte-bound speedups, the sequential schedule,
the dominant kernel's roofline measured on its launches inside the step, and
the CPU oracle timed on a sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
SEED = 1234
DECODE_TOKENS = 128


_T0 = time.perf_counter()


def progress(msg: str) -> None:
    """One line per finished phase on stderr (the JSON line stays alone on stdout)."""
    print(f"[bench {time.perf_counter() - _T0:7.1f}s] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=64, help="timed tokens (after the warm-up, within 128)")
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--layers", type=int, default=64)
    p.add_argument("--sweep", type=int, default=1, help="0 skips the keep sweep and the sequential schedule")
    p.add_argument("--dense", type=int, default=1, help="0 skips the dense path (profiling runs)")
    p.add_argument("--longctx", type=int, default=1,
                   help="0 skips the long-context composition stack (32 layers, d=4096, 2K-128K context)")
    p.add_argument("--batched", type=int, default=1,
                   help="0 skips the batched OPT-175B-share stack (48 layers, d=12288, batch 1-16)")
    p.add_argument("--batch-sizes", type=str, default="",
                   help="comma-separated batch sizes of the batched stack (default: all of them)")
    p.add_argument("--w4", type=int, default=1,
                   help="0 skips the 4-bit-weight sparse MLP (OPT-66B width, fp16 against 4-bit weights)")
    p.add_argument("--extra-steps", type=int, default=12, help="timed tokens per point of the two extra stacks")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU time per oracle timing (two timings)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="copy this many MiB device to device three times before the timed runs "
                        "(a copy of known size for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return p.parse_args()


# The sources the dominant kernel (k_qkv at batch 1, fp16) is compiled from:
# its traffic summary in profiles/ is used only while they are unchanged.
QKV_SOURCES = ("qkv.h", "pred.h", "rowdot.h", "dv_internal.h", "k_qkv.hip", "k_qkv_f16_b1.hip")


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "contextual_sparsity_decoding_amd", "csrc")
    for f in QKV_SOURCES:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_traffic(name: str, digest: str):
    """HBM bytes per launch from a committed PMC summary, if it was taken on
    the current kernel sources."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_sources") != digest:
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_info():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


class StackRun:
    """Graph-replayed decode of the stack, one token per replay."""

    def __init__(self, torch, dv, stack, X, ws, head_sets, neuron_sets, fc2_rows):
        self.torch, self.dv, self.st, self.X, self.ws = torch, dv, stack, X, ws
        self.head_sets, self.neuron_sets, self.fc2_rows = head_sets, neuron_sets, fc2_rows
        d = stack.dims.d
        self.x_cur = torch.empty(1, d, device="cuda")
        self.x_out = torch.empty(1, d, device="cuda")

    def call(self, cfg):
        self.dv.dv_decode_stack(self.st.layers_array(), cfg, self.x_cur, self.x_out, self.ws,
                                head_sets=self.head_sets, neuron_sets=self.neuron_sets, fc2_rows=self.fc2_rows)

    def run(self, cfg, warm, timed):
        """Decode warm + timed tokens from the seeded state; returns (ms per timed token,
        fc2 rows read per layer per timed token)."""
        torch = self.torch
        self.st.reset()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.call(cfg)
        for t in range(warm):
            self.x_cur.copy_(self.X[t])
            g.replay()
        torch.cuda.synchronize()
        self.fc2_rows.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for t in range(warm, warm + timed):
            self.x_cur.copy_(self.X[t])
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / timed
        rows = int(self.fc2_rows.item()) / (timed * self.st.L)
        del g
        return ms, rows

    def time_kernel(self, cfg, kernel, tokens, warm=2):
        """Durations of every launch of one kernel role inside `tokens` decode
        tokens run eagerly (events recorded by the library around each launch;
        the host keeps ahead of the GPU, so the launches queue back to back)."""
        torch = self.torch
        self.st.reset()
        for t in range(warm):
            self.x_cur.copy_(self.X[t])
            self.call(cfg)
        timer = self.dv.LaunchTimer(kernel, tokens * self.st.L)
        with timer:
            for t in range(warm, warm + tokens):
                self.x_cur.copy_(self.X[t])
                self.call(cfg)
        torch.cuda.synchronize()
        return timer.durations_ms()


def step_bytes(dv, cfg, L, n_att, fc2_rows):
    b = dv.dv_bytes_read(cfg, n_att, fc2_rows, 0.0)
    return b, L * b.total


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from contextual_sparsity_decoding_amd import configs, dv, synth
    from contextual_sparsity_decoding_amd.stack import Stack

    wl = configs.OPT66B_STACK
    dims = wl.dims
    L = args.layers
    W = max(0, args.warmup)
    K = max(1, min(args.steps, DECODE_TOKENS - W))
    max_len = wl.n_ctx + DECODE_TOKENS + 8
    scale = 1 / math.sqrt(dims.d_h)
    torch.cuda.set_device(0)

    t0 = time.perf_counter()
    stack = Stack(dims, L, wl.n_ctx, max_len, SEED)
    X = torch.empty(DECODE_TOKENS, 1, dims.d, device="cuda")
    dv.dv_fill_normal(X, SEED, synth.stream_id(0, "x"))
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t0
    progress(f"generated the {L}-layer stack in {gen_s:.1f} s")
    resident = sum(t.numel() * t.element_size() for w in stack.W for k, t in w.items() if k[:2] not in ("ln",))

    sparse_flags = dv.DV_HOLE_FILL | dv.DV_SKIP_NONPOS_FC2 | dv.DV_ADVANCE_POS
    sweep_keep = (0.05, 0.10, 0.25, 0.50, 1.00)
    k_of = {k: int(math.floor(k * dims.N)) for k in sweep_keep}
    head_k = wl.k_heads
    ahead_cfg = lambda kn: stack.cfg(head_k, kn, sparse_flags | dv.DV_LOOKAHEAD, scale)
    seq_cfg = stack.cfg(head_k, k_of[0.10], sparse_flags, scale)
    dense_cfg = stack.cfg(dims.h, dims.N, dv.DV_DENSE_ATTN | dv.DV_DENSE_MLP | dv.DV_ADVANCE_POS, scale)
    cfgs = [ahead_cfg(k_of[k]) for k in sweep_keep] + [seq_cfg, dense_cfg]
    ws = dv.workspace(max(dv.dv_stack_workspace_bytes(c, max_len) for c in cfgs))
    head_sets = torch.zeros(L, dims.h, dtype=torch.int32, device="cuda")
    neuron_sets = torch.zeros(L, dims.N, dtype=torch.int32, device="cuda")
    fc2_rows = torch.zeros(1, dtype=torch.int32, device="cuda")
    run = StackRun(torch, dv, stack, X, ws, head_sets, neuron_sets, fc2_rows)
    n_att = wl.n_ctx + W + (K - 1) / 2 + 1          # positions attended, averaged over the timed tokens

    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src_t = torch.ones(n, device="cuda")
        dst_t = torch.empty(n, device="cuda")
        for _ in range(3):
            dst_t.copy_(src_t)
        torch.cuda.synchronize()
        del src_t, dst_t
        progress(f"copied {args.calibrate_copy_mib} MiB three times")

    # headline: 10% of neurons, look-ahead schedule
    head_cfg = ahead_cfg(k_of[0.10])
    ms_tok, rows = run.run(head_cfg, W, K)
    hb, tok_bytes = step_bytes(dv, head_cfg, L, n_att, rows)
    progress(f"headline: {ms_tok:.3f} ms per token")

    # dense path of the same library: every head and neuron, every fc2 row
    dense_ms, dense_bytes = float("nan"), float("nan")
    if args.dense:
        dense_ms, _ = run.run(dense_cfg, W, K)
        progress(f"dense path: {dense_ms:.3f} ms per token")
    _, dense_bytes = step_bytes(dv, dense_cfg, L, n_att, dims.N)

    sweep, seq_ms = [], None
    if args.sweep:
        for keep in sweep_keep:
            if keep == 0.10:
                ms, r = ms_tok, rows
            else:
                ms, r = run.run(ahead_cfg(k_of[keep]), W, K)
            progress(f"keep {keep:.2f}: {ms:.3f} ms per token")
            _, b = step_bytes(dv, ahead_cfg(k_of[keep]), L, n_att, r)
            sweep.append({"keep_neurons": keep, "k_neurons": k_of[keep], "ms_per_token": round(ms, 4),
                          "tokens_per_s": round(1000.0 / ms, 2),
                          "bytes_per_token": int(b), "fc2_rows_per_layer": round(r, 1),
                          "effective_hbm_GBps": round(b / (ms * 1e-3) / 1e9, 1),
                          "pct_of_peak_hbm": round(100 * b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 1),
                          "speedup_vs_dense": round(dense_ms / ms, 3),
                          "byte_bound_speedup": round(dense_bytes / b, 3),
                          "speedup_over_bound": round((dense_ms / ms) / (dense_bytes / b), 3)})
        seq_ms, _ = run.run(seq_cfg, W, K)
        progress(f"sequential schedule: {seq_ms:.3f} ms per token")

    # the dominant kernel, timed on its own launches inside the headline step.
    # Riders: the next layer's predictor layer one (both predictors) rides in
    # Q/K/V and layer two in the attention launch, in every layer but the
    # last (so (L - 1) / L of them per launch on average).
    ride = (L - 1) / L
    p1_bytes = ride * 2 * (dims.r_attn + dims.r_mlp) * dims.d
    p2_bytes = ride * 2 * (dims.r_attn * dims.h + dims.r_mlp * dims.N)
    kinds = {"k_qkv (Q/K/V + KV append + hole fill, LN1 and next-layer predictor rows folded in)":
             (dv.DV_KERNEL_QKV, hb.qkv + 4 * dims.d + 2 * 2 * head_k * dims.d_h + p1_bytes),
             "k_rowdot_ln (sparse fc1, LN2 folded in)": (dv.DV_KERNEL_FC1, hb.fc1 + 4 * dims.d),
             "k_axpy<ATTN> (W^O gather-AXPY, split-K merge)": (dv.DV_KERNEL_OUT, hb.out_proj),
             "k_axpy (fc2 gather-AXPY)": (dv.DV_KERNEL_FC2, hb.fc2),
             "k_attn_split (split-K attention, next-layer predictor layer two)": (dv.DV_KERNEL_ATTN,
                                                                                  hb.kv_read + p2_bytes)}
    kernels = {}
    for name, (kind, nbytes) in kinds.items():
        d_ms = run.time_kernel(head_cfg, kind, tokens=2, warm=W)   # from the state the timed tokens start in
        progress(f"timed the launches of {name.split(' ')[0]}")
        avg = float(np.mean(d_ms)) if d_ms else float("nan")
        kernels[name] = {"avg_launch_ms": round(avg, 5), "launches": len(d_ms), "bytes_per_launch": int(nbytes),
                         "GBps": round(nbytes / (avg * 1e-3) / 1e9, 1),
                         "frac": round(nbytes / (avg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
    dom = max(kernels, key=lambda k: kernels[k]["avg_launch_ms"] * kernels[k]["launches"])
    dk = kernels[dom]
    digest = kernel_source_digest()
    traffic = read_traffic("traffic_qkv_opt66b_stack.txt", digest)

    result = {
        "metric": "decode tokens/s + effective HBM GB/s (% of peak) vs keep ratio, 1 GPU",
        "value": round(1000.0 / ms_tok, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_tok, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 weights, f32 accumulate",
        "data": "synthetic (seeded N(0,0.02^2) weights generated on the device, N(0,1) inputs and KV cache)",
        "config": {
            "workload": f"opt66b-stack decode: {L} layers, d=9216, 72 heads x 128, d_ffn=36864 ReLU, fp16, batch 1, "
                        "1024 cached tokens per layer, keep 10% neurons (3686) and 50% heads (36), rank-128 "
                        "predictors one layer ahead (DejaVu 4.3) inside the layers' launches, hole fill, one HIP "
                        "graph per token",
            "global_batch": 1, "layers": L, "seq_len": wl.n_ctx, "keep_neurons": 0.10, "keep_heads": 0.50,
            "decode_tokens": DECODE_TOKENS,
        },
        "effective_hbm_GBps": round(tok_bytes / (ms_tok * 1e-3) / 1e9, 1),
        "pct_of_peak_hbm": round(100 * tok_bytes / (ms_tok * 1e-3) / 1e9 / PEAK_HBM_GBPS, 1),
        "bytes_per_token": int(tok_bytes),
        "fc2_rows_per_layer": round(rows, 1),
        "dense_ms_per_token": round(dense_ms, 4),
        "dense_bytes_per_token": int(dense_bytes),
        "dense_effective_hbm_GBps": round(dense_bytes / (dense_ms * 1e-3) / 1e9, 1),
        "speedup_vs_dense": round(dense_ms / ms_tok, 3),
        "byte_bound_speedup": round(dense_bytes / tok_bytes, 3),
        "sequential_ms_per_token": None if seq_ms is None else round(seq_ms, 4),
        "keep_sweep": sweep,
        "kernels": kernels,
        "roofline": {
            "kernel": dom, "bound": "hbm", "achieved": dk["GBps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": dk["frac"], "traffic": traffic, "bytes_per_launch": dk["bytes_per_launch"],
            "avg_launch_ms": dk["avg_launch_ms"],
        },
        "generate_s": round(gen_s, 2),
        "resident_weight_GB": round(resident / 1e9, 2),
    }
    Xh = X[:16].cpu()
    del run, stack, ws, head_sets, neuron_sets, X
    torch.cuda.empty_cache()
    if args.longctx:
        result["longctx_composition"] = bench_longctx(torch, dv, synth, configs, args)
    if args.batched:
        result["batched_union"] = bench_batched(torch, dv, synth, configs, args)
    if args.w4:
        result["w4_sparse_mlp"] = bench_w4(torch, dv, synth, configs, args)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(dims, wl, L, Xh, head_cfg, args.cpu_seconds)
    print(json.dumps(result))


def time_stack(torch, dv, stack, X, ws, cfg, warm, timed, head_sets=None, neuron_sets=None, neuron_counts=None):
    """ms per step over `timed` graph-replayed steps after `warm`, from the
    stack's seeded state; fc2 rows per layer per step; and, for a
    threshold-sparse stack, the channels kept per layer per step by each of
    its four projection inputs."""
    B, d = stack.B, stack.dims.d
    x_cur = torch.empty(B, d, device="cuda")
    x_out = torch.empty(B, d, device="cuda")
    fc2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    stack.reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dv.dv_decode_stack(stack.layers_array(), cfg, x_cur, x_out, ws, head_sets=head_sets, neuron_sets=neuron_sets,
                           neuron_counts=neuron_counts, fc2_rows=fc2)
    for t in range(warm):
        x_cur.copy_(X[t])
        g.replay()
    torch.cuda.synchronize()
    fc2.zero_()
    if stack.teal_rows is not None:
        stack.teal_rows.zero_()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(warm, warm + timed):
        x_cur.copy_(X[t])
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    kept = None
    if stack.teal_rows is not None:
        kept = [float(v) / (timed * stack.L) for v in stack.teal_rows.tolist()]
    return e0.elapsed_time(e1) / timed, int(fc2.item()) / (timed * stack.L), kept


def attn_paths(torch, dv, stack, n, b, scale, reps=10):
    """ByteCross §4.4 and App. D: one layer's attention (layer 0, 32 heads,
    batch 1) at n cached positions, dense and through the KV window (4 sinks
    plus the b - 4 most recent positions), on three attention paths:
      splitk  the library's split-K kernel (splits chosen by the library);
      fused   the same kernel with one 256-thread workgroup per head walking
              all of that head's positions (num_splits = 4: a wave per quarter);
      masked  PyTorch eager attention as transformer code writes it: the
              score vector materialised by a batched product, an additive
              mask, an fp32 softmax and a second product; the window reads a
              compacted copy of its positions, built before timing.
    The masked path is PyTorch's, not the library's: it is the baseline whose
    speedups ByteCross shows to be inflated, timed here for that contrast only."""
    dims = stack.dims
    h, dh = dims.h, dims.d_h
    K, V = stack.K[0], stack.V[0]
    q = torch.empty(1, h, dh, device="cuda")
    dv.dv_fill_normal(q, SEED + 9, 0)
    heads = torch.arange(h, dtype=torch.int32, device="cuda")
    o = torch.empty(1, h, dh, device="cuda")
    win = (4, b - 4)
    views = {"dense": dv.kv_view(K, V, n), "window": dv.kv_view(K, V, n, win_sink=win[0], win_len=win[1])}
    npos = {"dense": n, "window": b}
    ws = dv.workspace(dv.dv_splitk_workspace_bytes(1, h, dh, n, 0) + dv.dv_splitk_workspace_bytes(1, h, dh, n, 4))
    q16 = q.half().unsqueeze(-1)                                   # [1][h][dh][1]
    Kw = torch.cat([K[:, :, :win[0]], K[:, :, n - win[1]:n]], dim=2).contiguous()
    Vw = torch.cat([V[:, :, :win[0]], V[:, :, n - win[1]:n]], dim=2).contiguous()
    kv_of = {"dense": (K[:, :, :n], V[:, :, :n]), "window": (Kw, Vw)}
    masks = {m: torch.zeros(1, 1, npos[m], device="cuda") for m in npos}

    def masked(m):
        Kn, Vn = kv_of[m]
        s = torch.matmul(Kn, q16).squeeze(-1).float() * scale + masks[m]
        p = torch.softmax(s, dim=-1).half().unsqueeze(-2)
        return torch.matmul(p, Vn).squeeze(-2)

    def run(path, m):
        if path == "masked":
            return masked(m)
        dv.dv_splitk_attn(q, heads, h, views[m], scale, o, ws, num_splits=0 if path == "splitk" else 4)
        return o

    out = {}
    for m in ("dense", "window"):
        ref_o = run("splitk", m).clone()
        for path in ("splitk", "fused", "masked"):
            got = run(path, m).float()
            err = float((got - ref_o).abs().max())
            assert err < 2e-2, f"attention path {path}/{m} disagrees with split-K by {err}"
            run(path, m)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                run(path, m)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            by = 2.0 * h * npos[m] * dh * 2                         # K and V rows read once
            out[(path, m)] = ms
            out.setdefault(path, {})[m] = {"ms": round(ms, 4), "GBps": round(by / (ms * 1e-3) / 1e9, 1),
                                           "frac_peak": round(by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 3),
                                           "max_abs_vs_splitk": round(err, 6)}
    for path in ("splitk", "fused", "masked"):
        out[path]["window_speedup"] = round(out[(path, "dense")] / out[(path, "window")], 3)
    del ws, Kw, Vw
    return out


def bench_longctx(torch, dv, synth, configs, args):
    """ByteCross's composition at long context (§3.3, §4.1-4.4): a 32-layer
    stack (d = 4096, 32 heads, d_ffn = 16384) at 2K / 8K / 16K / 32K / 128K
    cached tokens, every mode through the same kernels and the same split-K
    attention:
      dense     every head and neuron;
      proj      DejaVu's MLP sparsity: 10% of neurons, predicted one layer ahead;
      teal      ByteCross's projection branch: threshold sparsity on the input
                of every projection at 50% keep (thresholds calibrated per
                context on 8 seeded tokens, as the pages' TEAL thresholds are
                calibrated once per model);
      kv        10% of cached positions per head chosen by the
                attention-scored selection, plus the decoded tokens;
      window    the KV window: 4 sinks plus the most recent positions, the
                same 10% budget;
      composed  proj + kv;   teal_kv  teal + kv (ByteCross's composition).
    The selection's scoring pass runs once per context after the seeded
    prompt and is timed on its own, outside tokens/s.

    §4.3's cost-aware crossing: a second sweep at 4K / 12K / 24K / 64K gives
    each branch's cost beyond its byte-scaled dense time; with the dense time
    of the first sweep interpolated log-log and the costs linearly, the branch
    latencies are predicted and their crossing with the KV branch set beside
    the measured one and the crossing of the bytes alone (for proj and teal).
    §4.4: at every context of the first sweep, one layer's attention on three
    paths (attn_paths)."""
    from contextual_sparsity_decoding_amd.stack import Stack
    wl = configs.LONGCTX_STACK
    dims, L = wl.dims, wl.layers
    W, K = 2, max(1, args.extra_steps)
    T = W + K
    scale = 1 / math.sqrt(dims.d_h)
    kM = wl.k_neurons
    teal_keep = 0.5
    stack = Stack(dims, L, 16, 32, SEED + 5, hole_fill=False, teal=True)
    X = torch.empty(T, 1, dims.d, device="cuda")
    dv.dv_fill_normal(X, SEED + 5, synth.stream_id(0, "x"))
    Xcal = torch.empty(8, 1, dims.d, device="cuda")
    dv.dv_fill_normal(Xcal, SEED + 5, synth.stream_id(0, "x_cal"))
    base = dv.DV_DENSE_ATTN | dv.DV_ADVANCE_POS
    ahead = dv.DV_SKIP_NONPOS_FC2 | dv.DV_LOOKAHEAD       # neuron sets predicted one layer ahead (DejaVu 4.3)
    teal = dv.DV_DENSE_MLP | dv.DV_TEAL
    modes = {"dense": (base | dv.DV_DENSE_MLP, dims.N),
             "proj": (base | ahead, kM),
             "teal": (base | teal, dims.N),
             "kv": (base | dv.DV_DENSE_MLP | dv.DV_KV_SELECT, dims.N),
             "window": (base | dv.DV_DENSE_MLP | dv.DV_KV_WINDOW, dims.N),
             "composed": (base | ahead | dv.DV_KV_SELECT, kM),
             "teal_kv": (base | teal | dv.DV_KV_SELECT, dims.N)}
    nsets = torch.zeros(L, kM, dtype=torch.int32, device="cuda")

    def mode_cfg(name, b):
        flags, k = modes[name]
        cfg = stack.cfg(dims.h, k, flags, scale)
        if flags & dv.DV_KV_WINDOW:
            cfg.win_sink, cfg.win_len = 4, b - 4
        return cfg

    def positions(name, n, b):
        """Mean positions a head reads per timed token."""
        flags = modes[name][0]
        tail = W + (K - 1) / 2 + 1                          # decoded tokens: always read by the selection
        if flags & dv.DV_KV_SELECT:
            return b + tail
        if flags & dv.DV_KV_WINDOW:
            return float(b)
        return n + tail

    def step_bytes_of(name, n, b, rows, kept=None):
        cfg = mode_cfg(name, b)
        if modes[name][0] & dv.DV_TEAL:
            return L * dv.dv_bytes_read_teal(cfg, positions(name, n, b), kept).total
        dense_m = bool(modes[name][0] & dv.DV_DENSE_MLP)
        return L * dv.dv_bytes_read(cfg, positions(name, n, b), dims.N if dense_m else rows, 0.0).total

    def sweep(ctxs, names, paths):
        pts = []
        for n in ctxs:
            progress(f"long context: {n} tokens, modes {', '.join(names)}")
            b = int(math.floor(wl.kv_keep * n))
            max_len = n + T + 8
            stack.set_context(n, max_len)
            torch.cuda.synchronize()
            row = {"n_ctx": n, "kv_budget": b}
            if any(modes[m][0] & dv.DV_KV_SELECT for m in names):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                stack.select_kv(b)
                e1.record()
                torch.cuda.synchronize()
                row["scoring_ms_all_layers"] = round(e0.elapsed_time(e1), 3)
            ws = dv.workspace(max(dv.dv_stack_workspace_bytes(mode_cfg(m, b), max_len) for m in names))
            if any(modes[m][0] & dv.DV_TEAL for m in names):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                stack.calibrate_teal(teal_keep, Xcal, ws, mode_cfg("teal", b))
                e1.record()
                torch.cuda.synchronize()
                row["teal_calibration_ms"] = round(e0.elapsed_time(e1), 3)
            res = {}
            for name in names:
                cfg = mode_cfg(name, b)
                ms, rows, kept = time_stack(torch, dv, stack, X, ws, cfg, W, K,
                                            neuron_sets=nsets if modes[name][0] & dv.DV_LOOKAHEAD else None)
                by = step_bytes_of(name, n, b, rows, kept)
                res[name] = (ms, by)
                row[name] = {"ms_per_token": round(ms, 4), "tokens_per_s": round(1000 / ms, 2),
                             "bytes_per_token": int(by), "effective_hbm_GBps": round(by / (ms * 1e-3) / 1e9, 1)}
                if modes[name][0] & dv.DV_TEAL:
                    widths = (dims.d, dims.h * dims.d_h, dims.d, dims.N)
                    row[name]["kept_fraction"] = [round(k / w_, 4) for k, w_ in zip(kept, widths)]
                    row[name]["kept_channels"] = [round(k, 1) for k in kept]
                elif name != "dense":
                    row[name]["fc2_rows_per_layer"] = round(rows, 1)
            for name in names:
                if name != "dense":
                    row[name]["speedup"] = round(res["dense"][0] / res[name][0], 3)
                    row[name]["byte_bound_speedup"] = round(res["dense"][1] / res[name][1], 3)
                    # ByteCross §4.3: the branch's cost beyond its byte-scaled dense time
                    row[name]["cost_ms"] = round(res[name][0] - res["dense"][0] * res[name][1] / res["dense"][1], 4)
            if paths:
                ap = attn_paths(torch, dv, stack, n, b, scale)
                # the step with its split-K attention time replaced by each path's (derived, not timed)
                derived = {}
                for path in ("splitk", "fused", "masked"):
                    st = {m: res[m][0] + L * (ap[path][m]["ms"] - ap["splitk"][m]["ms"]) for m in ("dense", "window")}
                    derived[path] = round(st["dense"] / st["window"], 3)
                row["attention_paths_one_layer"] = {k: v for k, v in ap.items() if isinstance(k, str)}
                row["window_step_speedup_by_attention_path_derived"] = derived
                row["window_byte_bound_speedup"] = row["window"]["byte_bound_speedup"]
            pts.append(row)
            del ws
        return pts

    out = sweep(wl.ctx_sweep, list(modes), True)
    cost_pts = sweep((4096, 12288, 24576, 65536), ["dense", "proj", "teal", "kv", "window"], False)

    def cross_of(pts, key, pb):
        """log-linear crossing of branch pb and kv in `key` (speedup), or None."""
        vals = [(r["n_ctx"], r[pb][key] - r["kv"][key]) for r in pts]
        for (n0, a0), (n1, a1) in zip(vals, vals[1:]):
            if a0 >= 0 > a1 or a0 > 0 >= a1:
                f = a0 / (a0 - a1)
                return round(math.exp(math.log(n0) + f * (math.log(n1) - math.log(n0))))
        return None

    at32 = next(r for r in out if r["n_ctx"] == 32768)
    rows_p = at32["proj"]["fc2_rows_per_layer"]
    kept_t = at32["teal"]["kept_channels"]

    def bytes_of(m, n):
        b = int(math.floor(wl.kv_keep * n))
        return step_bytes_of(m, n, b, rows_p, kept_t)

    def bytes_cross(pb):
        """The context where branch pb and the KV branch read the same bytes
        (fc2 survivors and kept channels as measured at 32K)."""
        lo, hi = 1024.0, 1048576.0
        gap = lambda n: bytes_of(pb, n) - bytes_of("kv", n)
        if not gap(lo) < 0 < gap(hi):
            return None
        for _ in range(60):
            mid = math.sqrt(lo * hi)
            lo, hi = (mid, hi) if gap(mid) < 0 else (lo, mid)
        return round(lo)

    # cost-aware prediction: dense time log-log from the first sweep, costs
    # linear in n from the second, byte ratios from the byte account
    dn = [(math.log(r["n_ctx"]), math.log(r["dense"]["ms_per_token"])) for r in out]

    def interp(xy, x):
        xs = [p[0] for p in xy]
        i = max(0, min(len(xy) - 2, sum(1 for v in xs if v <= x) - 1))
        (x0, y0), (x1, y1) = xy[i], xy[i + 1]
        return y0 + (y1 - y0) * (x - x0) / (x1 - x0)

    costs = {m: [(r["n_ctx"], r[m]["cost_ms"]) for r in cost_pts] for m in ("proj", "teal", "kv", "window")}

    def predict(m, n):
        td = math.exp(interp(dn, math.log(n)))
        return td * bytes_of(m, n) / bytes_of("dense", n) + interp(costs[m], n)

    def pred_cross(pb):
        grid = [2048 * 2 ** (i / 64) for i in range(64 * 6 + 1)]
        for n0, n1 in zip(grid, grid[1:]):
            a0, a1 = predict(pb, n0) - predict("kv", n0), predict(pb, n1) - predict("kv", n1)
            if a0 <= 0 < a1 or a0 < 0 <= a1:
                return round(n0 + (n1 - n0) * (-a0) / (a1 - a0))
        return None

    crossings = {pb: {"measured_n": cross_of(out, "speedup", pb), "cost_aware_predicted_n": pred_cross(pb),
                      "bytes_n": bytes_cross(pb)} for pb in ("proj", "teal")}
    pred_at = [{"n_ctx": r["n_ctx"], **{m: {"predicted_ms": round(predict(m, r["n_ctx"]), 4),
                                             "measured_ms": r[m]["ms_per_token"]}
                                        for m in ("proj", "teal", "kv", "window")}} for r in out]
    del stack, X, Xcal, nsets
    torch.cuda.empty_cache()
    return {"workload": "longctx-32L-d4096-h32-ffn16384-fp16: 32 layers, batch 1, heads dense; projection branch "
                        "10% of MLP neurons (DejaVu) or threshold sparsity at 50% keep on every projection input "
                        "(ByteCross/TEAL); KV branch 10% of positions per head (attention-scored, 4 sinks + "
                        "64-token window forced) or the window of 4 sinks + the most recent positions",
            "points": out, "cost_sweep": cost_pts, "crossings_with_kv": crossings,
            "crossover_measured_n": crossings["proj"]["measured_n"], "crossover_bytes_n": crossings["proj"]["bytes_n"],
            "crossover_cost_aware_predicted_n": crossings["proj"]["cost_aware_predicted_n"],
            "cost_model_check": pred_at, "warmup": W, "steps": K}


def bench_batched(torch, dv, synth, configs, args):
    """DejaVu §5.2 / App. C.1: 48 OPT-175B-shaped layers (one GPU's share of
    the stack; d = 12288, 96 heads dense, d_ffn = 49152) decoding batches of
    1-16 independent sequences with 512 cached tokens each; each layer's MLP
    reads the union of the sequences' top-10% neuron sets.  tokens/s =
    B x steps/s; |U|/N is the union's share of the neurons."""
    from contextual_sparsity_decoding_amd.stack import Stack
    wl = configs.OPT175B_SHARE
    dims, L = wl.dims, wl.layers
    W, K = 2, max(1, args.extra_steps)
    T = W + K
    scale = 1 / math.sqrt(dims.d_h)
    kM = wl.k_neurons
    out = []
    stack = None
    sizes = [int(b) for b in args.batch_sizes.split(",") if b] if args.batch_sizes else list(wl.batch)
    for B in sizes:
        if B not in wl.batch:
            raise SystemExit(f"--batch-sizes: {B} is not one of {list(wl.batch)}")
        progress(f"batched stack: B = {B}")
        if stack is None:
            stack = Stack(dims, L, wl.n_ctx, wl.n_ctx + T + 8, SEED + 7, batch=max(wl.batch), hole_fill=False)
        # one stack holds the largest batch's caches; a smaller batch uses the first B of them
        sub = stack.batch_view(B)
        X = torch.empty(T, B, dims.d, device="cuda")
        dv.dv_fill_normal(X, SEED + 7, synth.stream_id(B, "x"))
        flags = dv.DV_DENSE_ATTN | dv.DV_SKIP_NONPOS_FC2 | dv.DV_ADVANCE_POS
        cfg = sub.cfg(dims.h, kM, flags, scale)
        dcfg = sub.cfg(dims.h, dims.N, dv.DV_DENSE_ATTN | dv.DV_DENSE_MLP | dv.DV_ADVANCE_POS, scale)
        ws = dv.workspace(max(dv.dv_stack_workspace_bytes(c, sub.max_len) for c in (cfg, dcfg)))
        nmax = min(dims.N, B * kM)
        nsets = torch.zeros(L, nmax, dtype=torch.int32, device="cuda")
        counts = torch.zeros(L, dtype=torch.int32, device="cuda")
        ms, rows, _ = time_stack(torch, dv, sub, X, ws, cfg, W, K, neuron_sets=nsets, neuron_counts=counts)
        u = counts.float().mean().item()
        dms = time_stack(torch, dv, sub, X, ws, dcfg, W, K)[0] if args.dense else None
        n_att = wl.n_ctx + W + (K - 1) / 2 + 1
        ucfg = sub.cfg(dims.h, int(round(u)), flags, scale)
        by = L * dv.dv_bytes_read(ucfg, n_att, rows, 0.0).total
        dby = L * dv.dv_bytes_read(dcfg, n_att, dims.N, 0.0).total
        out.append({"batch": B, "ms_per_step": round(ms, 4), "tokens_per_s": round(B * 1000 / ms, 2),
                    "union_neurons": round(u, 1), "union_frac": round(u / dims.N, 4),
                    "fc2_rows_per_layer": round(rows, 1), "bytes_per_step": int(by),
                    "effective_hbm_GBps": round(by / (ms * 1e-3) / 1e9, 1),
                    "dense_ms_per_step": round(dms, 4) if dms else None,
                    "speedup_vs_dense": round(dms / ms, 3) if dms else None,
                    "byte_bound_speedup": round(dby / by, 3)})
        del ws, X, nsets, counts
    del stack, sub
    torch.cuda.empty_cache()
    return {"workload": "opt175b-48L-d12288-h96-ffn49152-fp16: 48 layers (one GPU's share), heads dense, 512 cached "
                        "tokens per sequence, neuron keep 10% (4915) per sequence, union per layer",
            "points": out, "warmup": W, "steps": K}


def bench_w4(torch, dv, synth, configs, args):
    """DejaVu §5 (Compatibility with Quantization): the sparse MLP block at
    the OPT-66B width (d = 9216, d_ffn = 36864, batch 1, fc2 rows of zero
    activations skipped) at 10% and 100% of neurons, with fp16 weights and
    with the library's 4-bit weights (dv_quantize_w4), each over 8 layers'
    weights in turn (so that no call finds its rows in the 256 MB
    last-level cache), one HIP graph of the 8 calls replayed."""
    wl = configs.OPT66B_STACK
    d, N = wl.dims.d, wl.dims.N
    L, reps = 8, max(2, args.extra_steps)
    g = torch.Generator(device="cpu").manual_seed(SEED)
    y = torch.empty(L, 1, d, device="cuda")
    dv.dv_fill_normal(y, SEED + 11, synth.stream_id(0, "x"))
    layers = []
    for l in range(L):
        w = {}
        for name, shp in (("w1_t", (N, d)), ("b1", (N,)), ("w2_t", (N, d)), ("b2", (d,))):
            t = torch.empty(shp, dtype=torch.float16, device="cuda")
            dv.dv_fill_normal(t, SEED + 11, synth.stream_id(l, name), std=synth.WEIGHT_STD)
            w[name] = t
        for name in ("w1_t", "w2_t"):
            q = torch.empty(N, d // 2, dtype=torch.uint8, device="cuda")
            sc = torch.empty(N, d // 128, dtype=torch.float16, device="cuda")
            dv.dv_quantize_w4(w[name], q, sc)
            w[name + "_q"], w[name + "_s"] = q, sc
        layers.append(w)
    out = torch.empty(1, d, device="cuda")
    rows = torch.zeros(1, dtype=torch.int32, device="cuda")
    result = {"workload": "sparse MLP block, d=9216, d_ffn=36864, batch 1, fc2 rows of zero activations skipped; "
                          "fp16 weights vs 4-bit group-128 weights with fp16 scales; 8 layers' weights in turn"}
    for keep in (0.10, 1.00):
        k = int(math.floor(keep * N))
        idx = [torch.sort(torch.randperm(N, generator=g)[:k]).values.to(torch.int32).cuda() for _ in range(L)]
        ws16 = dv.workspace(dv.dv_sparse_mlp_workspace_bytes(1, d, k, dv.DV_F16))
        ws4 = dv.workspace(dv.lib.dv_sparse_mlp_w4_workspace_bytes(d, k))

        def call(fmt, l):
            w = layers[l]
            if fmt == "fp16":
                dv.dv_sparse_mlp(y[l], w["w1_t"], w["b1"], w["w2_t"], w["b2"], idx[l], k, out, ws16, residual=y[l],
                                 fc2_rows=rows, flags=dv.DV_SKIP_NONPOS_FC2)
            else:
                dv.dv_sparse_mlp_w4(y[l], N, w["w1_t_q"], w["w1_t_s"], w["b1"], w["w2_t_q"], w["w2_t_s"], w["b2"],
                                    idx[l], out, ws4, n_idx_max=k, residual=y[l], fc2_rows=rows,
                                    flags=dv.DV_SKIP_NONPOS_FC2)

        res = {"k_neurons": k}
        for fmt in ("fp16", "w4"):
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for l in range(L):
                    call(fmt, l)
            gr.replay()
            torch.cuda.synchronize()
            rows.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                gr.replay()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / (reps * L)
            live = int(rows.item()) / (reps * L)
            row_b = d * 2 if fmt == "fp16" else d // 2 + (d // 128) * 2
            by = k * row_b + live * row_b + (k + d) * 2 + 3 * d * 4 + 8 * k
            res[fmt] = {"ms_per_call": round(ms, 5), "fc2_rows": round(live, 1), "bytes_per_call": int(by),
                        "GBps": round(by / (ms * 1e-3) / 1e9, 1),
                        "frac_of_8TBps": round(by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 3)}
            del gr
            progress(f"4-bit MLP, keep {keep:.2f}: {fmt} {ms * 1e3:.1f} us per call")
        res["speedup_w4_over_fp16"] = round(res["fp16"]["ms_per_call"] / res["w4"]["ms_per_call"], 3)
        res["byte_ratio"] = round(res["fp16"]["bytes_per_call"] / res["w4"]["bytes_per_call"], 3)
        result[f"keep_{keep:.2f}"] = res
        del ws16, ws4, idx
    del layers, y
    torch.cuda.empty_cache()
    return result


def cpu_baseline(dims, wl, L, X, cfg, budget_s):
    """The oracle, as it stands, on a sample of the same workload: decode
    steps of layer 0 of the stack (its weights regenerated on the host from
    the same seeded streams) in the look-ahead form, run once with one BLAS
    thread and once with all of them; tokens/s of the whole stack is the
    per-layer rate divided by the layer count (extrapolated: the stack does
    not fit in host memory)."""
    from contextual_sparsity_decoding_amd import synth
    from oracle import ref
    from threadpoolctl import threadpool_info, threadpool_limits

    n_cpu, model = cpu_info()
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    W = synth.stack_layer_weights(dims, SEED, 0)
    Wn = synth.stack_layer_weights(dims, SEED, 1, names=["pa1_t", "pa2_t", "pm1_t", "pm2_t"])
    max_len = wl.n_ctx + 16
    K = synth.philox_tensor((1, dims.h, max_len, dims.d_h), SEED, 0, "K", 1.0, np.float16)
    V = synth.philox_tensor((1, dims.h, max_len, dims.d_h), SEED, 0, "V", 1.0, np.float16)
    Xh = X.numpy()
    g = np.random.default_rng(SEED)

    def timing(threads):
        kv = ref.KVState(K.copy(), V.copy(), np.zeros((1, max_len, dims.d)), np.full((1, dims.h), wl.n_ctx - 1))
        heads = np.sort(g.choice(dims.h, cfg.k_heads, replace=False))
        neurons = np.sort(g.choice(dims.N, cfg.k_neurons, replace=False))
        steps, t0 = 0, time.perf_counter()
        with threadpool_limits(threads):
            while steps == 0 or (time.perf_counter() - t0 < budget_s and steps < len(Xh)):
                _, rec = ref.decode_layer_lookahead(Xh[steps], W, Wn, kv, wl.n_ctx + steps, head_idx=heads,
                                                    neuron_idx=neurons, k_heads=cfg.k_heads, k_neurons=cfg.k_neurons,
                                                    scale=cfg.scale, skip_nonpos=True, hole_fill=True)
                heads, neurons = rec["next_head_idx"], rec["next_neuron_idx"]
                steps += 1
        dt = time.perf_counter() - t0
        return steps, dt

    progress("CPU baseline: layer 0 regenerated on the host")
    s1, t1 = timing(1)
    progress(f"CPU baseline: {s1} steps with one thread in {t1:.1f} s")
    sa, ta = timing(blas)
    progress(f"CPU baseline: {sa} steps with {blas} threads in {ta:.1f} s")
    per_layer_all = ta / sa
    return {"value": round(1.0 / (per_layer_all * L), 5), "unit": "tokens/s", "cores": blas, "kind": "oracle",
            "sample": f"{sa} decode steps of layer 0 of the stack (float64 NumPy oracle, look-ahead form, "
                      f"{blas} BLAS threads) in {ta:.1f} s; tokens/s = 1 / ({L} x per-layer time), extrapolated",
            "single_thread_tokens_per_s": round(1.0 / (t1 / s1 * L), 5),
            "single_thread_sample": f"{s1} steps in {t1:.1f} s with 1 thread",
            "host_cpus": n_cpu, "cpu_model": model}


if __name__ == "__main__":
    main()
