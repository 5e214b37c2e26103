"""Benchmark: sparse decode of one OPT-13B-shaped layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one decode token through one layer (d=5120, 40 heads x 128,
d_ffn=20480 ReLU, fp16 weights, fp32 accumulate, 2048 cached tokens), with
10% of neurons and 50% of heads selected by rank-128 predictors, hole fill
on and fc2 rows of non-positive neurons skipped.  The timed schedule is
DejaVu §4.3's parallel form: the step runs Q/K/V + KV append (LN folded in)
-> split-K attention -> W^O -> fc1 (LN folded in) -> fc2 on the sets
predicted during the previous step, while the next step's head and neuron
predictors and selections ride in those launches as extra workgroups (the
predictors' first layers beside Q/K/V, their second layers beside
attention, the neuron top-k split over W^O, its finalize and fc2).  The same
schedule with the predictions on a second stream is timed too.  Four
independent layer copies
are used in turn so that the 256 MB Infinity Cache cannot serve repeated
reads; each copy's position advances by one per step it takes, and step s
predicts for copy (s + 1) mod 4 with that copy's predictors.

Prints one JSON line: decode tokens/s, effective HBM bandwidth on the bytes
the step must read, the dominant kernel's roofline, the two-stream and
sequential schedules and the dense path of the same library, a neuron
keep-ratio sweep, and the
CPU oracle timed on a sample of the same workload.
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=64)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--copies", type=int, default=4)
    p.add_argument("--kernel-launches", type=int, default=64)
    p.add_argument("--dense-steps", type=int, default=16)
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--sweep-steps", type=int, default=32,
                   help="steps per point of the neuron keep-ratio sweep (0 skips the sweep)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="before the Q/K/V launches, copy this many MiB device to device three times "
                        "(a copy of known size for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return p.parse_args()


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "contextual_sparsity_decoding_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_traffic(name: str, digest: str):
    """HBM traffic per launch from a committed PMC summary, if it was taken
    on the current kernel sources."""
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


class Copy:
    """One layer copy's weights and decode state on the device.  The decode
    position lives on the device (pos_dev) so captured steps can be replayed."""

    def __init__(self, dv, torch, dims, n0, max_len, seed):
        from contextual_sparsity_decoding_amd import synth
        self.W = synth.layer_weights(dims, seed, layer=0)
        K, V = synth.kv_cache(dims.h, dims.d_h, n0, max_len, seed)
        self.host_K, self.host_V = K, V
        self.Wd = {k: torch.from_numpy(v).cuda() for k, v in self.W.items()}
        self.K, self.V = torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda()
        self.y_buf = torch.zeros(1, max_len, dims.d, device="cuda")
        self.valid = torch.full((1, dims.h), n0 - 1, dtype=torch.int32, device="cuda")
        self.pos_dev = torch.full((1,), n0, dtype=torch.int32, device="cuda")
        self.wts = dv.layer_weights(self.Wd)
        self.st = dv.LayerState()
        # pos (the host field) is only the bound of the device position
        self.st.kv = dv.kv_state(self.K, self.V, max_len - 1, self.y_buf, self.valid, self.pos_dev)
        self.head_idx = torch.zeros(dims.h, dtype=torch.int32, device="cuda")
        self.st.head_idx_out = self.head_idx.data_ptr()


class Ahead:
    """What the look-ahead schedule (DejaVu §4.3, parallel form) carries from
    step to step: two ping-pong pairs of index buffers (step s reads pair s % 2
    and writes the next step's sets into the other), and for the two-stream
    form the second stream and the fork/join events (without them the
    predictions ride in the layer's own launches)."""

    def __init__(self, torch, dims, two_stream=False):
        self.two_stream = two_stream
        self.aux = torch.cuda.Stream()
        self.evs = [torch.cuda.Event(), torch.cuda.Event()]
        for e in self.evs:
            e.record()
        torch.cuda.synchronize()
        self.hb = [torch.zeros(dims.h, dtype=torch.int32, device="cuda") for _ in range(2)]
        self.nb = [torch.zeros(dims.N, dtype=torch.int32, device="cuda") for _ in range(2)]
        self.dims = dims

    def seed_sets(self, torch, k_heads, k_neurons, seed):
        """Sets for the very first step (every later step uses predicted ones)."""
        g = np.random.default_rng(seed)
        self.hb[0][:k_heads] = torch.from_numpy(np.sort(g.choice(self.dims.h, k_heads, replace=False)).astype(np.int32))
        self.nb[0][:k_neurons] = torch.from_numpy(np.sort(g.choice(self.dims.N, k_neurons, replace=False)).astype(np.int32))


def capture_steps(dv, torch, copies, cfg, X, first, count, out, ws, fc2_rows, ahead=None):
    """A HIP graph of `count` decode steps (step s uses copy s % R and input
    X[first + s]).  With `ahead`, step s runs copy s % R on the sets predicted
    by step s - 1 and predicts copy (s + 1) % R's sets with that copy's
    predictors (on the second stream when ahead.two_stream)."""
    g = torch.cuda.CUDAGraph()
    R = len(copies)
    with torch.cuda.graph(g):
        stream = torch.cuda.current_stream().cuda_stream
        for i in range(count):
            cp = copies[i % R]
            st = cp.st
            if ahead is not None:
                nxt = copies[(i + 1) % R]
                st = dv.LayerState()
                st.kv = cp.st.kv
                p, q = i % 2, (i + 1) % 2
                st.head_idx_in, st.neuron_idx_in = ahead.hb[p].data_ptr(), ahead.nb[p].data_ptr()
                st.next_head_idx, st.next_neuron_idx = ahead.hb[q].data_ptr(), ahead.nb[q].data_ptr()
                st.next_pa1_t, st.next_pa2_t = nxt.Wd["pa1_t"].data_ptr(), nxt.Wd["pa2_t"].data_ptr()
                st.next_pm1_t, st.next_pm2_t = nxt.Wd["pm1_t"].data_ptr(), nxt.Wd["pm2_t"].data_ptr()
                if ahead.two_stream:
                    st.aux_stream = ahead.aux.cuda_stream
                    st.ev_fork, st.ev_join = ahead.evs[0].cuda_event, ahead.evs[1].cuda_event
            st.fc2_rows_out = fc2_rows.data_ptr() if fc2_rows is not None else 0
            rc = dv.lib.dv_decode_layer(dv.C.byref(cp.wts), dv.C.byref(cfg), dv.C.byref(st),
                                        X[first + i].data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel(), stream)
            if rc != 0:
                raise dv.DVError("dv_decode_layer", rc)
    return g


def time_graph(torch, g):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1), time.perf_counter() - t0


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from contextual_sparsity_decoding_amd import account, configs, dv, synth

    w = configs.OPT13B_LAYER
    dims = w.dims
    R = args.copies
    K = args.steps
    warm_reps = max(1, math.ceil(args.warmup / K))
    Kd = args.dense_steps
    sweep_keep = (0.05, 0.10, 0.25, 0.50, 1.00)
    total_steps = (warm_reps + 1) * K + 4 * K + (2 * Kd if Kd > 0 else 0) + 2 * args.sweep_steps * len(sweep_keep)
    max_len = w.n_ctx + math.ceil(total_steps / R) + 8
    torch.cuda.set_device(0)
    copies = [Copy(dv, torch, dims, w.n_ctx, max_len, SEED + c) for c in range(R)]
    X = torch.from_numpy(np.ascontiguousarray(synth.layer_inputs(dims.d, max(K, Kd, args.sweep_steps, 16), 1,
                                                                 SEED))).cuda()
    out = torch.empty(1, dims.d, device="cuda")
    flags = dv.DV_HOLE_FILL | dv.DV_SKIP_NONPOS_FC2 | dv.DV_ADVANCE_POS

    def cfg(flags_, k_neurons=w.k_neurons):
        dense_a = bool(flags_ & dv.DV_DENSE_ATTN)
        dense_m = bool(flags_ & dv.DV_DENSE_MLP)
        return dv.decode_cfg(B=1, d=dims.d, h=dims.h, d_h=dims.d_h, N=dims.N, r_attn=dims.r_attn,
                             r_mlp=dims.r_mlp, k_heads=dims.h if dense_a else w.k_heads,
                             k_neurons=dims.N if dense_m else k_neurons, wdt=dv.DV_F16,
                             pred_act=dv.DV_ACT_RELU, eps=1e-5, scale=1 / math.sqrt(dims.d_h), flags=flags_)

    ahead_flags = flags | dv.DV_LOOKAHEAD
    sparse_cfg = cfg(ahead_flags)
    seq_cfg = cfg(flags)
    dense_cfg = cfg(flags | dv.DV_DENSE_ATTN | dv.DV_DENSE_MLP)
    ws = dv.workspace(max([dv.dv_decode_workspace_bytes(c, max_len) for c in (sparse_cfg, seq_cfg, dense_cfg)] +
                          [dv.dv_decode_workspace_bytes(cfg(ahead_flags, int(math.floor(k * dims.N))), max_len)
                           for k in sweep_keep]))
    fc2_rows = torch.zeros(1, dtype=torch.int32, device="cuda")
    ahead = Ahead(torch, dims)
    ahead.seed_sets(torch, w.k_heads, w.k_neurons, SEED)

    # K sparse steps (look-ahead schedule) captured once; warm-up replays, then one timed replay
    g_sparse = capture_steps(dv, torch, copies, sparse_cfg, X, 0, K, out, ws, fc2_rows, ahead)
    for _ in range(warm_reps):
        g_sparse.replay()
    torch.cuda.synchronize()
    fc2_rows.zero_()
    ms_total, wall = time_graph(torch, g_sparse)
    ms_step = ms_total / K
    rows_per_step = int(fc2_rows.item()) / K
    del g_sparse

    # the same schedule with the predictions on a second stream (a fork and a join per step)
    ahead2 = Ahead(torch, dims, two_stream=True)
    ahead2.seed_sets(torch, w.k_heads, w.k_neurons, SEED)
    g_two = capture_steps(dv, torch, copies, sparse_cfg, X, 0, K, out, ws, None, ahead2)
    g_two.replay()
    two_ms = time_graph(torch, g_two)[0] / K
    del g_two

    # the sequential schedule (each block's predictor before the block) through the same kernels
    g_seq = capture_steps(dv, torch, copies, seq_cfg, X, 0, K, out, ws, None)
    g_seq.replay()
    seq_ms = time_graph(torch, g_seq)[0] / K
    del g_seq

    # dense path through the same kernels
    dense_ms = None
    if Kd > 0:
        g_dense = capture_steps(dv, torch, copies, dense_cfg, X, 0, Kd, out, ws, None)
        g_dense.replay()
        dense_ms = time_graph(torch, g_dense)[0] / Kd

    # neuron keep-ratio sweep at 50% heads: same kernels, same copies, one graph per point
    sweep = []
    if args.sweep_steps > 0:
        Ks = args.sweep_steps
        for keep in sweep_keep:
            kn = int(math.floor(keep * dims.N))
            ahead.seed_sets(torch, w.k_heads, kn, SEED + 1)
            fc2_rows.zero_()
            g = capture_steps(dv, torch, copies, cfg(ahead_flags, kn), X, 0, Ks, out, ws, fc2_rows, ahead)
            g.replay()
            torch.cuda.synchronize()
            fc2_rows.zero_()
            ms = time_graph(torch, g)[0] / Ks
            rows = int(fc2_rows.item()) / Ks
            b = account.step_bytes(dims, w.k_heads, kn, n_att=w.n_ctx + 1, fc2_rows=rows)
            db_ = account.step_bytes(dims, dims.h, dims.N, n_att=w.n_ctx + 1, fc2_rows=dims.N, head_pred=False,
                                     neuron_pred=False)
            sweep.append({"keep_neurons": keep, "k_neurons": kn, "ms_per_step": round(ms, 5),
                          "tokens_per_s": round(1000.0 / ms, 1),
                          "effective_hbm_GBps": round(b.total / (ms * 1e-3) / 1e9, 1),
                          "speedup_vs_dense": None if dense_ms is None else round(dense_ms / ms, 3),
                          "byte_bound_speedup": round(db_.total / b.total, 3)})
            del g

    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src_t = torch.ones(n, device="cuda")
        dst_t = torch.empty(n, device="cuda")
        for _ in range(3):
            dst_t.copy_(src_t)
        torch.cuda.synchronize()
        del src_t, dst_t

    # dominant kernel: sparse Q/K/V projection with KV append, `kernel_launches` launches captured in one HIP
    # graph (copies in turn, each rewriting its current slot; no missing positions remain, so no hole-fill
    # state is passed and the graph holds the projection kernel only), replayed once untimed, once timed
    qws = dv.workspace(dv.dv_attn_proj_workspace_bytes(0, 1, dims.d, dims.h, dims.d_h, w.k_heads, dv.DV_F16))
    q = torch.empty(1, w.k_heads, dims.d_h, device="cuda")
    yq = torch.from_numpy(np.ascontiguousarray(synth.normal((1, dims.d), SEED, 9, "x"))).cuda()
    last = [int(cp.pos_dev.item()) - 1 for cp in copies]
    kvs = [dv.kv_state(cp.K, cp.V, last[c], None, None) for c, cp in enumerate(copies)]
    nq = max(1, args.kernel_launches)
    g_qkv = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_qkv):
        for i in range(nq):
            c = i % R
            dv.dv_sparse_attn_proj(dv.DV_PROJ_QKV, dims.h, dims.d_h, copies[c].head_idx, w.k_heads, copies[c].Wd["w_qkv_t"],
                                   copies[c].Wd["b_qkv"], yq, q, qws, kv=kvs[c])
    g_qkv.replay()
    qkv_ms = time_graph(torch, g_qkv)[0] / nq

    # byte account
    sb = account.step_bytes(dims, w.k_heads, w.k_neurons, n_att=w.n_ctx + 1, fc2_rows=rows_per_step)
    db = account.step_bytes(dims, dims.h, dims.N, n_att=w.n_ctx + 1, fc2_rows=dims.N, head_pred=False,
                            neuron_pred=False)
    qkv_bytes = account.step_bytes(dims, w.k_heads, 0, 0, 0).qkv
    achieved = qkv_bytes / (qkv_ms * 1e-3) / 1e9
    digest = kernel_source_digest()
    traffic = read_traffic("traffic_qkv_opt13b_layer.txt", digest)

    result = {
        "metric": "decode tokens/s + effective HBM GB/s (% of peak) vs keep ratio, 1 GPU",
        "value": round(1000.0 / ms_step, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warm_reps * K,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 weights, f32 accumulate",
        "data": "synthetic (seeded N(0,0.02^2) weights, N(0,1) inputs and KV cache)",
        "config": {
            "workload": "opt13b-layer decode: d=5120, 40 heads x 128, d_ffn=20480 ReLU, fp16, batch 1, "
                        "2048 cached tokens, keep 10% neurons (2048) and 50% heads (20), rank-128 predictors run "
                        "one layer ahead inside the layer's own launches, 4 rotating layer copies, one HIP graph of "
                        "the timed steps",
            "global_batch": 1, "seq_len": w.n_ctx, "keep_neurons": 0.10, "keep_heads": 0.50,
        },
        "effective_hbm_GBps": round(sb.total / (ms_step * 1e-3) / 1e9, 1),
        "pct_of_peak_hbm": round(100 * sb.total / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBPS, 1),
        "bytes_per_step": int(sb.total),
        "fc2_rows_per_step": round(rows_per_step, 1),
        "dense_ms_per_step": None if dense_ms is None else round(dense_ms, 5),
        "speedup_vs_dense": None if dense_ms is None else round(dense_ms / ms_step, 3),
        "byte_bound_speedup": round(db.total / sb.total, 3),
        "host_wall_ms_per_step": round(1000 * wall / K, 4),
        "sequential_ms_per_step": round(seq_ms, 5),
        "two_stream_ms_per_step": round(two_ms, 5),
        "keep_sweep": sweep,
        "roofline": {
            "kernel": "k_qkv (sparse Q/K/V gather-GEMV + KV append)",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
            "bytes_per_launch": int(qkv_bytes), "avg_launch_ms": round(qkv_ms, 5),
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(copies[0], dims, w, X, args.cpu_seconds)
    print(json.dumps(result))


def cpu_baseline(cp, dims, w, X, budget_s):
    """The oracle, as it stands, on a sample of the same workload: decode
    steps of layer copy 0 from its seeded state, until ~budget_s of CPU time."""
    from oracle import ref
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    Xh = X.cpu().numpy()
    L = cp.host_K.shape[2]
    kv = ref.KVState(cp.host_K.copy(), cp.host_V.copy(), np.zeros((1, L, dims.d)), np.full((1, dims.h), w.n_ctx - 1))
    steps, t0 = 0, time.perf_counter()
    cap = min(len(Xh), L - w.n_ctx)
    while steps == 0 or (time.perf_counter() - t0 < budget_s and steps < cap):
        ref.decode_layer(Xh[steps], cp.W, kv, w.n_ctx + steps, k_heads=w.k_heads, k_neurons=w.k_neurons,
                         scale=1 / math.sqrt(dims.d_h), skip_nonpos=True, hole_fill=True)
        steps += 1
    dt = time.perf_counter() - t0
    return {"value": round(steps / dt, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{steps} decode steps of one OPT-13B-shaped layer (float64 NumPy oracle), {dt:.1f} s"}


if __name__ == "__main__":
    main()
