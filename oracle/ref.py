"""The decode step of contextual sparsity, in float64 NumPy (test infrastructure).

Plain and slow on purpose: every function is the definition on the page it
cites, with no blocking, fusion or reordering.  Weights arrive in the storage
layouts documented in ``contextual_sparsity_decoding_amd.synth`` (the
transposed rows of fc1/fc2 and of the output projection); each function turns
them back into the page's matrices explicitly.  fp16 inputs are exact in
float64.  Values the method stores in fp16 (the KV cache) are rounded to fp16
round-to-nearest-even where they are stored.

Pages (see ``oracle/__init__.py``): DejaVu, Explainer, ByteCross.

Readings taken where the pages are silent (each is listed in the design doc):
  * the predictor's hidden activation is ReLU by default, no biases;
  * selection order is score descending, ties to the lower index, NaN last;
    selected sets are returned ascending;
  * attention scores carry a ``scale`` (1/sqrt(d_h) by default; 1 gives Eq. 2
    exactly);
  * LayerNorm uses the population variance and eps = 1e-5;
  * a head not selected at a step leaves its K/V slot empty; when it is
    selected later, every empty slot since its last selection is recomputed
    from the stored layer input (DejaVu §4.2);
  * for a batch, every sequence computes over the union of the per-sequence
    sets (DejaVu §5.2 and App. C.1), for neurons and heads alike;
  * the KV window is the first n_sink positions plus the last win_len
    positions of the cache, a position in both counted once.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np

F64 = np.float64


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


def relu(z: np.ndarray) -> np.ndarray:
    return np.where(z > 0, z, 0.0)


# ---------------------------------------------------------------- LayerNorm --

def layernorm(x, gamma, beta, eps: float = 1e-5) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) * gamma + beta over the last axis.

    DejaVu App. B: a normalization layer precedes each block F(X) of the
    residual stream X + F(X) (pre-LN OPT).  Population variance.
    """
    x = _f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * _f64(gamma) + _f64(beta)


# ---------------------------------------------------------------- predictor --

def predictor(y, p1_t, p2_t, act: str = "relu") -> np.ndarray:
    """Sparsity predictor SP(y) = act(y P1) P2, one score per neuron or head.

    DejaVu §4.1 ("a small two-layer fully connected network") and §4.2 (the
    head predictor has the same architecture); Explainer §4.1 writes it as
    sigma_pred(y W1_pred) W2_pred.  P1 (d x r) is stored transposed as
    ``p1_t`` [r][d], P2 (r x n_out) as ``p2_t`` [n_out][r].
    """
    P1 = _f64(p1_t).T          # d x r
    P2 = _f64(p2_t).T          # r x n_out
    hidden = _f64(y) @ P1
    if act == "relu":
        hidden = relu(hidden)
    elif act != "none":
        raise ValueError(act)
    return hidden @ P2


# ---------------------------------------------------------------- selection --

def topk_select(scores, k: int) -> np.ndarray:
    """The k entries that come first in the order (score descending, index
    ascending), NaN after every number; returned as ascending indices.

    DejaVu §2.3: the selected set S_M (or S_A) under a budget on its size;
    Explainer §2.3 states the budget |S_M| <= (1 - sparsity) * 4d.  The pages
    do not say how ties at the k-th score are broken: the lower index wins.
    The decision is taken on the values as given (fp32 scores stay fp32).
    """
    s = np.asarray(scores)
    if s.ndim != 1:
        raise ValueError("one row at a time")
    n = s.shape[0]
    if not 0 <= k <= n:
        raise ValueError(f"k={k} outside [0, {n}]")
    nan = np.isnan(s)
    neg = np.where(nan, 0, -s)            # -(+0.0) == -(-0.0): zeros tie
    order = np.lexsort((np.arange(n), neg, nan))   # last key is primary
    return np.sort(order[:k]).astype(np.int64)


def topk_rows(scores, k: int) -> List[np.ndarray]:
    return [topk_select(row, k) for row in np.asarray(scores)]


def union_sorted(sets: Sequence[np.ndarray]) -> np.ndarray:
    """U = union of the per-sequence sets, ascending (DejaVu §5.2, App. C.1:
    "the union operation is essential to realize a fast sparse GEMM")."""
    u = set()
    for s in sets:
        u.update(int(i) for i in s)
    return np.array(sorted(u), dtype=np.int64)


# ---------------------------------------------------------------------- MLP --

def sparse_mlp(y, w1_t, b1, w2_t, b2, idx, residual=None, skip_nonpos: bool = False):
    """MLP_S(y) = sigma(y W1_S) (W2_S)^T + b2 (+ residual), sigma = ReLU.

    DejaVu §2.3 Eq. (1), with OPT's biases b1 (per selected neuron) and b2.
    W1 and W2 are d x N; their columns W1_j, W2_j are the rows ``w1_t[j]``
    and ``w2_t[j]``.  ``y`` is [B][d]; every row uses the same set ``idx``.

    fc2 is the plain ordered sum over j in S of a_j * W2_j.  With
    ``skip_nonpos`` the terms of neurons whose activation is zero for every
    row are left out (DejaVu §2.3: the ReLU output sparsifies the second
    linear layer; Explainer §4.4: load W2 rows only for surviving neurons).

    Returns (out [B][d], a [B][|S|]).
    """
    y = _f64(np.atleast_2d(y))
    idx = np.asarray(idx, dtype=np.int64)
    W1_S = _f64(w1_t[idx]).T                # d x |S|, columns W1_j
    a = relu(y @ W1_S + _f64(b1)[idx])       # B x |S|
    out = np.zeros((y.shape[0], y.shape[1]), F64) + _f64(b2)
    if residual is not None:
        out = out + _f64(np.atleast_2d(residual))
    W2_S = _f64(w2_t[idx])                   # |S| x d, rows W2_j
    for jj in range(len(idx)):
        if skip_nonpos and not np.any(a[:, jj] > 0):
            continue
        out = out + a[:, jj:jj + 1] * W2_S[jj][None, :]
    return out, a


def dense_mlp(y, w1_t, b1, w2_t, b2, residual=None):
    """MLP(y) with every neuron: S = [N]."""
    return sparse_mlp(y, w1_t, b1, w2_t, b2, np.arange(np.asarray(w1_t).shape[0]), residual)


# ---------------------------------------------------------------- attention --

@dataclass
class KVState:
    """Per-layer decode state.

    K, V       fp16 [B][h][max_len][d_h]
    y_buf      float64 [B][max_len][d]: layer inputs kept for recomputing
               missing K/V (DejaVu §4.2), or None
    valid_upto int [B][h]: position of each head's last written K/V, or None
    """
    K: np.ndarray
    V: np.ndarray
    y_buf: Optional[np.ndarray] = None
    valid_upto: Optional[np.ndarray] = None


def head_rows(w_qkv_t, b_qkv, which: int, head: int):
    """The d x d_h matrix W_i^{Q,K,V} (DejaVu §2.3) and its bias, from the
    stored [3][h][d_h][d] block (which = 0 Q, 1 K, 2 V)."""
    return _f64(w_qkv_t[which, head]).T, _f64(b_qkv[which, head])


def qkv_step(y, w_qkv_t, b_qkv, head_idx, kv: KVState, pos: int, hole_fill: bool = True):
    """Selected heads' q, k, v for the token at ``pos``; K/V stored in fp16.

    DejaVu §4.2: for the predicted heads compute keys and values and store
    them in the KV cache; save y for the other heads; when a head with
    missing entries is selected later, recompute them from the stored y.
    Explainer §4.2 spells the same procedure out step by step.

    y [B][d]; returns q [B][n_sel][d_h] (float64).  Mutates ``kv``.
    """
    y = _f64(np.atleast_2d(y))
    B = y.shape[0]
    head_idx = np.asarray(head_idx, dtype=np.int64)
    d_h = w_qkv_t.shape[2]
    q = np.zeros((B, len(head_idx), d_h), F64)
    fill = hole_fill and kv.y_buf is not None and kv.valid_upto is not None
    if kv.y_buf is not None:
        kv.y_buf[:, pos] = y
    for s, i in enumerate(head_idx):
        WQ, bQ = head_rows(w_qkv_t, b_qkv, 0, i)
        WK, bK = head_rows(w_qkv_t, b_qkv, 1, i)
        WV, bV = head_rows(w_qkv_t, b_qkv, 2, i)
        for b in range(B):
            q[b, s] = y[b] @ WQ + bQ
            first = int(kv.valid_upto[b, i]) + 1 if fill else pos
            for p in range(min(first, pos), pos + 1):
                yp = y[b] if p == pos else kv.y_buf[b, p]
                kv.K[b, i, p] = (yp @ WK + bK).astype(np.float16)
                kv.V[b, i, p] = (yp @ WV + bV).astype(np.float16)
            if kv.valid_upto is not None:
                kv.valid_upto[b, i] = pos
    return q


def attend(q, K, V, scale: float) -> np.ndarray:
    """H(y) = D^-1 exp(scale * q K^T) V for one head over the rows given.

    DejaVu §2.3 Eq. (2) with q = y W^Q and K = X W^K, V = X W^V the cached
    projections; ``scale`` = 1 is Eq. (2) as printed.  The maximum is
    subtracted before exp (an identity of the quotient).
    """
    q, K, V = _f64(q), _f64(K), _f64(V)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], F64)
    s = scale * (K @ q)
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


def retained_positions(n_ctx: int, sel: Optional[np.ndarray] = None,
                       sel_end: Optional[int] = None) -> np.ndarray:
    """Positions one head attends to: all of [0, n_ctx), or the retained set
    ``sel`` (ascending, each < sel_end) plus every position in [sel_end, n_ctx)
    (ByteCross §3.2: the cache keeps receiving entries; the new ones are read)."""
    if sel is None:
        return np.arange(n_ctx)
    tail = np.arange(sel_end, n_ctx)
    return np.concatenate([np.asarray(sel, dtype=np.int64), tail])


def window_positions(n_ctx: int, n_sink: int, win_len: int) -> np.ndarray:
    """The KV window (ByteCross §5.1 and App. A): the first ``n_sink``
    positions (the sinks) and the last ``win_len`` positions before n_ctx,
    each once, ascending.  The window moves on as the cache grows."""
    sinks = np.arange(min(n_sink, n_ctx))
    recent = np.arange(max(len(sinks), n_ctx - win_len), n_ctx)
    return np.concatenate([sinks, recent])


def attention(q, kv: KVState, head_idx, n_ctx: int, scale: float,
              sel_idx=None, sel_len=None, sel_end: Optional[int] = None,
              window: Optional[Tuple[int, int]] = None) -> np.ndarray:
    """o [B][n_sel][d_h]: Eq. (2) for every selected head over its positions.

    ``sel_idx`` [B][h][cap] / ``sel_len`` [B][h] give retained positions per
    head for the KV branch (ByteCross §4.1); ``window`` = (n_sink, win_len)
    reads the KV window instead; neither attends to all n_ctx.
    """
    q = _f64(q)
    B, n_sel, d_h = q.shape
    o = np.zeros((B, n_sel, d_h), F64)
    for b in range(B):
        for s, i in enumerate(np.asarray(head_idx, dtype=np.int64)):
            if window is not None:
                P = window_positions(n_ctx, *window)
            elif sel_idx is None:
                P = retained_positions(n_ctx)
            else:
                P = retained_positions(n_ctx, sel_idx[b, i, :int(sel_len[b, i])], sel_end)
            o[b, s] = attend(q[b, s], kv.K[b, i, P], kv.V[b, i, P], scale)
    return o


def out_proj(o, w_o_t, b_o, head_idx, residual=None) -> np.ndarray:
    """MHA_{S_A}(y) = sum_{i in S_A} H_i(y) W_i^O + b_O (+ residual).

    DejaVu §2.3 (sparsified MHA); W_i^O (d_h x d) is rows i*d_h..i*d_h+d_h-1
    of the stored ``w_o_t`` (DejaVu §4.4 stores W^O so that a head's block is
    contiguous).  o [B][n_sel][d_h]; returns [B][d].
    """
    o = _f64(o)
    B, _, d_h = o.shape
    W = _f64(w_o_t)
    out = np.zeros((B, W.shape[1]), F64) + _f64(b_o)
    if residual is not None:
        out = out + _f64(np.atleast_2d(residual))
    for s, i in enumerate(np.asarray(head_idx, dtype=np.int64)):
        out = out + o[:, s, :] @ W[i * d_h:(i + 1) * d_h]
    return out


# ---------------------------------------------------------- split-K algebra --

def splitk_partials(q, K, V, scale: float, bounds: Sequence[int]):
    """Per split c over rows [bounds[c], bounds[c+1]): m_c = max score,
    l_c = sum exp(s - m_c), o_c = sum exp(s - m_c) v.  Empty splits give
    (m, l, o) = (-inf, 0, 0).  (The pages name split-K attention -- ByteCross
    §4.1, App. A -- without its algebra; this is the log-sum-exp identity.)"""
    q, K, V = _f64(q), _f64(K), _f64(V)
    parts = []
    for c in range(len(bounds) - 1):
        lo, hi = bounds[c], bounds[c + 1]
        if hi <= lo:
            parts.append((-np.inf, 0.0, np.zeros(V.shape[1], F64)))
            continue
        s = scale * (K[lo:hi] @ q)
        m = s.max()
        p = np.exp(s - m)
        parts.append((m, p.sum(), p @ V[lo:hi]))
    return parts


def splitk_combine(parts) -> np.ndarray:
    """o = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c, M = max_c m_c;
    empty splits (l = 0) contribute nothing."""
    live = [(m, l, o) for (m, l, o) in parts if l > 0]
    if not live:
        return np.zeros_like(parts[0][2])
    M = max(m for m, _, _ in live)
    num = sum(np.exp(m - M) * o for m, _, o in live)
    den = sum(np.exp(m - M) * l for m, l, _ in live)
    return num / den


# ------------------------------------------------------ KV-position scoring --

def kv_position_scores(q_obs, K, n: int, scale: float) -> np.ndarray:
    """Attention received by each cached position from the last n_obs prompt
    queries of one head, summed over those queries.

    ByteCross App. A: positions are ranked by attention from the last 64
    prompt tokens, pooled across query heads (one query head per KV head
    here, so pooling is the identity).  Query w sits at position
    n - n_obs + w and attends causally to positions 0..n - n_obs + w.
    """
    q_obs, K = _f64(q_obs), _f64(K)
    n_obs = q_obs.shape[0]
    acc = np.zeros(n, F64)
    for w in range(n_obs):
        t = n - n_obs + w
        s = scale * (K[:t + 1] @ q_obs[w])
        p = np.exp(s - s.max())
        acc[:t + 1] += p / p.sum()
    return acc


def moving_average(s, width: int) -> np.ndarray:
    """Centred width-``width`` mean, zero outside [0, n), divided by width
    (ByteCross App. A: smoothed with a width-7 average)."""
    s = _f64(s)
    n, half = s.shape[0], width // 2
    c = np.concatenate([[0.0], np.cumsum(s)])
    j = np.arange(n)
    hi = np.minimum(n, j + half + 1)
    lo = np.maximum(0, j - half)
    return (c[hi] - c[lo]) / width


def kv_select(q_obs, K, n: int, scale: float, budget: int, n_sink: int = 4,
              n_window: Optional[int] = None, width: int = 7):
    """Retained positions of one head: the ``budget`` best under the smoothed
    scores, with the sinks [0, n_sink) and the observation window
    [n - n_window, n) forced in (ByteCross §4.1 and App. A).  The budget
    counts the forced positions.  Scores are rounded to fp32 before the
    selection, the precision the selection kernel decides in.

    Returns (ascending positions, fp64 smoothed scores before forcing).
    """
    n_obs = np.asarray(q_obs).shape[0]
    n_window = n_obs if n_window is None else n_window
    raw = kv_position_scores(q_obs, K, n, scale)
    sm = moving_average(raw, width)
    forced = sm.astype(np.float32)
    forced[:min(n_sink, n)] = np.inf
    forced[max(0, n - n_window):n] = np.inf
    return topk_select(forced, min(budget, n)), sm


# --------------------------------------------------------------- the layer --

def decode_layer(x, W: dict, kv: KVState, pos: int, *, k_heads: int, k_neurons: int,
                 scale: float, eps: float = 1e-5, pred_act: str = "relu",
                 dense_attn: bool = False, dense_mlp: bool = False,
                 skip_nonpos: bool = True, hole_fill: bool = True,
                 sel_idx=None, sel_len=None, sel_end: Optional[int] = None,
                 window: Optional[Tuple[int, int]] = None):
    """One decode step of one pre-LN OPT-style layer under contextual sparsity.

    DejaVu §4.3, the sequential form:  S_A <- SP_A(y);  y~ <- MHA_{S_A}(y);
    S_M <- SP_M(y~);  y^ <- MLP_{S_M}(y~), with the residual stream and a
    LayerNorm before each block (App. B).  The predictors read the block's
    own normalised input.  The token sits at ``pos`` and attends to
    positions 0..pos (or, with ``sel_idx``, to the retained positions plus
    [sel_end, pos]; with ``window`` = (n_sink, win_len), to the KV window of
    pos + 1 positions).  Scores are rounded to fp32 before selection.

    x [B][d].  Returns (x_out [B][d], record dict).  Mutates ``kv``.
    """
    x = _f64(np.atleast_2d(x))
    B, d = x.shape
    h = W["w_qkv_t"].shape[1]
    N = W["w1_t"].shape[0]
    rec = {}
    y = layernorm(x, W["ln1_g"], W["ln1_b"], eps)
    if dense_attn:
        head_idx = np.arange(h)
    else:
        sA = predictor(y, W["pa1_t"], W["pa2_t"], pred_act).astype(np.float32)
        rec["head_scores"] = sA
        head_idx = union_sorted(topk_rows(sA, k_heads))
    rec["head_idx"] = head_idx
    q = qkv_step(y, W["w_qkv_t"], W["b_qkv"], head_idx, kv, pos, hole_fill)
    o = attention(q, kv, head_idx, pos + 1, scale, sel_idx, sel_len, sel_end, window)
    hres = out_proj(o, W["w_o_t"], W["b_o"], head_idx, residual=x)
    y2 = layernorm(hres, W["ln2_g"], W["ln2_b"], eps)
    if dense_mlp:
        idx = np.arange(N)
    else:
        sM = predictor(y2, W["pm1_t"], W["pm2_t"], pred_act).astype(np.float32)
        rec["neuron_scores"] = sM
        idx = union_sorted(topk_rows(sM, k_neurons))
    rec["neuron_idx"] = idx
    out, a = sparse_mlp(y2, W["w1_t"], W["b1"], W["w2_t"], W["b2"], idx,
                        residual=hres, skip_nonpos=skip_nonpos)
    rec.update(y=y, q=q, o=o, h=hres, y2=y2, a=a)
    return out, rec


def decode_layer_lookahead(x, W: dict, W_next: Optional[dict], kv: KVState, pos: int, *,
                           head_idx, neuron_idx, k_heads: int, k_neurons: int, scale: float,
                           eps: float = 1e-5, pred_act: str = "relu", skip_nonpos: bool = True,
                           hole_fill: bool = True, sel_idx=None, sel_len=None, sel_end: Optional[int] = None,
                           window: Optional[Tuple[int, int]] = None):
    """One decode step in DejaVu §4.3's parallel form (batch of one).

    This layer's sets S_A^l = ``head_idx`` and S_M^l = ``neuron_idx`` were
    predicted one layer ahead and are given; the layer computes
    y~ = MHA_{S_A^l}(y) and y^ = MLP_{S_M^l}(y~) with the same pre-LN residual
    structure as ``decode_layer``.  Alongside, the next layer's predictors
    (``W_next``'s pa1/pa2 and pm1/pm2) read this layer's normalised input
    y = LN1(x): S_A^{l+1} = top-k_heads(SP_A^{l+1}(y)), S_M^{l+1} =
    top-k_neurons(SP_M^{l+1}(y)) (DejaVu §4.3: both sets for layer l+1 come
    from layer l's input, computed in parallel with layer l; Explainer §4.3).
    ``head_idx`` / ``neuron_idx`` of None mean every head / neuron.

    x [1][d].  Returns (x_out [1][d], record dict with next_head_idx,
    next_neuron_idx and their fp32 scores).  Mutates ``kv``.
    """
    x = _f64(np.atleast_2d(x))
    assert x.shape[0] == 1, "the parallel form is defined here for one sequence"
    h = W["w_qkv_t"].shape[1]
    N = W["w1_t"].shape[0]
    rec = {}
    y = layernorm(x, W["ln1_g"], W["ln1_b"], eps)
    heads = np.arange(h) if head_idx is None else np.asarray(head_idx, dtype=np.int64)
    q = qkv_step(y, W["w_qkv_t"], W["b_qkv"], heads, kv, pos, hole_fill)
    o = attention(q, kv, heads, pos + 1, scale, sel_idx, sel_len, sel_end, window)
    hres = out_proj(o, W["w_o_t"], W["b_o"], heads, residual=x)
    y2 = layernorm(hres, W["ln2_g"], W["ln2_b"], eps)
    idx = np.arange(N) if neuron_idx is None else np.asarray(neuron_idx, dtype=np.int64)
    out, a = sparse_mlp(y2, W["w1_t"], W["b1"], W["w2_t"], W["b2"], idx, residual=hres, skip_nonpos=skip_nonpos)
    if W_next is not None:
        sA = predictor(y, W_next["pa1_t"], W_next["pa2_t"], pred_act).astype(np.float32)
        sM = predictor(y, W_next["pm1_t"], W_next["pm2_t"], pred_act).astype(np.float32)
        rec.update(next_head_scores=sA, next_neuron_scores=sM,
                   next_head_idx=topk_select(sA[0], k_heads), next_neuron_idx=topk_select(sM[0], k_neurons))
    rec.update(y=y, q=q, o=o, h=hres, y2=y2, a=a, head_idx=heads, neuron_idx=idx)
    return out, rec


# ------------------------------------------------------ threshold sparsity --

TEAL_INPUTS = ("qkv", "o", "fc1", "fc2")       # the input of each projection, in order


def teal_mask(x, t: float) -> np.ndarray:
    """x with every entry whose magnitude is not above t set to zero.

    ByteCross §4.1 and App. A: the projection branch is TEAL activation
    sparsity, a magnitude threshold on the input of each projection; a
    projection then reads only the weights of the input channels kept
    (§2: projection-side methods threshold active channels to cut weight
    reads)."""
    x = _f64(x)
    return np.where(np.abs(x) > t, x, 0.0)


def teal_layer(x, W: dict, kv: KVState, pos: int, *, thr: Sequence[float], scale: float, eps: float = 1e-5,
               sel_idx=None, sel_len=None, sel_end: Optional[int] = None,
               window: Optional[Tuple[int, int]] = None, masks: Optional[dict] = None):
    """One decode step of the pre-LN layer with threshold sparsity on the
    input of every projection and every head and neuron computed.

    thr = (t_qkv, t_o, t_fc1, t_fc2), the thresholds of the four projection
    inputs y = LN1(x), o (the heads' attention outputs), y2 = LN2(h) and the
    ReLU activations a.  K/V of the token are stored (fp16) for every head;
    attention reads every position, or the retained set / window as in
    ``attention`` (the composition with the KV branch, ByteCross §4.2).

    ``masks`` (optional, per input name a bool array [B][width]) replaces
    the threshold's decision for that input: a comparison with a device
    that rounds the inputs differently follows its decisions where an
    entry's magnitude lies within rounding of the threshold.

    x [B][d].  Returns (x_out [B][d], record with the inputs before the
    threshold, the decisions taken (``masks``) and ``kept``: per projection
    input, the channels some sequence of the batch keeps, ascending).
    Mutates ``kv``.
    """
    x = _f64(np.atleast_2d(x))
    B = x.shape[0]
    h = W["w_qkv_t"].shape[1]
    heads = np.arange(h)
    ts = dict(zip(TEAL_INPUTS, (float(t) for t in thr)))
    inputs, used = {}, {}

    def cut(name, v):
        inputs[name] = v.reshape(B, -1)
        m = np.abs(inputs[name]) > ts[name] if masks is None or name not in masks else np.asarray(masks[name], bool)
        used[name] = m
        return np.where(m, inputs[name], 0.0).reshape(v.shape)

    y = layernorm(x, W["ln1_g"], W["ln1_b"], eps)
    q = qkv_step(cut("qkv", y), W["w_qkv_t"], W["b_qkv"], heads, kv, pos, hole_fill=False)
    o = attention(q, kv, heads, pos + 1, scale, sel_idx, sel_len, sel_end, window)
    hres = out_proj(cut("o", o), W["w_o_t"], W["b_o"], heads, residual=x)
    y2 = layernorm(hres, W["ln2_g"], W["ln2_b"], eps)
    a = relu(cut("fc1", y2) @ _f64(W["w1_t"]).T + _f64(W["b1"]))
    out = hres + cut("fc2", a) @ _f64(W["w2_t"]) + _f64(W["b2"])
    kept = {k: np.flatnonzero(np.any(m, axis=0)) for k, m in used.items()}
    return out, dict(inputs=inputs, masks=used, kept=kept, q=q, h=hres)


def teal_layer_bytes(d: int, h: int, d_h: int, N: int, kept: dict, wb: int = 2) -> float:
    """Weight bytes one threshold-sparse step reads: the kept channels' rows
    of the input-major projections (Q/K/V: 3 h d_h per input channel; W^O:
    d; fc1: N; fc2: d), plus every bias."""
    rows = (len(kept["qkv"]) * 3 * h * d_h + len(kept["o"]) * d + len(kept["fc1"]) * N
            + len(kept["fc2"]) * d)
    return wb * (rows + 3 * h * d_h + d + N + d)


# --------------------------------------------------------- 4-bit weights --

W4_GROUP = 128


def quantize_w4(w) -> Tuple[np.ndarray, np.ndarray]:
    """Group-wise symmetric int4 of a [rows][cols] matrix (cols a multiple of
    128), the W4A16 weights DejaVu §5 combines with contextual sparsity
    (Compatibility with Quantization, Table 7; the pages give no quantizer,
    this one is a reading): per row, per group of 128 consecutive entries,
    the scale s = fp16(max|w| / 7) (the division in fp32) and the codes
    v = clamp(rint(w / s), -8, 7) (w / s in fp32, rint to nearest even; a
    group of zeros has s = 0 and v = 0).  Integer decisions are taken in
    fp32, the precision the device takes them in.
    Returns (v int8 [rows][cols], s fp16 [rows][cols / 128])."""
    w32 = np.asarray(w, dtype=np.float16).astype(np.float32)
    rows, cols = w32.shape
    g = w32.reshape(rows, cols // W4_GROUP, W4_GROUP)
    m = np.abs(g).max(axis=2)
    s16 = (m / np.float32(7.0)).astype(np.float16)
    s32 = s16.astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(s32 > 0, np.clip(np.rint(g / s32), -8, 7), 0.0)
    return v.reshape(rows, cols).astype(np.int8), s16


def pack_w4(v) -> np.ndarray:
    """The stored codes: entry c of a row in byte c // 2, the low nibble for
    even c, each nibble holding v + 8."""
    u = (np.asarray(v, dtype=np.int16) + 8).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def dequantize_w4(v, s) -> np.ndarray:
    """The weights the codes stand for, v * s, in float64."""
    v = np.asarray(v, dtype=np.float64)
    rows, cols = v.shape
    return (v.reshape(rows, cols // W4_GROUP, W4_GROUP) * _f64(s)[:, :, None]).reshape(rows, cols)


def sparse_mlp_w4(y, v1, s1, b1, v2, s2, b2, idx, residual=None, skip_nonpos: bool = False):
    """DejaVu Eq. (1) over the selected neurons with 4-bit weights: the
    sparse MLP of ``sparse_mlp`` on the dequantized rows of W1^T and W2^T
    (biases stay fp16).  v1, v2 int8 [N][d] codes; s1, s2 fp16 [N][d/128]."""
    idx = np.asarray(idx, dtype=np.int64)
    W1 = dequantize_w4(np.asarray(v1)[idx], np.asarray(s1)[idx])
    W2 = dequantize_w4(np.asarray(v2)[idx], np.asarray(s2)[idx])
    return sparse_mlp(y, W1, _f64(b1)[idx], W2, b2, np.arange(len(idx)), residual, skip_nonpos)


# ---------------------------------------------------------------- the stack --

def predict_sets(x, W: dict, k_heads: int, k_neurons: int, eps: float = 1e-5, pred_act: str = "relu"):
    """Sets of one layer from its own predictors on its normalised input
    y = LN1(x): S_A = top-k_heads(SP_A(y)), S_M = top-k_neurons(SP_M(y)).

    DejaVu §4.3's parallel form predicts layer l+1 from layer l's input; the
    first layer of a stack has no layer before it, so its sets come from its
    own input (the plainest reading consistent with that form).  Scores are
    rounded to fp32 before selection.  x [1][d].
    Returns (head_idx, neuron_idx, head scores, neuron scores).
    """
    y = layernorm(np.atleast_2d(x), W["ln1_g"], W["ln1_b"], eps)
    sA = predictor(y, W["pa1_t"], W["pa2_t"], pred_act).astype(np.float32)
    sM = predictor(y, W["pm1_t"], W["pm2_t"], pred_act).astype(np.float32)
    return topk_select(sA[0], k_heads), topk_select(sM[0], k_neurons), sA, sM


def decode_stack_lookahead(x, Ws: Sequence[dict], kvs: Sequence[KVState], pos: int, *, k_heads: int,
                           k_neurons: int, scale: float, eps: float = 1e-5, pred_act: str = "relu",
                           skip_nonpos: bool = True, hole_fill: bool = True,
                           window: Optional[Tuple[int, int]] = None, n_dense_prefix: int = 0):
    """One token through a stack of layers in DejaVu §4.3's parallel form.

    The output of layer l is the input of layer l+1 (§3, the residual
    stream).  The first ``n_dense_prefix`` layers compute every head and
    neuron (Explainer, "Handling the first layer").  The first sparse layer
    runs on the sets the last dense layer predicted, or, with no dense
    prefix, layer 0 on the sets its own predictors give for LN1(x)
    (``predict_sets``); every later layer runs on the sets layer l-1's
    ``decode_layer_lookahead`` predicted from its normalised input with
    layer l's predictors.  Every layer's token sits at ``pos``.

    x [1][d].  Returns (x_out [1][d], list of per-layer records, each with
    the layer's input ``x`` and the sets it ran on).  Mutates ``kvs``.
    """
    P = n_dense_prefix
    heads = neurons = None
    if P == 0:
        heads, neurons, _, _ = predict_sets(x, Ws[0], k_heads, k_neurons, eps, pred_act)
    recs = []
    for l, W in enumerate(Ws):
        W_next = Ws[l + 1] if l + 1 < len(Ws) and l + 1 >= P else None
        x_in = _f64(np.atleast_2d(x))
        x, rec = decode_layer_lookahead(x, W, W_next, kvs[l], pos, head_idx=heads, neuron_idx=neurons,
                                        k_heads=k_heads, k_neurons=k_neurons, scale=scale, eps=eps,
                                        pred_act=pred_act, skip_nonpos=skip_nonpos, hole_fill=hole_fill,
                                        window=window)
        rec["x"] = x_in
        recs.append(rec)
        if W_next is not None:
            heads, neurons = rec["next_head_idx"], rec["next_neuron_idx"]
    return x, recs
