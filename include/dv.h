/*
 * dv.h -- C ABI of libdv, the decode step of contextual sparsity on AMD
 * MI355X (gfx950).
 *
 * Pages cited:
 *   DejaVu    "Deja Vu: Contextual Sparsity for Efficient LLMs at Inference
 *             Time" (arXiv 2310.17157).
 *   ByteCross "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM
 *             Decoding" (arXiv 2609.33889v1).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named as device memory must be HIP device allocations on the
 *   current device; scalars (sizes, counts, positions) are host values.
 * - Every call validates its arguments on the host first.  On error nothing
 *   is enqueued, a DV_ERR_* code is returned and dv_last_error() holds a
 *   message for the calling thread.  A failed launch returns DV_ERR_HIP.
 *   Faults inside a kernel surface at the caller's next synchronisation.
 * - Every call enqueues its kernels on `stream` (a hipStream_t; NULL is the
 *   null stream) and returns without synchronising.  The library never
 *   allocates, frees or synchronises.
 * - Scratch memory is the caller's `ws` of at least the size the matching
 *   *_workspace_bytes() query returns, 256-byte aligned.  Its first 4096
 *   bytes are reserved for counters; zero fill the workspace before its
 *   first use.  One workspace serves any number of calls, of any shapes,
 *   issued in order on one stream; calls that overlap in time must use
 *   separate workspaces.
 * - d (the model width) is at most 261,888 (one counter per 256 columns).
 * - Weight pointers must be 16-byte aligned and a weight row (d elements)
 *   must be a multiple of 16 bytes (d % 8 == 0 for fp16, d % 4 == 0 for
 *   fp32), else DV_ERR_ALIGN.
 * - Index sets are int32 and ascending, as dv_topk_select writes them.
 * - Layouts are row-major.  Weights are stored so that each selected unit is
 *   one contiguous run (DejaVu §4.4 "Memory coalescing": W1, W2 and W^O are
 *   kept transposed):
 *     w1_t, w2_t  [N][d]        row j = neuron j's fc1 / fc2 weights
 *     w_qkv_t     [3][h][d_h][d] Q, K, V block of head i = [which][i]
 *     w_o_t       [h*d_h][d]    rows i*d_h..i*d_h+d_h-1 = W_i^O
 *     p1_t [r][d], p2_t [n_out][r]   predictor layers, transposed
 *     K, V cache  fp16 [B][h][max_len][d_h]
 *   Activations (x, y, q, o, scores) are fp32.
 */
#ifndef DV_H
#define DV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DV_API_VERSION 1

typedef enum {
    DV_OK = 0,
    DV_ERR_NULL = 1,        /* a required pointer is NULL */
    DV_ERR_SHAPE = 2,       /* a size is out of its valid range or sizes disagree */
    DV_ERR_DTYPE = 3,       /* unknown dtype, activation or mode value */
    DV_ERR_ALIGN = 4,       /* pointer or row not 16-byte aligned */
    DV_ERR_RANGE = 5,       /* k > n, pos >= max_len, count > capacity ... */
    DV_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than its query */
    DV_ERR_UNSUPPORTED = 7, /* a valid combination this build does not implement */
    DV_ERR_HIP = 8          /* a HIP launch failed */
} dv_status;

typedef enum { DV_F32 = 0, DV_F16 = 1, DV_U32 = 2 /* dv_fill_normal only */ } dv_dtype;
typedef enum { DV_ACT_NONE = 0, DV_ACT_RELU = 1 } dv_act;
typedef enum { DV_PROJ_QKV = 0, DV_PROJ_OUT = 1 } dv_proj_mode;

/* dv_sparse_mlp / dv_decode_layer flags */
#define DV_SKIP_NONPOS_FC2 0x1u  /* do not read fc2 rows of neurons whose ReLU output is 0 */
#define DV_DENSE_ATTN      0x2u  /* every head, no head predictor */
#define DV_DENSE_MLP       0x4u  /* every neuron, no neuron predictor */
#define DV_HOLE_FILL       0x8u  /* recompute skipped heads' K/V (DejaVu §4.2) */
#define DV_KV_SELECT       0x10u /* attend to retained KV positions only (ByteCross §4.1) */
#define DV_ADVANCE_POS     0x20u /* dv_decode_layer: add 1 to *kv.pos_dev when the step is done */
#define DV_LOOKAHEAD       0x40u /* dv_decode_layer: DejaVu §4.3 parallel form (see dv_layer_state) */
#define DV_KV_WINDOW       0x80u /* attend to the KV window of dv_decode_cfg.win_* (ByteCross §5.1) */
#define DV_TEAL            0x100u /* threshold sparsity on every projection input (ByteCross §4.1), see dv_layer_state */

int dv_api_version(void);
const char* dv_status_str(int status);
/* Message of the last error returned on the calling thread ("" if none). */
const char* dv_last_error(void);

/* ------------------------------------------------------------------------
 * LayerNorm: y[b] = (x[b] - mean) / sqrt(var + eps) * gamma + beta, the
 * normalisation before each block (DejaVu App. B), population variance.
 * x, y: device fp32 [B][d]; gamma, beta: device fp32 [d].  y may alias x.
 */
dv_status dv_layernorm(const float* x, int B, int d, const float* gamma, const float* beta,
                       float eps, float* y, void* stream);

/* ------------------------------------------------------------------------
 * Sparsity predictor, DejaVu §4.1 (MLP) and §4.2 (heads, same
 * architecture): scores[b] = act(y[b] P1) P2, a two-layer fully connected
 * network without biases, one score per neuron or head.
 *   y       device fp32 [B][d]
 *   p1_t    device [r][d]      (P1 transposed), dtype wdt
 *   p2_t    device [n_out][r]  (P2 transposed), dtype wdt
 *   act     dv_act applied to the r hidden units
 *   scores  device fp32 [B][n_out]
 * Accumulation is fp32.  1 <= B <= 16.
 */
size_t dv_predict_workspace_bytes(int B, int d, int r, int wdt);
dv_status dv_predict(const float* y, int B, int d, const void* p1_t, int r, const void* p2_t,
                     int n_out, int wdt, int act, float* scores, void* ws, size_t ws_bytes,
                     void* stream);

/* ------------------------------------------------------------------------
 * Top-k selection of the set S (DejaVu §2.3: S_M subset of [4d], S_A
 * subset of [h], under a budget on its size).  Row b of `scores` yields the
 * k indices that come first in the order: score descending, ties to the
 * lower index, NaN after every number (+0 and -0 tie).  Written ascending.
 *   scores      device fp32 [B][n]
 *   idx         device int32 [B][k]
 *   union_idx   device int32 [n] or NULL: ascending union of the B sets
 *               (DejaVu §5.2 / App. C.1, the batch union), when B > 1
 *   union_count device int32 [1] or NULL: size of that union
 * 0 <= k <= n <= 4194304 (2^22); k > n gives DV_ERR_RANGE.  1 <= B <= 64.
 * The union needs n <= 262144 (2^18).
 */
size_t dv_topk_workspace_bytes(int B, int n, int k);
dv_status dv_topk_select(const float* scores, int B, int n, int k, int32_t* idx,
                         int32_t* union_idx, int32_t* union_count, void* ws, size_t ws_bytes,
                         void* stream);

/* ------------------------------------------------------------------------
 * Sparse MLP, DejaVu §2.3 Eq. (1) with OPT's biases:
 *   a[b][u]  = max(0, w1_t[idx[u]] . y[b] + b1[idx[u]])
 *   out[b]   = residual[b] + b2 + sum_u a[b][u] * w2_t[idx[u]]
 * Every row b uses the same set idx (a batch passes the union).  With
 * DV_SKIP_NONPOS_FC2 the fc2 rows of neurons with a[b][u] == 0 for every b
 * are not read (the second layer is sparsified by the ReLU, DejaVu §2.3).
 *   y        device fp32 [B][d]
 *   w1_t, w2_t device [N][d]; b1 device [N]; b2 device [d]; dtype wdt
 *   idx      device int32 [n_idx_max] ascending, or NULL = every neuron
 *            (then n_idx_max must equal N)
 *   n_idx_dev device int32 [1] or NULL: the count actually used, <= n_idx_max
 *   residual device fp32 [B][d] or NULL
 *   out      device fp32 [B][d] (must not alias y or residual)
 *   act_out  device fp32 [B][n_idx_max] or NULL: the activations a
 *   fc2_rows device int32 [1] or NULL: incremented by the number of fc2
 *            rows read (the caller zeroes it)
 * 1 <= B <= 16.
 */
size_t dv_sparse_mlp_workspace_bytes(int B, int d, int n_idx_max, int wdt);
dv_status dv_sparse_mlp(const float* y, int B, int d, int N, const void* w1_t, const void* b1,
                        const void* w2_t, const void* b2, int wdt, const int32_t* idx,
                        int n_idx_max, const int32_t* n_idx_dev, const float* residual,
                        float* out, float* act_out, int32_t* fc2_rows, unsigned flags, void* ws,
                        size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * dv_sparse_mlp without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  Same arguments, results and errors as
 * dv_sparse_mlp; its scratch is a device array of DV_NOALLOC_SCRATCH_BYTES
 * built into the library (each GPU the library runs on holds its own copy
 * until the process ends).  A shape whose dv_sparse_mlp_workspace_bytes()
 * exceeds that size gets DV_ERR_WORKSPACE.  The call allocates nothing
 * (no hipMalloc, no allocating library routine).  Every call on one GPU
 * uses that GPU's one array: calls that overlap in time on the same GPU
 * (different streams, different host threads) race and must not be made.
 */
#define DV_NOALLOC_SCRATCH_BYTES (8u << 20)
dv_status dv_sparse_mlp_noalloc(const float* y, int B, int d, int N, const void* w1_t, const void* b1,
                                const void* w2_t, const void* b2, int wdt, const int32_t* idx, int n_idx_max,
                                const int32_t* n_idx_dev, const float* residual, float* out, float* act_out,
                                int32_t* fc2_rows, unsigned flags, void* stream);

/* ------------------------------------------------------------------------
 * 4-bit weights (W4A16).  DejaVu §5 (Compatibility with Quantization,
 * Table 7) applies 4-bit weight quantization together with contextual
 * sparsity without naming the quantizer; this format is the library's:
 * a matrix w [rows][cols] (fp16, cols a multiple of 128) is stored as
 *   q       uint8 [rows][cols / 2]: entry c of a row in byte c / 2, the low
 *           nibble for even c; a nibble holds v + 8, v in [-8, 7]
 *   scales  fp16 [rows][cols / 128]: per row and group of 128 entries,
 *           s = fp16(max |w| / 7) (fp32 division, round to nearest even)
 * and stands for w' = v * s, with v = clamp(rint(w / s), -8, 7) (w / s in
 * fp32, correctly rounded; rint to nearest even) and v = 0 where s = 0.
 * w must be finite.  dv_quantize_w4 writes q and scales from w (device
 * pointers, 16-byte aligned; rows >= 1; DV_ERR_SHAPE for cols not a
 * multiple of 128).
 */
dv_status dv_quantize_w4(const void* w, int rows, int cols, uint8_t* q, void* scales, void* stream);

/* dv_sparse_mlp (DejaVu §2.3 Eq. 1, the same a and out) with fc1 and fc2
 * weights in the 4-bit format above, dequantized inside the gathers:
 *   q1, s1   W1^T [N][d] as codes and scales; q2, s2 W2^T [N][d] likewise
 *   b1 fp16 [N], b2 fp16 [d]
 * Batch of one (B = 1); d a multiple of 128 and at most 16384; other
 * arguments as in dv_sparse_mlp (flags: DV_SKIP_NONPOS_FC2). */
size_t dv_sparse_mlp_w4_workspace_bytes(int d, int n_idx_max);
dv_status dv_sparse_mlp_w4(const float* y, int d, int N, const uint8_t* q1, const void* s1, const void* b1,
                           const uint8_t* q2, const void* s2, const void* b2, const int32_t* idx, int n_idx_max,
                           const int32_t* n_idx_dev, const float* residual, float* out, float* act_out,
                           int32_t* fc2_rows, unsigned flags, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * KV state of one layer, updated by dv_sparse_attn_proj(DV_PROJ_QKV).
 *   k_cache, v_cache  device fp16 [B][h][max_len][d_h]
 *   pos               slot written by this step, 0 <= pos < max_len
 *   y_buf             device fp32 [B][max_len][d]: every step's layer input,
 *                     kept for heads that were not selected (DejaVu §4.2);
 *                     16-byte aligned (else DV_ERR_ALIGN); NULL disables
 *                     hole fill
 *   valid_upto        device int32 [B][h]: last position whose K/V head i
 *                     holds; NULL disables hole fill
 *   pos_dev           device int32 [1] or NULL: when set, the slot is read
 *                     from here when the kernels run (so a captured HIP
 *                     graph can be replayed step after step) and `pos` is
 *                     only its upper bound, used to size launches; a run-time
 *                     value outside [0, max_len) makes the step write nothing
 * With hole fill, a selected head whose valid_upto < pos - 1 first gets its
 * K/V at positions valid_upto+1 .. pos-1 recomputed from y_buf, then
 * valid_upto = pos.  Without it, skipped slots keep their old contents.
 */
typedef struct {
    void* k_cache;
    void* v_cache;
    int max_len;
    int pos;
    float* y_buf;
    int32_t* valid_upto;
    int32_t* pos_dev;
} dv_kv_state;

/* ------------------------------------------------------------------------
 * Sparse attention projections, DejaVu §2.3 Eq. (2) / §4.2 / App. E.
 * DV_PROJ_QKV: for each selected head i = head_idx[s]:
 *     q[b][s] = W_i^Q y[b] + b^Q_i;  k, v likewise, rounded to fp16 (RNE)
 *     and written to slot pos of head i; y[b] saved to y_buf[b][pos].
 *   w_t  [3][h][d_h][d]; bias [3][h][d_h]; in = y [B][d]; out = q [B][n_sel][d_h];
 *   residual unused; kv required.
 * DV_PROJ_OUT: out[b] = residual[b] + bias + sum_s o[b][s] . W^O_{head_idx[s]}
 *   w_t  [h*d_h][d]; bias [d]; in = o [B][n_sel][d_h]; out [B][d]; kv unused.
 * head_idx device int32 [n_sel] ascending, or NULL = heads 0..n_sel-1 (dense).
 * The head set is shared by the batch.  d_h in {32, 64, 128, 256}.
 */
size_t dv_attn_proj_workspace_bytes(int mode, int B, int d, int h, int d_h, int n_sel, int wdt);
dv_status dv_sparse_attn_proj(int mode, int B, int d, int h, int d_h, const int32_t* head_idx,
                              int n_sel, const void* w_t, const void* bias, int wdt,
                              const float* in, const float* residual, float* out,
                              const dv_kv_state* kv, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Which cached positions attention reads.
 *   n_ctx    positions 0..n_ctx-1 exist (the current token included)
 *   sel_idx  device int32 [B][h][sel_cap] or NULL (dense): per head, the
 *            retained positions (ascending, each < sel_end) of the KV
 *            branch (ByteCross §4.1: top positions per KV head kept)
 *   sel_len  device int32 [B][h]: entries of sel_idx in use (<= sel_cap)
 *   sel_end  positions sel_end..n_ctx-1 are always read (the cache keeps
 *            receiving entries, ByteCross §3.2)
 *   n_ctx_dev device int32 [1] or NULL: when set, the count is read from
 *            here at run time (clamped to [0, n_ctx]) and n_ctx is its bound
 *   win_sink, win_len  (win_len > 0, sel_idx NULL) the KV window policy
 *            (ByteCross §5.1 and App. A): the positions < win_sink and the
 *            last win_len positions before n_ctx, read in place; the window
 *            slides as tokens are appended.  Both zero: every position.
 *            win_len > 0 with sel_idx set is DV_ERR_UNSUPPORTED.
 */
typedef struct {
    const void* k_cache;
    const void* v_cache;
    int h;
    int max_len;
    int n_ctx;
    const int32_t* sel_idx;
    const int32_t* sel_len;
    int sel_cap;
    int sel_end;
    const int32_t* n_ctx_dev;
    int win_sink;
    int win_len;
} dv_kv_view;

/* ------------------------------------------------------------------------
 * Split-K decode attention over the selected heads, DejaVu §2.3 Eq. (2):
 *   o[b][s] = softmax(scale * q[b][s] . K_i^T) V_i,  i = head_idx[s],
 * over the positions of `kv`.  The positions are split into num_splits
 * ranges read in parallel; each yields (max, sum of exp, weighted V) and a
 * combine step merges them (the split-K kernel ByteCross §4.1 times every
 * mode with).  Empty ranges contribute nothing; a head with no position
 * gets o = 0.
 *   q  device fp32 [B][n_sel][d_h];  o device fp32 [B][n_sel][d_h]
 *   head_idx as in dv_sparse_attn_proj;  num_splits 0 = chosen by the library
 */
size_t dv_splitk_workspace_bytes(int B, int n_sel, int d_h, int max_positions, int num_splits);
dv_status dv_splitk_attn(const float* q, int B, int d_h, const int32_t* head_idx, int n_sel,
                         const dv_kv_view* kv, float scale, int num_splits, float* o, void* ws,
                         size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Attention-scored KV selection scores, ByteCross §4.1 / App. A: the
 * attention each cached position receives from the last n_obs prompt
 * queries (query w at position n - n_obs + w attends causally), summed over
 * those queries, then a centred width-`width` moving average (zero outside
 * [0, n), divided by width); positions < n_sink and >= n - n_window are
 * set to +inf so that a following dv_topk_select(k = budget) keeps them.
 *   q_obs   device fp16 [B][h][n_obs][d_h]
 *   scores  device fp32 [B][h][n]
 * width odd, 1 <= width <= 63.
 */
size_t dv_kv_score_workspace_bytes(int B, int h, int n, int n_obs);
dv_status dv_kv_score(const void* q_obs, int B, int h, int d_h, int n_obs, const dv_kv_view* kv,
                      float scale, int n_sink, int n_window, int width, float* scores, void* ws,
                      size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * One decode step of one pre-LN OPT-style layer, DejaVu §4.3 sequential
 * form: y = LN1(x); S_A = top-k_heads(SP_A(y)); h = x + MHA_{S_A}(y);
 * y2 = LN2(h); S_M = top-k_neurons(SP_M(y2)); x_out = h + MLP_{S_M}(y2).
 * A batch uses the union of its rows' neuron sets (DejaVu App. C.1); head
 * sparsity needs B == 1 in this build (DV_ERR_UNSUPPORTED otherwise).
 * With st->kv.pos_dev set the step position is read on the device (and
 * n_ctx = position + 1), so the whole call can be captured in a HIP graph
 * once and replayed; DV_ADVANCE_POS then moves the position on by one.
 */
typedef struct {
    int B, d, h, d_h, N;
    int r_attn, r_mlp;        /* predictor ranks */
    int k_heads, k_neurons;   /* budgets (ignored with DV_DENSE_ATTN / DV_DENSE_MLP) */
    int wdt;                  /* dv_dtype of every weight */
    int pred_act;             /* dv_act of the predictors' hidden layer */
    float eps;                /* LayerNorm epsilon */
    float scale;              /* attention score scale */
    unsigned flags;           /* DV_* flags above */
    int win_sink, win_len;    /* DV_KV_WINDOW: sink and recent positions, as in dv_kv_view */
    int n_dense_prefix;       /* dv_decode_stack: the first n layers run dense (>= 0; ignored by dv_decode_layer) */
} dv_decode_cfg;

typedef struct {
    const float *ln1_g, *ln1_b, *ln2_g, *ln2_b;   /* fp32 [d] */
    const void *w_qkv_t, *b_qkv;                   /* [3][h][d_h][d], [3][h][d_h] */
    const void *w_o_t, *b_o;                       /* [h*d_h][d], [d] */
    const void *w1_t, *b1, *w2_t, *b2;             /* [N][d], [N], [N][d], [d] */
    const void *pa1_t, *pa2_t;                     /* [r_attn][d], [h][r_attn] */
    const void *pm1_t, *pm2_t;                     /* [r_mlp][d], [N][r_mlp] */
    /* DV_TEAL only: the projections stored input-major, so that an input
     * channel's weights are one contiguous row (W^O and W2^T above already
     * are): w_qkv_in[i][which][head][e] = w_qkv_t[which][head][e][i],
     * w1_in[i][j] = w1_t[j][i]. */
    const void *w_qkv_in;                          /* [d][3][h][d_h] */
    const void *w1_in;                             /* [d][N] */
} dv_layer_weights;

typedef struct {
    dv_kv_state kv;             /* the cache and hole-fill state */
    const int32_t* sel_idx;     /* DV_KV_SELECT: as in dv_kv_view */
    const int32_t* sel_len;
    int sel_cap;
    int sel_end;
    /* optional device outputs (NULL to skip) */
    int32_t* head_idx_out;      /* [k_heads] selected heads */
    int32_t* neuron_idx_out;    /* [min(N, B*k_neurons)] selected (union) neurons */
    int32_t* neuron_count_out;  /* [1] number of entries in neuron_idx_out */
    int32_t* fc2_rows_out;      /* [1] incremented by the fc2 rows read */
    /* DV_LOOKAHEAD (DejaVu §4.3, the parallel form; B == 1).  This layer's
     * sets were predicted one layer ahead and are given; the layer computes
     * h = x + MHA_{S_A}(LN1(x)) and x_out = h + MLP_{S_M}(LN2(h)).  Alongside,
     * the next layer's predictors read this layer's y = LN1(x):
     * next_head_idx = top-k_heads(SP_A'(y)), next_neuron_idx =
     * top-k_neurons(SP_M'(y)), with this call's ranks, budgets and act.  With
     * aux_stream set, those predictions run on it: the call records ev_fork
     * on `stream`, makes aux_stream wait for it, records ev_join on
     * aux_stream after the predictions and makes `stream` wait for ev_join
     * before returning (a captured graph gets two branches).  Without
     * aux_stream they run on `stream` as extra workgroups of this layer's
     * own launches (both predictors' first layers beside Q/K/V, the second
     * layers and head selection beside attention, the neuron selection
     * split over the output projection, its finalize and fc2; when both
     * predictors are given and the neuron count is a multiple of 4 and at
     * most 20480, else in launches of their own).  The results are the
     * same either way.  The events and the stream are the caller's (created
     * once, reused by every call).  The workspace of a look-ahead call must
     * not be shared with a call running concurrently.  next_head_idx and
     * next_neuron_idx are written while the call's launches still read
     * head_idx_in and neuron_idx_in: the four buffers must not overlap
     * (else DV_ERR_RANGE). */
    const int32_t* head_idx_in;     /* [k_heads] ascending; ignored with DV_DENSE_ATTN */
    const int32_t* neuron_idx_in;   /* [k_neurons] ascending; ignored with DV_DENSE_MLP */
    const void *next_pa1_t, *next_pa2_t;   /* next layer's head predictor, or NULL for none */
    const void *next_pm1_t, *next_pm2_t;   /* next layer's neuron predictor, or NULL for none */
    int32_t* next_head_idx;         /* [k_heads] out, ascending */
    int32_t* next_neuron_idx;       /* [k_neurons] out, ascending */
    void* aux_stream;               /* hipStream_t, or NULL */
    void* ev_fork;                  /* hipEvent_t, required with aux_stream */
    void* ev_join;                  /* hipEvent_t, required with aux_stream */
    /* DV_TEAL (with DV_DENSE_ATTN and DV_DENSE_MLP; not with DV_LOOKAHEAD or
     * DV_HOLE_FILL): the projection branch of ByteCross (§4.1, App. A; TEAL
     * activation sparsity).  Every head and neuron is computed; each
     * projection reads only the input-major rows of the input channels whose
     * magnitude exceeds its threshold (for a batch: in some sequence; each
     * sequence zeroes its own entries at or below the threshold):
     *   teal_thr = {t_qkv on y = LN1(x), t_o on the heads' attention
     *   outputs, t_fc1 on y2 = LN2(h), t_fc2 on the ReLU activations}.
     * teal_rows_out (device int32 [4] or NULL) is incremented by the rows
     * each of the four projections read.  teal_rec (device fp32
     * [4][B][max(d, h*d_h, N)] or NULL) receives the four inputs before the
     * threshold (for calibrating thresholds). */
    float teal_thr[4];
    int32_t* teal_rows_out;
    float* teal_rec;
} dv_layer_state;

size_t dv_decode_workspace_bytes(const dv_decode_cfg* cfg, int max_len);
dv_status dv_decode_layer(const dv_layer_weights* w, const dv_decode_cfg* cfg,
                          const dv_layer_state* st, const float* x_in, float* x_out, void* ws,
                          size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * A stack of n_layers decoder layers for one token (DejaVu §3: the token
 * passes every layer; §4.3: layer l's input predicts layer l+1's sets;
 * ByteCross §3.1: one step reads every layer's projections and KV).  The
 * output of layer l is the input of layer l+1; x_in feeds layer 0 and the
 * last layer writes x_out.  Every layer uses `cfg` (with per-layer weights
 * and state from layers[l]).
 *
 * The first cfg->n_dense_prefix layers compute every head and neuron
 * (Explainer, "Handling the first layer": the first one or two layers run
 * dense and prediction starts after them); the layers after them use cfg.
 *
 * With DV_LOOKAHEAD (batch of one), layer l runs on the sets layer l-1
 * predicted from its LN1 input, with layer l's predictors, while computing
 * its own block.  The first sparse layer's sets come from the last dense
 * layer, or, without a dense prefix, layer 0's from its own predictors on
 * LN1(x_in) (there is no layer before it).  The sets live in
 *   head_sets    device int32 [n_layers][k_heads]   (required unless DV_DENSE_ATTN)
 *   neuron_sets  device int32 [n_layers][k_neurons] (required unless DV_DENSE_MLP)
 * and hold, after the call, the sets each sparse layer ran on (the rows of
 * the dense prefix are not written).  Without it each
 * layer predicts its own blocks' sets in the sequential form, and the
 * optional head_sets / neuron_sets (NULL to skip) receive them; with a
 * batch, row l of neuron_sets ([n_layers][min(N, B*k_neurons)]) holds the
 * union and neuron_counts (device int32 [n_layers] or NULL) its size.
 * fc2_rows (device int32 [1] or NULL) is incremented by the fc2 rows read.
 * x_trace (device fp32 [n_layers - 1][B][d] or NULL) receives the output of
 * every layer but the last (the input of the next), in place of scratch.
 * With DV_ADVANCE_POS a decode position shared by several layers (the same
 * kv.pos_dev) moves on once, in the last layer that uses it.
 * Every layer is checked before anything is enqueued; the message names
 * the failing layer.  The workspace is dv_stack_workspace_bytes(cfg,
 * largest max_len) bytes; layers run in order on `stream`.
 */
typedef struct {
    dv_layer_weights w;
    dv_kv_state kv;
    const int32_t* sel_idx;     /* DV_KV_SELECT: as in dv_kv_view */
    const int32_t* sel_len;
    int sel_cap;
    int sel_end;
    float teal_thr[4];          /* DV_TEAL: as in dv_layer_state */
    int32_t* teal_rows_out;
    float* teal_rec;
} dv_stack_layer;

size_t dv_stack_workspace_bytes(const dv_decode_cfg* cfg, int max_len);
dv_status dv_decode_stack(const dv_stack_layer* layers, int n_layers, const dv_decode_cfg* cfg, int32_t* head_sets,
                          int32_t* neuron_sets, int32_t* neuron_counts, int32_t* fc2_rows, const float* x_in,
                          float* x_out, float* x_trace, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Seeded normal samples written into device memory (synthetic weights,
 * caches and inputs of stacks too large to pass through the host).  The
 * generator is Philox-4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
 * Random Numbers: As Easy as 1, 2, 3", SC 2011) with the Box-Muller
 * transform:
 *   element i of stream (seed, stream) lies in Philox block b = i / 4, whose
 *   counter is (b mod 2^32, b / 2^32, stream mod 2^32, stream / 2^32) and
 *   key (seed mod 2^32, seed / 2^32); its words x0..x3 form the pairs
 *   (x0, x1) and (x2, x3); for a pair (xa, xb), u = (xa + 1) / 2^32,
 *   v = xb / 2^32, r = sqrt(-2 ln u), za = r cos(2 pi v), zb = r sin(2 pi v)
 *   in double; element 4b + j takes z_j, and its value is
 *   mean + std * z_j in double, rounded to float (then to half, RNE).
 *   out     device, 16-byte aligned: n elements of dtype DV_F32, DV_F16, or
 *           DV_U32 (the raw words x_j)
 *   offset  index of out[0] within the stream (a range can be regenerated)
 */
dv_status dv_fill_normal(void* out, uint64_t n, int dtype, uint64_t seed, uint64_t stream, uint64_t offset,
                         float mean, float std, void* hip_stream);

/* ------------------------------------------------------------------------
 * Byte account of one decode step of one layer (ByteCross §3.1: a step
 * reads the projection weights it keeps and the KV entries it attends to;
 * DejaVu §2.3 Eqs. 1-2 and §4.1-4.2 name what is read): the algorithmic
 * bytes, i.e. what the step must move at least once, by kernel and by kind.
 *   n_att     positions each selected head attends to
 *   fc2_rows  fc2 rows read (the device count of dv_layer_state.fc2_rows_out
 *             per step; k_neurons when every selected row is read)
 *   holes     recomputed K/V positions summed over heads
 * Host only: nothing is enqueued.
 */
typedef struct {
    double head_pred, neuron_pred, qkv, out_proj, fc1, fc2;  /* weight and bias bytes by kernel */
    double weights;     /* their sum */
    double kv_read;     /* K and V entries attended to */
    double kv_write;    /* K/V appended and recomputed */
    double act;         /* fp32 activations, LayerNorm vectors, stored inputs re-read */
    double total;
} dv_bytes;
dv_status dv_bytes_read(const dv_decode_cfg* cfg, double n_att, double fc2_rows, double holes, dv_bytes* out);

/* The same account for a DV_TEAL step (ByteCross §3.1 with §4.1's
 * projection branch): each projection reads the input-major rows of its
 * kept input channels plus its bias; every head attends to n_att
 * positions.  kept[4] = channels kept per step for the Q/K/V, W^O, fc1 and
 * fc2 inputs (the device counts of dv_layer_state.teal_rows_out per step),
 * each within [0, width of that input].  cfg must carry DV_TEAL.  Host
 * only. */
dv_status dv_bytes_read_teal(const dv_decode_cfg* cfg, double n_att, const double* kept, dv_bytes* out);

/* ------------------------------------------------------------------------
 * Launch timing, for measuring one kernel role inside the real decode step
 * (effective bandwidth of that kernel on the bytes it must read, ByteCross
 * §4.4 reports bandwidth as a share of peak per path).  While set on the
 * calling thread, each launch of role `kernel` made by dv_decode_layer or
 * dv_decode_stack is bracketed by hipEventRecord(events[2i]) before and
 * events[2i + 1] after it, on the launch's stream (also inside a stream
 * capture), for the first n_events / 2 launches.  `events` is a host array
 * of hipEvent_t the caller created (with timing) and keeps alive until the
 * recorded work has run.  kernel 0 turns timing off.
 * dv_launch_events_used() gives the number of events recorded since.
 */
#define DV_KERNEL_QKV  1   /* sparse Q/K/V projection with KV append and hole fill */
#define DV_KERNEL_ATTN 2   /* split-K attention */
#define DV_KERNEL_OUT  3   /* output projection gather-AXPY (its reduction launch excluded) */
#define DV_KERNEL_FC1  4   /* sparse fc1 */
#define DV_KERNEL_FC2  5   /* sparse fc2 gather-AXPY (its reduction launch excluded) */
dv_status dv_time_launches(int kernel, void** events, int n_events);
int dv_launch_events_used(void);

#ifdef __cplusplus
}
#endif
#endif /* DV_H */
