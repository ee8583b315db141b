/*
 * mtgr.h - C ABI of the MTGR HSTU layer library for AMD Instinct MI355X (gfx950).
 *
 * The library computes the hot path of one MTGR ranking layer over a jagged
 * batch of user-aggregated token rows [U | S | R | C]:
 *   Group LayerNorm -> fused UQKV projection + SiLU -> SiLU attention under
 *   the dynamic mask -> GroupNorm(attention output) * U -> output projection
 *   + residual, and the backward of all of it.
 *
 * Sources (page titles and sections):
 *   [blog] "MTGR：工业级生成式推荐框架": 4 (aggregated row), 7 (HSTU encoder),
 *          8 (Group-Layer Normalization), 9 (dynamic masking).
 *   [wiki] "MTGR: Industrial-Scale Generative Recommendation Framework in
 *          Meituan/es", Métodos: attention and X-update equations.
 *   [pd]   "MTGR：美团外卖生成式推荐Scaling Law落地实践", 模型怎么搭 (layer
 *          order: linear+SiLU gives U,Q,K,V; SiLU(QK^T) without softmax;
 *          normalise the aggregate, gate by U, one linear layer),
 *          训练数据怎么组织 (jagged rows, timestamps kept for the mask).
 *   [fr]   "MTGR：混合范式建模" (fun-rec 7.3): 7.3.1 (loss at candidate
 *          positions), 7.3.3 (GLN formula), 7.3.4 (the three mask rules).
 *   [blog] also 5.4, 6, 7 (candidate head and loss) and 11.3 (batches
 *          sized by token count).
 *   [dr]   paper-daily deep reading of the Meituan blog post: 2 方法详解
 *          (extra norm on every layer's input), 3 核心技术贡献 and
 *          4 实验结果分析 / 工程指标 (fp16 serving, graph replay, P99).
 *
 * Conventions shared by every call
 *   - All pointers are caller-owned DEVICE memory unless stated otherwise.
 *     The library never allocates or frees device memory; scratch space
 *     comes only through `workspace`, sized by mtgr_workspace_size().  (The
 *     graph handles below hold host-side runtime objects only.)
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and never synchronises.
 *   - `dt` is one mtgr_dtype for every floating tensor of a call; statistics
 *     (mean, rstd) are always fp32, weight gradients always fp32.
 *   - Jagged metadata: offsets int32 [B+1] with offsets[0] = 0, non-decreasing,
 *     offsets[B] = T; group_ids uint8 [T] with 0=U, 1=S, 2=R, 3=C,
 *     NON-DECREASING inside each user; timestamps int64 [T] (values of U and S
 *     tokens are not read).
 *   - Return value: MTGR_OK or a negative mtgr_status.  Argument errors are
 *     detected on the host before anything is launched, so no output is
 *     written; MTGR_ERR_HIP reports a failed launch.
 *   - Sizes: T <= INT32_MAX; every row stride (ld_*) at most 2^22 elements.
 *   - Validation mode (environment MTGR_VALIDATE=1 at the first call, or
 *     mtgr_set_validate(1)): every call that takes jagged metadata first runs
 *     a device check of it, which reads only offsets[0..B] and
 *     group_ids[0..T), synchronises the stream and returns
 *     MTGR_ERR_VALIDATION, with nothing else launched and no output written,
 *     when offsets[0] != 0, offsets decrease, offsets[B] != T, a group id is
 *     >= 4 (>= G for the stand-alone group norms), group ids decrease inside
 *     a user, or (backward calls with max_len > 0) a row is longer than
 *     max_len.  It is a debugging aid: it synchronises, so a call under
 *     stream capture returns MTGR_ERR_UNSUPPORTED, and validated calls of one
 *     process run one at a time.  Without it, metadata outside these rules
 *     gives undefined results; the kernels clamp offsets into [0, T] and
 *     group ids below G, so they do not read or write outside the stated
 *     buffers.
 *   - Calls that share a workspace must not overlap; calls with distinct
 *     workspaces may run concurrently on different streams.
 */
#ifndef MTGR_H_
#define MTGR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MTGR_F32 = 0,
  MTGR_BF16 = 1,
  MTGR_F16 = 2
} mtgr_dtype;

typedef enum {
  MTGR_OK = 0,
  MTGR_ERR_INVALID_ARG = -1,        /* null required pointer, bad size, bad stride */
  MTGR_ERR_UNSUPPORTED = -2,        /* dtype / head_dim / d_model not supported */
  MTGR_ERR_WORKSPACE_TOO_SMALL = -3,
  MTGR_ERR_HIP = -4,                /* a kernel launch failed */
  MTGR_ERR_VALIDATION = -5          /* MTGR_VALIDATE=1 found bad jagged metadata */
} mtgr_status;

/* Operation ids for mtgr_workspace_size(). */
typedef enum {
  MTGR_OP_PREP = 0,
  MTGR_OP_GLN_FWD = 1,
  MTGR_OP_GLN_BWD = 2,
  MTGR_OP_ATTN_FWD = 3,
  MTGR_OP_ATTN_BWD = 4,
  MTGR_OP_LAYER_FWD = 5,
  MTGR_OP_LAYER_BWD = 6,
  MTGR_OP_STACK_FWD = 7,
  MTGR_OP_STOCHASTIC_LENGTH = 8
} mtgr_op;

typedef void* mtgr_stream_t; /* hipStream_t */
typedef struct mtgr_graph_s* mtgr_graph; /* a captured launch sequence (see mtgr_stack_graph_create) */

/* Library version string, e.g. "mtgr-hstu 0.1.0 gfx950". Host memory, static. */
const char* mtgr_version(void);

/* Human-readable text of a status code. Host memory, static. */
const char* mtgr_status_string(int status);

/* Switches validation mode (see the conventions above) on (1) or off (0) for
 * the whole process; on < 0 only queries.  Returns the previous state. */
int mtgr_set_validate(int on);

/* Bytes of workspace `op` needs for these sizes (0 = none).  d = model width,
 * H = heads, max_len = an upper bound on every row's length (tokens), used
 * only by the backward ops in bf16/f16: with max_len > 0 their workspace also
 * holds the score gradients dS of the whole batch (H * 32 KB per 128 x 128
 * block of a row, bounded from B, T and max_len), which the dK/dV pass writes
 * and the dQ pass streams instead of recomputing the scores; with
 * max_len = 0 the dQ pass recomputes them and the workspace is small.  The
 * value only grows with B, T and max_len, so a workspace sized for the
 * largest batch serves every smaller one. */
size_t mtgr_workspace_size(int op, int32_t B, int64_t T, int32_t max_len, int32_t d, int32_t H, int dt);

/*
 * a1 - jagged segments.  For each user b writes seg[b*5 + 0..4] =
 * {start of U, start of S, start of R, start of C, end} (token indices into
 * the batch), the layout of the aggregated row [U, S, R, (C,I)_1..K]
 * ([blog] 4; [fr] 7.3.1).  Groups absent from a user give empty ranges.
 *   offsets, group_ids : device, see conventions
 *   seg                : device int32 [B, 5], written
 *   workspace          : MTGR_OP_PREP bytes (may be NULL if that is 0)
 */
int mtgr_jagged_prep(const int32_t* offsets, const uint8_t* group_ids, int32_t B, int64_t T,
                     int32_t* seg, void* workspace, size_t ws_bytes, mtgr_stream_t stream);

/* Candidate head weights (device, dtype dt): W1 [h, d], b1 [h] or NULL,
 * W2 [n_tasks, h], b2 [n_tasks] or NULL; d and h multiples of 8, 1 <= n_tasks
 * <= 4. */
typedef struct {
  const void* W1;
  const void* b1;
  const void* W2;
  const void* b2;
  int32_t d, h, n_tasks;
} mtgr_head_params;

/* fp32 head gradients, OVERWRITTEN; b1 / b2 non-NULL exactly when the
 * params have them. */
typedef struct {
  float* W1; /* [h, d] */
  float* b1; /* [h] */
  float* W2; /* [n_tasks, h] */
  float* b2; /* [n_tasks] */
} mtgr_head_grads;

/* Workspace bytes of the two head calls below. */
size_t mtgr_head_workspace_size(int32_t B, int64_t n_cand, int32_t d, int32_t h, int32_t n_tasks, int dt);

/*
 * Candidate head after the last layer ([blog] 5.4 and 7: the candidate
 * tokens' outputs pass through an MLP to logits; [pd] 它解决什么问题: a click
 * rate and a conversion rate for every exposed candidate).  Reading: for the
 * candidate (group C) tokens in batch order,
 *   logits = SiLU(x_c W1^T + b1) W2^T + b2      [n_cand, n_tasks] fp32.
 *   x       : [T, d] the last layer's output, row stride ld_x, dtype dt
 *   n_cand  : the number of group-C tokens in the batch (the caller's data
 *             loader knows it); a wrong count gives undefined logits but no
 *             access outside the stated buffers
 *   workspace : mtgr_head_workspace_size bytes
 */
int mtgr_candidate_head_fwd(const mtgr_head_params* p, const void* x, int64_t ld_x, const int32_t* offsets,
                            const uint8_t* group_ids, int32_t B, int64_t T, int64_t n_cand, float* logits, int dt,
                            void* workspace, size_t ws_bytes, mtgr_stream_t stream);

/*
 * Forward, discriminative loss and backward of the candidate head ([blog] 6
 * and [fr] 7.3.1: a ranking loss at candidate positions only, not next-token
 * prediction).  Reading: loss = (1 / n_cand) sum over candidates and tasks
 * of the binary cross-entropy of the task's logit against its label.
 *   labels : [n_cand, n_tasks] fp32 in [0, 1] (device)
 *   loss   : [1] fp32 (device), written
 *   logits : [n_cand, n_tasks] fp32 or NULL
 *   dx     : [T, d] dtype dt, row stride ld_dx: d loss / d x, zero on every
 *            non-candidate row (the upstream gradient of the last layer's
 *            backward); must not alias x
 *   grads  : head weight gradients, fp32, overwritten
 *   workspace : mtgr_head_workspace_size bytes
 */
int mtgr_candidate_head_loss(const mtgr_head_params* p, const void* x, int64_t ld_x, const int32_t* offsets,
                             const uint8_t* group_ids, int32_t B, int64_t T, int64_t n_cand, const float* labels,
                             float* loss, float* logits, void* dx, int64_t ld_dx, const mtgr_head_grads* grads,
                             int dt, void* workspace, size_t ws_bytes, mtgr_stream_t stream);


/*
 * Stochastic Length sampling in front of the training path, and the cut of
 * the shortened users to a token budget.  [pd] 计算量涨了 65 倍，训练成本怎么压住:
 * training replaces a long user sequence by a randomly drawn segment of it
 * (scoring keeps the full sequence); [blog] 11.3: batches are sized by token
 * count.  Reading: each user's history S keeps a contiguous window of
 * min(n_s, s_keep) tokens, in order, starting (within S) at
 *   min(floor(u_b * (n_s - s_keep + 1)), n_s - s_keep)
 * (u_b * (n_s - s_keep + 1) one float32 product; draws outside [0, 1) are
 * clamped to the first / last window); U, R and C tokens are kept, in order.
 *   offsets, group_ids, timestamps : the input batch (B users, T tokens)
 *   x          : [T, d] features, row stride ld_x elements, dtype dt; each
 *                row d * sizeof(dt) bytes, a multiple of 16
 *   u          : [B] float32 draws in [0, 1) (device), one per user
 *   s_keep     : >= 0, history tokens kept per user
 *   token_budget : >= 0
 * Written (device):
 *   offsets_out    : [B + 1] offsets of all B shortened users, input order
 *   fit_out        : int64 [2]: the number of leading shortened users whose
 *                    tokens fit token_budget (users of zero length included
 *                    while they fit), and those tokens
 *   group_ids_out, timestamps_out, x_out (row stride ld_out elements):
 *                    capacity T rows; only the rows of the fitting users,
 *                    [0, fit_out[1]), are written (pass token_budget >= T
 *                    to materialise every shortened user).
 *   The training batch is offsets_out[0 .. fit_out[0]] over those rows; the
 *   caller reads fit_out when it needs B and T on the host.
 *   workspace      : MTGR_OP_STOCHASTIC_LENGTH bytes for B and T
 */
int mtgr_stochastic_length(const int32_t* offsets, const uint8_t* group_ids, const int64_t* timestamps,
                           const void* x, int64_t ld_x, int32_t B, int64_t T, int32_t d, int dt,
                           const float* u, int32_t s_keep, int64_t token_budget, int32_t* offsets_out,
                           uint8_t* group_ids_out, int64_t* timestamps_out, void* x_out, int64_t ld_out,
                           int64_t* fit_out, void* workspace, size_t ws_bytes, mtgr_stream_t stream);

/*
 * a2/a5 - Group LayerNorm ([fr] 7.3.3; [pd] 模型怎么搭; [blog] 8).
 *   y_i = (x_i - mean_i) / sqrt(var_i + eps) * gamma[g(i)] + beta[g(i)],
 * statistics per token over its d features (biased variance), affine
 * parameters chosen by the token's group g(i) in [0, G).
 *   x, y          : [T, d] row-major, dtype dt; y may alias x
 *   gamma, beta   : [G, d], dtype dt
 *   group_ids     : uint8 [T], every value < G
 *   mean_out, rstd_out : fp32 [T] or NULL (the backward needs them)
 *   d % 8 == 0, 8 <= d <= 8192, 1 <= G <= 8.
 */
int mtgr_group_layernorm(const void* x, void* y, const void* gamma, const void* beta,
                         const uint8_t* group_ids, int64_t T, int32_t d, int32_t G, float eps,
                         int dt, float* mean_out, float* rstd_out, mtgr_stream_t stream);

/*
 * Backward of mtgr_group_layernorm.  With n = (x - mean) * rstd and
 * e = dy * gamma[g]:  dx = rstd * (e - mean(e) - n * mean(e * n)),
 * dgamma[c] = sum over tokens of group c of dy * n,  dbeta[c] = sum of dy.
 *   dy, x, dx     : [T, d] dtype dt (dx written; may alias dy)
 *   mean, rstd    : fp32 [T] from the forward
 *   dgamma, dbeta : fp32 [G, d], OVERWRITTEN (not accumulated)
 *   workspace     : MTGR_OP_GLN_BWD bytes
 */
int mtgr_group_layernorm_bwd(const void* dy, const void* x, const float* mean, const float* rstd,
                             const void* gamma, const uint8_t* group_ids, int64_t T, int32_t d,
                             int32_t G, int dt, void* dx, float* dgamma, float* dbeta,
                             void* workspace, size_t ws_bytes, mtgr_stream_t stream);

/*
 * a4 - jagged SiLU attention under the dynamic mask ([wiki] Métodos;
 * [pd] 模型怎么搭; mask: [fr] 7.3.4 rules 1-3, [blog] 9).  Per user b, head h:
 *   O_i = attn_scale * sum_j M_ij * SiLU(alpha * <q_i, k_j>) * v_j
 * with M_ij = 1 when key j is a U/S token; when j is real-time and i is a
 * real-time or candidate token with t_j < t_i, or i == j; when j is a
 * candidate and i == j.  No softmax.
 *   q, k, v : [T, H*dh] views with row stride ld_qkv elements (they may point
 *             into one fused [T, 4d] buffer); head h = columns h*dh..h*dh+dh-1
 *   o       : [T, H*dh] with row stride ld_o, written
 *   bf16/f16: dh in {32, 64, 128} (MFMA kernels); f32: dh in {16, 32, 64, 128}.
 *   workspace : MTGR_OP_ATTN_FWD bytes (sized with the call's d = H*dh and
 *               H).  For 16-bit batches too short to occupy the GPU (one
 *               serving request) the key range of every query tile is split
 *               and fp32 partial sums are kept in the workspace, so a short
 *               batch can need more workspace than a long one; the sum is
 *               taken in a fixed order (results are deterministic).
 */
int mtgr_hstu_attn_fwd(const void* q, const void* k, const void* v, int64_t ld_qkv, void* o,
                       int64_t ld_o, const int32_t* offsets, const uint8_t* group_ids,
                       const int64_t* timestamps, int32_t B, int64_t T, int32_t H, int32_t dh,
                       float alpha, float attn_scale, int dt, void* workspace, size_t ws_bytes,
                       mtgr_stream_t stream);

/*
 * mtgr_hstu_attn_fwd for callers that cannot allocate device memory or pass
 * a workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, layout and results as
 * mtgr_hstu_attn_fwd without `workspace` (every (query tile, head) runs as
 * one workgroup, so results of short batches can differ from
 * mtgr_hstu_attn_fwd's split key runs by fp32 rounding order).  Its tile
 * lists live in a static device array of MTGR_NOALLOC_SCRATCH_BYTES per GPU,
 * held until the process ends; the call allocates nothing.  The lists take
 * about 48 bytes per user plus 16 bytes per 128 tokens (plus under 2 KB of
 * alignment): every batch with B <= 16384 and T <= 4,194,304 fits; a batch
 * that does not returns MTGR_ERR_UNSUPPORTED before any launch.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (other streams, other threads) race and
 * must be serialised by the caller.
 */
#define MTGR_NOALLOC_SCRATCH_BYTES (2 * 1024 * 1024)
int mtgr_hstu_attn_fwd_noalloc(const void* q, const void* k, const void* v, int64_t ld_qkv, void* o,
                               int64_t ld_o, const int32_t* offsets, const uint8_t* group_ids,
                               const int64_t* timestamps, int32_t B, int64_t T, int32_t H, int32_t dh,
                               float alpha, float attn_scale, int dt, mtgr_stream_t stream);

/*
 * a7 - backward of mtgr_hstu_attn_fwd.  With S = alpha q k^T,
 * A = SiLU(S) * M:  dV = c A^T dO,  dA = c dO V^T,  dS = dA * M * SiLU'(S),
 * dQ = alpha dS K,  dK = alpha dS^T Q  (c = attn_scale).  The attention
 * weights are recomputed; nothing is saved by the forward.
 *   d_o          : [T, H*dh] with row stride ld_do
 *   dq, dk, dv   : [T, H*dh] with row stride ld_dqkv, OVERWRITTEN
 *   max_len      : 0, or an upper bound on every row's length (see
 *                  mtgr_workspace_size); in bf16/f16 with max_len > 0 the
 *                  workspace must hold MTGR_OP_ATTN_BWD bytes for that
 *                  max_len, else MTGR_ERR_WORKSPACE_TOO_SMALL.  A row longer
 *                  than max_len whose dS blocks then do not fit has its dq
 *                  recomputed from the scores instead (slower, same result;
 *                  never an out-of-range access).
 *   workspace    : MTGR_OP_ATTN_BWD bytes for the same B, T, max_len, H
 */
int mtgr_hstu_attn_bwd(const void* q, const void* k, const void* v, int64_t ld_qkv,
                       const void* d_o, int64_t ld_do, void* dq, void* dk, void* dv,
                       int64_t ld_dqkv, const int32_t* offsets, const uint8_t* group_ids,
                       const int64_t* timestamps, int32_t B, int64_t T, int32_t max_len, int32_t H,
                       int32_t dh, float alpha, float attn_scale, int dt, void* workspace,
                       size_t ws_bytes, mtgr_stream_t stream);

/* Weights of one layer, all device memory of dtype dt. */
typedef struct {
  const void* W_uqkv; /* [4d, d]: output feature major, output blocks U | Q | K | V */
  const void* b_uqkv; /* [4d] or NULL */
  const void* gamma1; /* [G, d] input Group LayerNorm */
  const void* beta1;  /* [G, d] */
  const void* gamma2; /* [G, d] Group LayerNorm of the attention output */
  const void* beta2;  /* [G, d] */
  const void* W_o;    /* [d, d]: output feature major */
  const void* b_o;    /* [d] or NULL */
  int32_t d;          /* model width, = H * dh */
  int32_t H;
  int32_t dh;
  int32_t G;          /* rows of gamma/beta, 4 <= G <= 8 (groups U, S, R, C use rows 0..3) */
  float eps;          /* Group LayerNorm epsilon (1e-5) */
  float alpha;        /* factor inside the SiLU of the attention scores (1) */
} mtgr_layer_params;

/* Activations the forward keeps for the backward (device, caller-owned). */
typedef struct {
  void* xhat;    /* [T, d]  output of the input Group LayerNorm */
  float* mean1;  /* [T] */
  float* rstd1;  /* [T] */
  void* zgrad;   /* [T, 4d] SiLU'(z), z = xhat W^T + b the pre-SiLU projection */
  void* uqkv;    /* [T, 4d] SiLU(z): U | Q | K | V */
  void* o;       /* [T, d]  attention output */
  float* mean2;  /* [T] */
  float* rstd2;  /* [T] */
  void* y;       /* [T, d]  GroupNorm(o) * U, input of the output projection */
} mtgr_layer_saved;

/* fp32 weight gradients, OVERWRITTEN by mtgr_hstu_layer_bwd.  db_uqkv and
 * db_o may be NULL (then not computed). */
typedef struct {
  float* W_uqkv; /* [4d, d] */
  float* b_uqkv; /* [4d] */
  float* gamma1; /* [G, d] */
  float* beta1;
  float* gamma2;
  float* beta2;
  float* W_o;    /* [d, d] */
  float* b_o;    /* [d] */
} mtgr_layer_grads;

/* Optional intermediate gradients of the backward (device, dtype dt). */
typedef struct {
  void* d_uqkv; /* [T, 4d] gradient w.r.t. SiLU(z), blocks dU | dQ | dK | dV; or NULL */
  void* d_o;    /* [T, d] gradient w.r.t. the attention output; or NULL */
} mtgr_layer_bwd_extras;

/*
 * a2..a6 - forward of one HSTU layer ([pd] 模型怎么搭; [wiki] Métodos;
 * per-layer input norm: paper-daily deep reading, 2 方法详解):
 *   xhat = GLN1(x); [U|Q|K|V] = SiLU(xhat W_uqkv^T + b_uqkv);
 *   O = attention(Q, K, V); Y = GLN2(O) * U; x_out = x + Y W_o^T + b_o.
 *   x_in, x_out : [T, d] dtype dt (x_out must not alias x_in)
 *   saved       : NULL for inference; else every member must be non-NULL
 *   attn_scale  : the attention normaliser (1 / longest row of the batch)
 *   d % 64 == 0 for bf16/f16.
 *   workspace   : MTGR_OP_LAYER_FWD bytes (smaller when saved != NULL is not
 *                 assumed: size it with the same call)
 */
int mtgr_hstu_layer_fwd(const mtgr_layer_params* p, const void* x_in, void* x_out,
                        const mtgr_layer_saved* saved, const int32_t* offsets,
                        const uint8_t* group_ids, const int64_t* timestamps, int32_t B, int64_t T,
                        float attn_scale, int dt, void* workspace, size_t ws_bytes,
                        mtgr_stream_t stream);

/*
 * Serving forward of an L-layer encoder stack: the L identical blocks of
 * [blog] 7 and [pd] 模型怎么搭, each exactly as mtgr_hstu_layer_fwd, with
 * the jagged tile lists built once for all layers.  The serving reading of
 * [pd] 计算量涨了 65 倍，训练成本怎么压住 (one pass per request, all
 * candidates together, fp16) is a batch with B = 1.
 *   layers      : HOST array of L >= 1 parameter sets (device pointers
 *                 inside), all with the same d, H and G; read during the
 *                 call only
 *   x_in        : [T, d] input, not modified; x_out : [T, d] output of the
 *                 last layer, must not alias x_in
 *   workspace   : MTGR_OP_STACK_FWD bytes (independent of L)
 *   fp32 results are bit-identical to L chained mtgr_hstu_layer_fwd calls.
 *   16-bit batches too short to occupy the GPU (one serving request) split
 *   each output projection over K into fp32 planes that the next layer's
 *   input norm adds together with bias and residual, so their results agree
 *   with chained calls up to the order of fp32 additions.
 */
int mtgr_hstu_stack_fwd(const mtgr_layer_params* layers, int32_t L, const void* x_in, void* x_out,
                        const int32_t* offsets, const uint8_t* group_ids, const int64_t* timestamps,
                        int32_t B, int64_t T, float attn_scale, int dt, void* workspace,
                        size_t ws_bytes, mtgr_stream_t stream);

/*
 * A stack forward captured once as a HIP graph and replayed with one launch
 * (the graph replay of the serving path: [pd] 计算量涨了 65 倍，训练成本怎么压住
 * and [dr] 4 工程指标 report its throughput and P99 gains).
 *   mtgr_stack_graph_create: records mtgr_hstu_stack_fwd with exactly these
 *     arguments on a private stream and instantiates the graph; no kernel
 *     runs.  Argument errors are those of mtgr_hstu_stack_fwd; B = 0 or
 *     T = 0 is MTGR_ERR_INVALID_ARG; so is a call while mtgr_profile_enable(1)
 *     is in effect.  Capture or instantiation failure: MTGR_ERR_HIP.  On
 *     error *out is NULL.
 *   The graph keeps every device pointer and the values B, T, L,
 *   attn_scale, dt and each layer's scalars (eps, alpha, shapes).  Between
 *   launches the caller may rewrite the CONTENTS of the buffers (a new
 *   request of the same B and T: x_in, offsets, group_ids, timestamps,
 *   weights) but must neither free nor move them while the handle lives.
 *   One graph per (B, T) shape: a serving loop keeps one per candidate count.
 *   mtgr_stack_graph_launch: enqueues one replay on `stream`; replays that
 *     share a workspace must not overlap.  NULL handle: MTGR_ERR_INVALID_ARG.
 *   mtgr_stack_graph_destroy: releases the handle (NULL is accepted); the
 *     caller ensures no launch of it is still pending.
 */
int mtgr_stack_graph_create(const mtgr_layer_params* layers, int32_t L, const void* x_in, void* x_out,
                            const int32_t* offsets, const uint8_t* group_ids, const int64_t* timestamps,
                            int32_t B, int64_t T, float attn_scale, int dt, void* workspace,
                            size_t ws_bytes, mtgr_graph* out);
int mtgr_stack_graph_launch(mtgr_graph g, mtgr_stream_t stream);
int mtgr_stack_graph_destroy(mtgr_graph g);

/*
 * A whole serving request as one graph: mtgr_hstu_stack_fwd and then
 * mtgr_candidate_head_fwd on its output, recorded once and replayed with
 * mtgr_stack_graph_launch (released with mtgr_stack_graph_destroy).  The
 * scores of [pd] 计算量涨了 65 倍 (one pass per request, all candidates) come
 * out as logits [n_cand, n_tasks] fp32.  Same rules as
 * mtgr_stack_graph_create; n_cand >= 1; head->d equals the layers' d;
 * workspace: MTGR_OP_STACK_FWD bytes, head_ws: mtgr_head_workspace_size
 * bytes (distinct buffers).
 */
int mtgr_serving_graph_create(const mtgr_layer_params* layers, int32_t L, const mtgr_head_params* head,
                              const void* x_in, void* x_out, float* logits, int64_t n_cand,
                              const int32_t* offsets, const uint8_t* group_ids, const int64_t* timestamps,
                              int32_t B, int64_t T, float attn_scale, int dt, void* workspace, size_t ws_bytes,
                              void* head_ws, size_t head_ws_bytes, mtgr_graph* out);

/*
 * a6..a2 backward (a8 plus the attention backward a7): from dx_out computes
 * dx_in (including the residual path) and every weight gradient.
 *   x_in        : the forward's input [T, d]
 *   saved       : filled by mtgr_hstu_layer_fwd with the same inputs
 *   dx_out      : [T, d] upstream gradient; dx_in : [T, d] written
 *   grads       : fp32 weight gradients, overwritten
 *   extras      : NULL or intermediate gradients to copy out
 *   max_len     : as for mtgr_hstu_attn_bwd
 *   workspace   : MTGR_OP_LAYER_BWD bytes for the same B, T, max_len, d, H
 */
int mtgr_hstu_layer_bwd(const mtgr_layer_params* p, const void* x_in, const mtgr_layer_saved* saved,
                        const void* dx_out, void* dx_in, const mtgr_layer_grads* grads,
                        const mtgr_layer_bwd_extras* extras, const int32_t* offsets,
                        const uint8_t* group_ids, const int64_t* timestamps, int32_t B, int64_t T,
                        int32_t max_len, float attn_scale, int dt, void* workspace, size_t ws_bytes,
                        mtgr_stream_t stream);

/*
 * Benchmark instrumentation (not part of the method).  When enabled, every
 * kernel step launched by the calls above is bracketed by HIP events recorded
 * on the stream it runs on.  mtgr_profile_enable(1) clears earlier records
 * and starts recording, (0) clears and stops.  mtgr_profile_summary waits for
 * the recorded events and writes, per distinct step name (host strings owned
 * by the library), the summed milliseconds and the number of launches;
 * returns the number of distinct names (which may exceed max_entries) or a
 * negative mtgr_status.  Not for concurrent use from several threads.
 */
int mtgr_profile_enable(int on);
int mtgr_profile_summary(int max_entries, const char** names, double* total_ms, int32_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* MTGR_H_ */
