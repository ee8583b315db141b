// C ABI of the library: argument validation, workspace carving and the
// launch sequence of each entry point (declared in include/mtgr.h).
#include <stdlib.h>
#include <string.h>

#include "kernels.h"

using namespace mtgr;

namespace {

constexpr int kMaxG = 8;
// Largest row stride (elements) of any row-major operand: tile offsets
// inside a kernel are 32-bit byte offsets over at most 256 rows.
constexpr int64_t kMaxLd = (int64_t)1 << 22;
// The layer's token groups U, S, R, C: its group norms need G >= 4 rows of
// gamma / beta.
constexpr int kLayerGroups = 4;

inline hipStream_t S(mtgr_stream_t s) { return (hipStream_t)s; }

inline size_t elt(int dt) { return dt == MTGR_F32 ? 4 : 2; }

inline bool dt_ok(int dt) { return dt == MTGR_F32 || dt == MTGR_BF16 || dt == MTGR_F16; }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Row strides and base pointers must allow 16-byte vector access.
inline bool vec_ok(const void* p, int64_t ld, int dt) {
  if (!p) return true;
  return aligned16(p) && ld <= kMaxLd && (ld * (int64_t)elt(dt)) % 16 == 0;
}

bool attn_shape_ok(int dt, int dh) {
  if (dt == MTGR_F32) return dh == 16 || dh == 32 || dh == 64 || dh == 128;
  return dh == 32 || dh == 64 || dh == 128;
}

size_t attn_ws(int B, int64_t T) { return prep_workspace_bytes(B, T); }

// Carve a workspace sequentially.
struct Carver {
  char* p;
  size_t left;
  bool ok = true;
  void* take(size_t n) {
    n = align_up(n, 256);
    if (n > left) { ok = false; return nullptr; }
    void* r = p;
    p += n;
    left -= n;
    return r;
  }
};

// Forward attention: the tile lists plus, for short batches, the fp32
// partial sums of the key runs.
size_t attn_fwd_ws(int B, int64_t T, int H, int dh, int dt) {
  return align_up(attn_ws(B, T), 256) + align_up(attn_fwd_part_bytes(dt, B, T, H, dh), 256);
}

size_t layer_fwd_ws(int B, int64_t T, int d, int H, int dt) {
  const size_t e = elt(dt);
  size_t n = attn_fwd_ws(B, T, H, H > 0 ? d / H : 0, dt);
  n += align_up((size_t)T * d * e, 256);       // xhat, then y
  n += align_up((size_t)T * 4 * d * e, 256);   // uqkv
  n += align_up((size_t)T * d * e, 256);       // o
  return n;
}

// Split-K planes of the stack's output projections: used for 16-bit batches
// whose projection has too few tiles to occupy the GPU (0: not split).
int stack_out_planes(int64_t T, int d, int dt) {
  if (dt == MTGR_F32 || T <= 0) return 0;
  const int s = gemm_plane_splits((int)T, d, d);
  return s > 1 ? s : 0;
}

// fp32 partial planes of a stack forward: the attention's key runs and the
// output projections' split-K planes share one region.
size_t stack_part_bytes(int B, int64_t T, int d, int H, int dt) {
  const size_t a = attn_fwd_part_bytes(dt, B, T, H, H > 0 ? d / H : 0);
  const size_t g = (size_t)stack_out_planes(T, d, dt) * (size_t)T * d * sizeof(float);
  return a > g ? a : g;
}

// Tile lists, partial planes, the layer intermediates and one hidden-state
// buffer between layers.
size_t stack_fwd_ws(int B, int64_t T, int d, int H, int dt) {
  const size_t e = elt(dt);
  size_t n = align_up(attn_ws(B, T), 256);
  n += align_up(stack_part_bytes(B, T, d, H, dt), 256);
  n += align_up((size_t)T * d * e, 256);       // xhat, then y
  n += align_up((size_t)T * 4 * d * e, 256);   // uqkv
  n += align_up((size_t)T * d * e, 256);       // o
  n += align_up((size_t)T * d * e, 256);       // h
  return n;
}

// dS storage of the backward (bf16/f16 with a declared row bound only).
size_t ds_ws(int B, int64_t T, int max_len, int H, int dt) {
  return dt == MTGR_F32 ? 0 : attn_ds_bytes(B, T, max_len, H);
}

size_t attn_bwd_ws(int B, int64_t T, int max_len, int H, int dt) {
  return align_up(attn_ws(B, T), 256) + ds_ws(B, T, max_len, H, dt);
}

size_t layer_bwd_ws(int B, int64_t T, int max_len, int d, int H, int dt) {
  const size_t e = elt(dt);
  size_t n = align_up(attn_ws(B, T), 256);
  n += align_up((size_t)T * d * e, 256);       // dy, then dxhat
  n += align_up((size_t)T * d * e, 256);       // d_o
  n += align_up((size_t)T * 4 * d * e, 256);   // dz
  size_t r = gln_bwd_workspace_bytes(T, d, kMaxG);
  size_t c = colsum_workspace_bytes(T, 4 * d);
  n += align_up(r > c ? r : c, 256);
  n += ds_ws(B, T, max_len, H, dt);
  return n;
}

// Point the attention backward at its dS buffer when a row bound was given.
void set_ds(AttnArgs& a, void* buf, int max_len, int dt) {
  if (dt == MTGR_F32 || max_len <= 0 || !buf) return;
  a.ds = buf;
  a.ds_cap = (int64_t)(ds_ws(a.B, a.T, max_len, a.H, dt) / ((size_t)a.H * DS_TILE_BYTES));
}

bool jagged_ok(const int32_t* offsets, const uint8_t* g, const int64_t* ts, int32_t B, int64_t T) {
  if (B < 0 || T < 0 || T > INT32_MAX) return false;
  if (B > 0 && !offsets) return false;
  if (T > 0 && (!g || !ts)) return false;
  return true;
}

// Split-K factor of a weight-gradient product: about one 256x256 tile job per
// compute unit (fewer partial sums to add atomically, measured faster than two
// jobs per unit), each split at least 1024 deep.
int splits_for(int M, int N, int K) {
  const int tiles = ((M + 255) / 256) * ((N + 255) / 256);
  int s = (256 + tiles - 1) / tiles;
  const int maxs = K / 1024 > 0 ? K / 1024 : 1;
  if (s > maxs) s = maxs;
  return s < 1 ? 1 : s;
}

}  // namespace

extern "C" {

const char* mtgr_version(void) { return "mtgr-hstu 0.2.0 gfx950"; }

int mtgr_set_validate(int on) {
  const int prev = validation_enabled() ? 1 : 0;
  if (on >= 0) set_validation(on);
  return prev;
}

const char* mtgr_status_string(int status) {
  switch (status) {
    case MTGR_OK: return "ok";
    case MTGR_ERR_INVALID_ARG: return "invalid argument";
    case MTGR_ERR_UNSUPPORTED: return "unsupported dtype or shape";
    case MTGR_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MTGR_ERR_HIP: return "HIP launch error";
    case MTGR_ERR_VALIDATION: return "jagged metadata failed validation";
    default: return "unknown status";
  }
}

size_t mtgr_workspace_size(int op, int32_t B, int64_t T, int32_t max_len, int32_t d, int32_t H, int dt) {
  if (B < 0 || T < 0 || d < 0 || max_len < 0 || H < 0 || !dt_ok(dt)) return 0;
  switch (op) {
    case MTGR_OP_PREP: return 0;
    case MTGR_OP_GLN_FWD: return 0;
    case MTGR_OP_GLN_BWD: return gln_bwd_workspace_bytes(T, d, kMaxG);
    case MTGR_OP_ATTN_FWD: return H > 0 ? attn_fwd_ws(B, T, H, d / H, dt) : attn_ws(B, T);
    case MTGR_OP_ATTN_BWD: return attn_bwd_ws(B, T, max_len, H, dt);
    case MTGR_OP_LAYER_FWD: return layer_fwd_ws(B, T, d, H, dt);
    case MTGR_OP_LAYER_BWD: return layer_bwd_ws(B, T, max_len, d, H, dt);
    case MTGR_OP_STACK_FWD: return stack_fwd_ws(B, T, d, H, dt);
    case MTGR_OP_STOCHASTIC_LENGTH: return sl_workspace_bytes(B, T);
    default: return 0;
  }
}

int mtgr_jagged_prep(const int32_t* offsets, const uint8_t* group_ids, int32_t B, int64_t T,
                     int32_t* seg, void* workspace, size_t ws_bytes, mtgr_stream_t stream) {
  (void)workspace;
  (void)ws_bytes;
  if (B < 0 || T < 0) return MTGR_ERR_INVALID_ARG;
  if (B == 0) return MTGR_OK;
  if (!offsets || !seg || (T > 0 && !group_ids)) return MTGR_ERR_INVALID_ARG;
  const int vr = validate_jagged(offsets, group_ids, B, T, kLayerGroups, true, 0, S(stream));
  if (vr) return vr;
  return launch_seg_only(offsets, group_ids, B, T, seg, S(stream));
}

int mtgr_stochastic_length(const int32_t* offsets, const uint8_t* group_ids, const int64_t* timestamps,
                           const void* x, int64_t ld_x, int32_t B, int64_t T, int32_t d, int dt, const float* u,
                           int32_t s_keep, int64_t token_budget, int32_t* offsets_out, uint8_t* group_ids_out,
                           int64_t* timestamps_out, void* x_out, int64_t ld_out, int64_t* fit_out, void* workspace,
                           size_t ws_bytes, mtgr_stream_t stream) {
  if (!dt_ok(dt)) return MTGR_ERR_UNSUPPORTED;
  if (!jagged_ok(offsets, group_ids, timestamps, B, T) || d < 1 || s_keep < 0 || token_budget < 0)
    return MTGR_ERR_INVALID_ARG;
  if (!offsets_out || !fit_out) return MTGR_ERR_INVALID_ARG;
  if (B > 0 && !u) return MTGR_ERR_INVALID_ARG;
  if (T > 0 && (!x || !x_out || !group_ids_out || !timestamps_out)) return MTGR_ERR_INVALID_ARG;
  const int64_t row_bytes = (int64_t)d * elt(dt);
  if (ld_x < d || ld_out < d || row_bytes % 16) return MTGR_ERR_INVALID_ARG;
  if (!vec_ok(x, ld_x, dt) || !vec_ok(x_out, ld_out, dt)) return MTGR_ERR_INVALID_ARG;
  if (ws_bytes < sl_workspace_bytes(B, T) || !workspace) return MTGR_ERR_WORKSPACE_TOO_SMALL;
  const int vr = validate_jagged(offsets, group_ids, B, T, kLayerGroups, true, 0, S(stream));
  if (vr) return vr;
  // an empty batch still gets its offsets and budget cut written
  return launch_stochastic_length(offsets, group_ids, timestamps, x, ld_x * (int64_t)elt(dt), (int)row_bytes, B, T, u,
                                  s_keep, token_budget, offsets_out, group_ids_out, timestamps_out, x_out,
                                  ld_out * (int64_t)elt(dt), fit_out, workspace, S(stream));
}

}  // extern "C"

int mtgr::head_validate(const mtgr_head_params* p, const void* x, int64_t ld_x, const int32_t* offsets,
                        const uint8_t* group_ids, int32_t B, int64_t T, int64_t n_cand, int dt) {
  if (!p) return MTGR_ERR_INVALID_ARG;
  if (!dt_ok(dt)) return MTGR_ERR_UNSUPPORTED;
  if (p->n_tasks < 1 || p->n_tasks > 4) return MTGR_ERR_UNSUPPORTED;
  if (p->d < 8 || p->h < 8 || p->d % 8 || p->h % 8) return MTGR_ERR_UNSUPPORTED;
  if (!p->W1 || !p->W2) return MTGR_ERR_INVALID_ARG;
  if (!vec_ok(p->W1, p->d, dt) || !aligned16(p->W2) || (p->b1 && !aligned16(p->b1)) || (p->b2 && !aligned16(p->b2)))
    return MTGR_ERR_INVALID_ARG;
  if (B < 0 || T < 0 || n_cand < 0 || n_cand > T || T > INT32_MAX) return MTGR_ERR_INVALID_ARG;
  if (B > 0 && (!offsets || !group_ids)) return MTGR_ERR_INVALID_ARG;
  if (T > 0 && !x) return MTGR_ERR_INVALID_ARG;
  if (ld_x < p->d || !vec_ok(x, ld_x, dt)) return MTGR_ERR_INVALID_ARG;
  return MTGR_OK;
}

extern "C" {

size_t mtgr_head_workspace_size(int32_t B, int64_t n_cand, int32_t d, int32_t h, int32_t n_tasks, int dt) {
  if (B < 0 || n_cand < 0 || d < 1 || h < 1 || n_tasks < 1 || !dt_ok(dt)) return 0;
  return head_workspace_bytes(B, n_cand, d, h, n_tasks, dt);
}

int mtgr_candidate_head_fwd(const mtgr_head_params* p, const void* x, int64_t ld_x, const int32_t* offsets,
                            const uint8_t* group_ids, int32_t B, int64_t T, int64_t n_cand, float* logits, int dt,
                            void* workspace, size_t ws_bytes, mtgr_stream_t stream) {
  return head_fwd_run(p, x, ld_x, offsets, group_ids, B, T, n_cand, logits, dt, workspace, ws_bytes,
                      S(stream), true);
}

}  // extern "C"

int mtgr::head_fwd_run(const mtgr_head_params* p, const void* x, int64_t ld_x, const int32_t* offsets,
                       const uint8_t* group_ids, int32_t B, int64_t T, int64_t n_cand, float* logits, int dt,
                       void* workspace, size_t ws_bytes, hipStream_t stream, bool check_meta) {
  int r = head_validate(p, x, ld_x, offsets, group_ids, B, T, n_cand, dt);
  if (r) return r;
  if (n_cand > 0 && !logits) return MTGR_ERR_INVALID_ARG;
  if (ws_bytes < head_workspace_bytes(B, n_cand, p->d, p->h, p->n_tasks, dt) || !workspace)
    return MTGR_ERR_WORKSPACE_TOO_SMALL;
  if (check_meta) {
    r = validate_jagged(offsets, group_ids, B, T, kLayerGroups, true, 0, stream);
    if (r) return r;
  }
  if (n_cand == 0 || B == 0) return MTGR_OK;
  HeadArgs a = {};
  a.offsets = offsets; a.group_ids = group_ids; a.B = B; a.T = T; a.n_cand = n_cand;
  a.x = x; a.ldx = ld_x; a.d = p->d; a.h = p->h; a.nt = p->n_tasks;
  a.W1 = p->W1; a.b1 = p->b1; a.W2 = p->W2; a.b2 = p->b2;
  a.logits = logits;
  return launch_head(dt, a, workspace, stream);
}

extern "C" {

int mtgr_candidate_head_loss(const mtgr_head_params* p, const void* x, int64_t ld_x, const int32_t* offsets,
                             const uint8_t* group_ids, int32_t B, int64_t T, int64_t n_cand, const float* labels,
                             float* loss, float* logits, void* dx, int64_t ld_dx, const mtgr_head_grads* grads, int dt,
                             void* workspace, size_t ws_bytes, mtgr_stream_t stream) {
  int r = head_validate(p, x, ld_x, offsets, group_ids, B, T, n_cand, dt);
  if (r) return r;
  if (!loss || !grads || !grads->W1 || !grads->W2) return MTGR_ERR_INVALID_ARG;
  if ((p->b1 != nullptr) != (grads->b1 != nullptr) || (p->b2 != nullptr) != (grads->b2 != nullptr))
    return MTGR_ERR_INVALID_ARG;
  if (n_cand > 0 && !labels) return MTGR_ERR_INVALID_ARG;
  if (T > 0 && (!dx || ld_dx < p->d || !vec_ok(dx, ld_dx, dt))) return MTGR_ERR_INVALID_ARG;
  if (dx && dx == x) return MTGR_ERR_INVALID_ARG;
  if (ws_bytes < head_workspace_bytes(B, n_cand, p->d, p->h, p->n_tasks, dt) || !workspace)
    return MTGR_ERR_WORKSPACE_TOO_SMALL;
  r = validate_jagged(offsets, group_ids, B, T, kLayerGroups, true, 0, S(stream));
  if (r) return r;
  HeadArgs a = {};
  a.offsets = offsets; a.group_ids = group_ids; a.B = B; a.T = T; a.n_cand = B > 0 ? n_cand : 0;
  a.x = x; a.ldx = ld_x; a.d = p->d; a.h = p->h; a.nt = p->n_tasks;
  a.W1 = p->W1; a.b1 = p->b1; a.W2 = p->W2; a.b2 = p->b2;
  a.train = true; a.labels = labels; a.logits = logits; a.loss = loss;
  a.dx = dx; a.lddx = ld_dx;
  a.dW1 = grads->W1; a.db1 = grads->b1; a.dW2 = grads->W2; a.db2 = grads->b2;
  return launch_head(dt, a, workspace, S(stream));
}

int mtgr_group_layernorm(const void* x, void* y, const void* gamma, const void* beta,
                         const uint8_t* group_ids, int64_t T, int32_t d, int32_t G, float eps, int dt,
                         float* mean_out, float* rstd_out, mtgr_stream_t stream) {
  if (!dt_ok(dt)) return MTGR_ERR_UNSUPPORTED;
  if (T < 0 || d < 8 || d > 8192 || d % 8 != 0 || G < 1 || G > kMaxG) return MTGR_ERR_INVALID_ARG;
  if (T == 0) return MTGR_OK;
  if (!x || !y || !gamma || !beta || !group_ids) return MTGR_ERR_INVALID_ARG;
  if ((mean_out == nullptr) != (rstd_out == nullptr)) return MTGR_ERR_INVALID_ARG;
  if (!vec_ok(x, d, dt) || !vec_ok(y, d, dt) || !vec_ok(gamma, d, dt) || !vec_ok(beta, d, dt))
    return MTGR_ERR_INVALID_ARG;
  const int vr = validate_jagged(nullptr, group_ids, 0, T, G, false, 0, S(stream));
  if (vr) return vr;
  return launch_gln_fwd(dt, x, d, y, d, gamma, beta, group_ids, T, d, G, eps, mean_out, rstd_out, nullptr, 0,
                        S(stream));
}

int mtgr_group_layernorm_bwd(const void* dy, const void* x, const float* mean, const float* rstd,
                             const void* gamma, const uint8_t* group_ids, int64_t T, int32_t d, int32_t G,
                             int dt, void* dx, float* dgamma, float* dbeta, void* workspace,
                             size_t ws_bytes, mtgr_stream_t stream) {
  if (!dt_ok(dt)) return MTGR_ERR_UNSUPPORTED;
  if (T < 0 || d < 8 || d > 8192 || d % 8 != 0 || G < 1 || G > kMaxG || G * d > 8192)
    return MTGR_ERR_INVALID_ARG;
  if (!dgamma || !dbeta || !gamma) return MTGR_ERR_INVALID_ARG;
  if (T > 0 && (!dy || !x || !mean || !rstd || !group_ids || !dx)) return MTGR_ERR_INVALID_ARG;
  if (!vec_ok(dy, d, dt) || !vec_ok(x, d, dt) || !vec_ok(dx, d, dt) || !vec_ok(gamma, d, dt))
    return MTGR_ERR_INVALID_ARG;
  if (ws_bytes < gln_bwd_workspace_bytes(T, d, G) || (T > 0 && !workspace))
    return MTGR_ERR_WORKSPACE_TOO_SMALL;
  const int vr = validate_jagged(nullptr, group_ids, 0, T, G, false, 0, S(stream));
  if (vr) return vr;
  return launch_gln_bwd(dt, dy, d, x, d, mean, rstd, gamma, nullptr, group_ids, T, d, G, dx, d, nullptr, 0,
                        nullptr, 0, nullptr, 0, nullptr, 0, dgamma, dbeta, workspace, S(stream));
}

static int attn_arg_checks(const void* q, const void* k, const void* v, int64_t ldqkv, const int32_t* offsets,
                           const uint8_t* g, const int64_t* ts, int32_t B, int64_t T, int32_t H, int32_t dh,
                           int dt) {
  if (!dt_ok(dt)) return MTGR_ERR_UNSUPPORTED;
  if (!attn_shape_ok(dt, dh)) return MTGR_ERR_UNSUPPORTED;
  if (H < 1 || !jagged_ok(offsets, g, ts, B, T)) return MTGR_ERR_INVALID_ARG;
  if (ldqkv < (int64_t)H * dh) return MTGR_ERR_INVALID_ARG;
  if (T > 0 && (!q || !k || !v)) return MTGR_ERR_INVALID_ARG;
  if (!vec_ok(q, ldqkv, dt) || !vec_ok(k, ldqkv, dt) || !vec_ok(v, ldqkv, dt)) return MTGR_ERR_INVALID_ARG;
  return MTGR_OK;
}

static int attn_common_checks(const void* q, const void* k, const void* v, int64_t ldqkv,
                              const int32_t* offsets, const uint8_t* g, const int64_t* ts, int32_t B,
                              int64_t T, int32_t H, int32_t dh, int dt, void* workspace, size_t ws_bytes) {
  const int r = attn_arg_checks(q, k, v, ldqkv, offsets, g, ts, B, T, H, dh, dt);
  if (r) return r;
  if (ws_bytes < attn_ws(B, T) || (B > 0 && !workspace)) return MTGR_ERR_WORKSPACE_TOO_SMALL;
  return MTGR_OK;
}

}  // extern "C"

int mtgr::attn_fwd_arg_checks(const void* q, const void* k, const void* v, int64_t ld_qkv, const void* o,
                              int64_t ld_o, const int32_t* offsets, const uint8_t* group_ids,
                              const int64_t* timestamps, int32_t B, int64_t T, int32_t H, int32_t dh, int dt) {
  // no workspace here: the variant without one keeps its lists elsewhere
  const int r = attn_arg_checks(q, k, v, ld_qkv, offsets, group_ids, timestamps, B, T, H, dh, dt);
  if (r) return r;
  if (ld_o < (int64_t)H * dh || (T > 0 && !o) || !vec_ok(o, ld_o, dt)) return MTGR_ERR_INVALID_ARG;
  return MTGR_OK;
}

extern "C" {

int mtgr_hstu_attn_fwd(const void* q, const void* k, const void* v, int64_t ld_qkv, void* o, int64_t ld_o,
                       const int32_t* offsets, const uint8_t* group_ids, const int64_t* timestamps,
                       int32_t B, int64_t T, int32_t H, int32_t dh, float alpha, float attn_scale, int dt,
                       void* workspace, size_t ws_bytes, mtgr_stream_t stream) {
  int r = attn_common_checks(q, k, v, ld_qkv, offsets, group_ids, timestamps, B, T, H, dh, dt, workspace,
                             ws_bytes);
  if (r) return r;
  if (ld_o < (int64_t)H * dh || (T > 0 && !o) || !vec_ok(o, ld_o, dt)) return MTGR_ERR_INVALID_ARG;
  if (ws_bytes < attn_fwd_ws(B, T, H, dh, dt)) return MTGR_ERR_WORKSPACE_TOO_SMALL;
  if (B == 0 || T == 0) return MTGR_OK;
  r = validate_jagged(offsets, group_ids, B, T, kLayerGroups, true, 0, S(stream));
  if (r) return r;
  Carver cv{(char*)workspace, ws_bytes};
  void* ws_prep = cv.take(attn_ws(B, T));
  const size_t pb = attn_fwd_part_bytes(dt, B, T, H, dh);
  void* ws_part = pb ? cv.take(pb) : nullptr;
  if (!cv.ok) return MTGR_ERR_WORKSPACE_TOO_SMALL;
  PrepView pv;
  r = launch_prep(offsets, group_ids, B, T, ws_prep, S(stream), &pv);
  if (r) return r;
  AttnArgs a = {};
  a.q = q; a.k = k; a.v = v; a.ldqkv = ld_qkv;
  a.o = o; a.ldo = ld_o;
  a.ts = timestamps; a.B = B; a.T = T; a.H = H; a.dh = dh; a.alpha = alpha; a.scale = attn_scale;
  a.part = (float*)ws_part; a.nsplit = attn_fwd_splits(dt, B, T, H);
  r = launch_attn_fwd(dt, a, pv, S(stream));
  if (r || !ws_part || a.nsplit < 2) return r;
  PartialRows pr = {};
  pr.part = (const float*)ws_part; pr.n = a.nsplit; pr.plane = T * H * dh; pr.ldp = (int64_t)H * dh;
  pr.xs = o; pr.ldxs = ld_o;
  ProfScope ps("attn_fwd_sum", S(stream));
  return launch_partial_reduce(dt, pr, T, H * dh, S(stream));
}

int mtgr_hstu_attn_bwd(const void* q, const void* k, const void* v, int64_t ld_qkv, const void* d_o,
                       int64_t ld_do, void* dq, void* dk, void* dv, int64_t ld_dqkv, const int32_t* offsets,
                       const uint8_t* group_ids, const int64_t* timestamps, int32_t B, int64_t T,
                       int32_t max_len, int32_t H, int32_t dh, float alpha, float attn_scale, int dt,
                       void* workspace, size_t ws_bytes, mtgr_stream_t stream) {
  int r = attn_common_checks(q, k, v, ld_qkv, offsets, group_ids, timestamps, B, T, H, dh, dt, workspace,
                             ws_bytes);
  if (r) return r;
  if (max_len < 0) return MTGR_ERR_INVALID_ARG;
  if (ws_bytes < attn_bwd_ws(B, T, max_len, H, dt)) return MTGR_ERR_WORKSPACE_TOO_SMALL;
  if (ld_do < (int64_t)H * dh || ld_dqkv < (int64_t)H * dh) return MTGR_ERR_INVALID_ARG;
  if (T > 0 && (!d_o || !dq || !dk || !dv)) return MTGR_ERR_INVALID_ARG;
  if (!vec_ok(d_o, ld_do, dt) || !vec_ok(dq, ld_dqkv, dt) || !vec_ok(dk, ld_dqkv, dt) ||
      !vec_ok(dv, ld_dqkv, dt))
    return MTGR_ERR_INVALID_ARG;
  if (B == 0 || T == 0) return MTGR_OK;
  r = validate_jagged(offsets, group_ids, B, T, kLayerGroups, true, max_len, S(stream));
  if (r) return r;
  PrepView pv;
  r = launch_prep(offsets, group_ids, B, T, workspace, S(stream), &pv);
  if (r) return r;
  AttnArgs a = {};
  a.q = q; a.k = k; a.v = v; a.ldqkv = ld_qkv;
  a.d_o = d_o; a.lddo = ld_do;
  a.dq = dq; a.dk = dk; a.dv = dv; a.lddqkv = ld_dqkv;
  a.ts = timestamps; a.B = B; a.T = T; a.H = H; a.dh = dh; a.alpha = alpha; a.scale = attn_scale;
  set_ds(a, (char*)workspace + align_up(attn_ws(B, T), 256), max_len, dt);
  return launch_attn_bwd(dt, a, pv, S(stream));
}

static int layer_param_checks(const mtgr_layer_params* p, int dt) {
  if (!p) return MTGR_ERR_INVALID_ARG;
  if (!dt_ok(dt)) return MTGR_ERR_UNSUPPORTED;
  if (p->H < 1 || p->dh < 1 || p->d != p->H * p->dh || p->G < 1 || p->G > kMaxG) return MTGR_ERR_INVALID_ARG;
  // group ids of a layer run over U, S, R, C: fewer parameter rows cannot
  // serve them
  if (p->G < kLayerGroups) return MTGR_ERR_UNSUPPORTED;
  if (!attn_shape_ok(dt, p->dh)) return MTGR_ERR_UNSUPPORTED;
  if (p->d % 8 != 0 || p->d > 8192 || p->G * p->d > 8192) return MTGR_ERR_UNSUPPORTED;
  if (dt != MTGR_F32 && p->d % 64 != 0) return MTGR_ERR_UNSUPPORTED;
  if (!p->W_uqkv || !p->gamma1 || !p->beta1 || !p->gamma2 || !p->beta2 || !p->W_o) return MTGR_ERR_INVALID_ARG;
  if (!vec_ok(p->gamma1, p->d, dt) || !vec_ok(p->beta1, p->d, dt) || !vec_ok(p->gamma2, p->d, dt) ||
      !vec_ok(p->beta2, p->d, dt) || !vec_ok(p->W_uqkv, p->d, dt) || !vec_ok(p->W_o, p->d, dt) ||
      (p->b_uqkv && !aligned16(p->b_uqkv)) || (p->b_o && !aligned16(p->b_o)))
    return MTGR_ERR_INVALID_ARG;
  return MTGR_OK;
}

// a2..a6 of one layer on a prepared batch (the tile lists in pv); xhat,
// uqkv and o are the layer's intermediates, y may alias xhat.  part: fp32
// partial planes for the split-key attention of short batches (the group
// norm of a5 adds them) and, with out_planes > 0, for the output projection.
// in_planes: when set, the layer input is the sum it describes (the previous
// layer's projection planes plus bias and residual, stored to in_planes->xs
// on the way) instead of x_in.  With out_planes > 0 the projection writes
// out_planes fp32 planes of y W_o^T into part and x_out is not written: the
// next step adds bias and residual.
static int layer_fwd_body(const mtgr_layer_params* p, const void* x_in, void* x_out, const mtgr_layer_saved* saved,
                          const uint8_t* group_ids, const int64_t* timestamps, int32_t B, int64_t T,
                          float attn_scale, int dt, const PrepView& pv, void* part, void* xhat, void* uqkv, void* o,
                          void* y, const PartialRows* in_planes, int out_planes, hipStream_t st) {
  const int d = p->d;
  const size_t e = elt(dt);
  int r;
  // a2: input group norm
  {
    ProfScope ps("gln1_fwd", st);
    if (in_planes)
      r = launch_gln_fwd_part(dt, *in_planes, xhat, d, p->gamma1, p->beta1, group_ids, T, d, p->G, p->eps,
                              saved ? saved->mean1 : nullptr, saved ? saved->rstd1 : nullptr, nullptr, 0, st);
    else
      r = launch_gln_fwd(dt, x_in, d, xhat, d, p->gamma1, p->beta1, group_ids, T, d, p->G, p->eps,
                         saved ? saved->mean1 : nullptr, saved ? saved->rstd1 : nullptr, nullptr, 0, st);
  }
  if (r) return r;
  // a3: [U|Q|K|V] = SiLU(xhat W^T + b)
  GemmEpiArgs ep = {};
  ep.kind = EPI_BIAS_SILU;
  ep.C = uqkv; ep.ldc = 4 * d; ep.bias = p->b_uqkv;
  // the backward needs only SiLU'(z), which the epilogue forms from the
  // sigmoid it computes anyway
  ep.Z = saved ? saved->zgrad : nullptr; ep.ldz = 4 * d; ep.zgrad = 1;
  {
    ProfScope ps("gemm_uqkv_silu", st);
    r = launch_gemm(dt, xhat, d, true, p->W_uqkv, d, true, (int)T, 4 * d, d, ep, 1, st);
  }
  if (r) return r;
  // a4: attention
  const char* base = (const char*)uqkv;
  AttnArgs a = {};
  a.q = base + (size_t)d * e; a.k = base + (size_t)2 * d * e; a.v = base + (size_t)3 * d * e;
  a.ldqkv = 4 * d; a.o = o; a.ldo = d;
  a.ts = timestamps; a.B = B; a.T = T; a.H = p->H; a.dh = p->dh; a.alpha = p->alpha; a.scale = attn_scale;
  a.part = (float*)part; a.nsplit = attn_fwd_splits(dt, B, T, p->H);
  const bool attn_planes = part && a.nsplit > 1;
  r = launch_attn_fwd(dt, a, pv, st);
  if (r) return r;
  // a5: y = GLN2(o) * U, o summed from the key-run planes when split (and
  // stored only when it is kept for the backward)
  {
    ProfScope ps("gln2_gate_fwd", st);
    if (attn_planes) {
      PartialRows pr = {};
      pr.part = (const float*)part; pr.n = a.nsplit; pr.plane = T * d; pr.ldp = d;
      pr.xs = saved ? saved->o : nullptr; pr.ldxs = d;
      r = launch_gln_fwd_part(dt, pr, y, d, p->gamma2, p->beta2, group_ids, T, d, p->G, p->eps,
                              saved ? saved->mean2 : nullptr, saved ? saved->rstd2 : nullptr, uqkv, 4 * d, st);
    } else {
      r = launch_gln_fwd(dt, o, d, y, d, p->gamma2, p->beta2, group_ids, T, d, p->G, p->eps,
                         saved ? saved->mean2 : nullptr, saved ? saved->rstd2 : nullptr, uqkv, 4 * d, st);
    }
  }
  if (r) return r;
  // a6: x_out = x + y W_o^T + b_o
  GemmEpiArgs eo = {};
  ProfScope ps("gemm_out_resid", st);
  if (out_planes > 0) {
    eo.kind = EPI_F32_PLANES;
    eo.C = part; eo.ldc = d; eo.plane = T * d;
    return launch_gemm(dt, y, d, true, p->W_o, d, true, (int)T, d, d, eo, out_planes, st);
  }
  eo.kind = EPI_BIAS_RESID;
  eo.C = x_out; eo.ldc = d; eo.bias = p->b_o; eo.R = x_in; eo.ldr = d;
  return launch_gemm(dt, y, d, true, p->W_o, d, true, (int)T, d, d, eo, 1, st);
}

int mtgr_hstu_layer_fwd(const mtgr_layer_params* p, const void* x_in, void* x_out, const mtgr_layer_saved* saved,
                        const int32_t* offsets, const uint8_t* group_ids, const int64_t* timestamps, int32_t B,
                        int64_t T, float attn_scale, int dt, void* workspace, size_t ws_bytes,
                        mtgr_stream_t stream) {
  int r = layer_param_checks(p, dt);
  if (r) return r;
  if (!jagged_ok(offsets, group_ids, timestamps, B, T)) return MTGR_ERR_INVALID_ARG;
  const int d = p->d;
  if (T > 0 && (!x_in || !x_out)) return MTGR_ERR_INVALID_ARG;
  if (x_in == x_out && T > 0) return MTGR_ERR_INVALID_ARG;
  if (!vec_ok(x_in, d, dt) || !vec_ok(x_out, d, dt)) return MTGR_ERR_INVALID_ARG;
  if (saved && (!saved->xhat || !saved->mean1 || !saved->rstd1 || !saved->zgrad || !saved->uqkv || !saved->o ||
                !saved->mean2 || !saved->rstd2 || !saved->y))
    return MTGR_ERR_INVALID_ARG;
  if (ws_bytes < layer_fwd_ws(B, T, d, p->H, dt) || (T > 0 && !workspace)) return MTGR_ERR_WORKSPACE_TOO_SMALL;
  if (T == 0 || B == 0) return MTGR_OK;
  r = validate_jagged(offsets, group_ids, B, T, kLayerGroups, true, 0, S(stream));
  if (r) return r;
  hipStream_t st = S(stream);
  const size_t e = elt(dt);
  Carver cv{(char*)workspace, ws_bytes};
  void* ws_prep = cv.take(attn_ws(B, T));
  const size_t pb = attn_fwd_part_bytes(dt, B, T, p->H, p->dh);
  void* ws_part = pb ? cv.take(pb) : nullptr;
  void* ws_xhat = cv.take((size_t)T * d * e);
  void* ws_uqkv = cv.take((size_t)T * 4 * d * e);
  void* ws_o = cv.take((size_t)T * d * e);
  if (!cv.ok) return MTGR_ERR_WORKSPACE_TOO_SMALL;
  void* xhat = saved ? saved->xhat : ws_xhat;
  void* uqkv = saved ? saved->uqkv : ws_uqkv;
  void* o = saved ? saved->o : ws_o;
  void* y = saved ? saved->y : ws_xhat;  // xhat is dead once the projection has run
  PrepView pv;
  {
    ProfScope ps("prep", st);
    r = launch_prep(offsets, group_ids, B, T, ws_prep, st, &pv);
  }
  if (r) return r;
  return layer_fwd_body(p, x_in, x_out, saved, group_ids, timestamps, B, T, attn_scale, dt, pv, ws_part, xhat, uqkv,
                        o, y, nullptr, 0, st);
}

}  // extern "C"

namespace mtgr {

int stack_fwd_validate(const mtgr_layer_params* layers, int32_t L, const void* x_in, void* x_out,
                       const int32_t* offsets, const uint8_t* group_ids, const int64_t* timestamps, int32_t B,
                       int64_t T, int dt, const void* workspace, size_t ws_bytes) {
  if (L < 1 || !layers) return MTGR_ERR_INVALID_ARG;
  for (int l = 0; l < L; ++l) {
    const int r = layer_param_checks(&layers[l], dt);
    if (r) return r;
    if (layers[l].d != layers[0].d || layers[l].H != layers[0].H || layers[l].G != layers[0].G)
      return MTGR_ERR_INVALID_ARG;
  }
  if (!jagged_ok(offsets, group_ids, timestamps, B, T)) return MTGR_ERR_INVALID_ARG;
  const int d = layers[0].d;
  if (T > 0 && (!x_in || !x_out)) return MTGR_ERR_INVALID_ARG;
  if (x_in == x_out && T > 0) return MTGR_ERR_INVALID_ARG;
  if (!vec_ok(x_in, d, dt) || !vec_ok(x_out, d, dt)) return MTGR_ERR_INVALID_ARG;
  if (ws_bytes < stack_fwd_ws(B, T, d, layers[0].H, dt) || (T > 0 && !workspace))
    return MTGR_ERR_WORKSPACE_TOO_SMALL;
  return MTGR_OK;
}

}  // namespace mtgr

extern "C" {

int mtgr_hstu_stack_fwd(const mtgr_layer_params* layers, int32_t L, const void* x_in, void* x_out,
                        const int32_t* offsets, const uint8_t* group_ids, const int64_t* timestamps, int32_t B,
                        int64_t T, float attn_scale, int dt, void* workspace, size_t ws_bytes,
                        mtgr_stream_t stream) {
  return stack_fwd_run(layers, L, x_in, x_out, offsets, group_ids, timestamps, B, T, attn_scale, dt, workspace,
                       ws_bytes, S(stream), true);
}

}  // extern "C"

int mtgr::stack_fwd_run(const mtgr_layer_params* layers, int32_t L, const void* x_in, void* x_out,
                        const int32_t* offsets, const uint8_t* group_ids, const int64_t* timestamps, int32_t B,
                        int64_t T, float attn_scale, int dt, void* workspace, size_t ws_bytes, hipStream_t st,
                        bool check_meta) {
  int r = stack_fwd_validate(layers, L, x_in, x_out, offsets, group_ids, timestamps, B, T, dt, workspace, ws_bytes);
  if (r) return r;
  if (T == 0 || B == 0) return MTGR_OK;
  if (check_meta) {
    r = validate_jagged(offsets, group_ids, B, T, kLayerGroups, true, 0, st);
    if (r) return r;
  }
  const int d = layers[0].d;
  const size_t e = elt(dt);
  const int H = layers[0].H;
  Carver cv{(char*)workspace, ws_bytes};
  void* ws_prep = cv.take(attn_ws(B, T));
  const size_t pb = stack_part_bytes(B, T, d, H, dt);
  void* ws_part = pb ? cv.take(pb) : nullptr;
  void* xhat = cv.take((size_t)T * d * e);
  void* uqkv = cv.take((size_t)T * 4 * d * e);
  void* o = cv.take((size_t)T * d * e);
  void* h = cv.take((size_t)T * d * e);
  if (!cv.ok) return MTGR_ERR_WORKSPACE_TOO_SMALL;
  PrepView pv;
  {
    ProfScope ps("prep", st);
    r = launch_prep(offsets, group_ids, B, T, ws_prep, st, &pv);
  }
  if (r) return r;
  const int so = stack_out_planes(T, d, dt);
  if (so > 0) {
    // Short batches: each output projection leaves so fp32 planes; the next
    // layer's input norm (or the final sum) adds them with bias and
    // residual and stores the new residual stream in x_out (in place from
    // the second layer on).
    PartialRows pr = {};
    pr.part = (const float*)ws_part; pr.n = so; pr.plane = T * d; pr.ldp = d;
    pr.ldr = d; pr.xs = x_out; pr.ldxs = d;
    for (int l = 0; l < L; ++l) {
      if (l > 0) {
        pr.bias = layers[l - 1].b_o;
        pr.resid = l == 1 ? x_in : x_out;
      }
      r = layer_fwd_body(&layers[l], x_in, nullptr, nullptr, group_ids, timestamps, B, T, attn_scale, dt, pv, ws_part,
                         xhat, uqkv, o, xhat, l > 0 ? &pr : nullptr, so, st);
      if (r) return r;
    }
    pr.bias = layers[L - 1].b_o;
    pr.resid = L == 1 ? x_in : x_out;
    ProfScope ps("out_sum", st);
    return launch_partial_reduce(dt, pr, T, d, st);
  }
  // Layer l writes x_out when L-1-l is even and the spare buffer h otherwise,
  // so consecutive layers alternate and the last one lands in x_out.
  const void* src = x_in;
  for (int l = 0; l < L; ++l) {
    void* dst = ((L - 1 - l) % 2 == 0) ? x_out : h;
    r = layer_fwd_body(&layers[l], src, dst, nullptr, group_ids, timestamps, B, T, attn_scale, dt, pv, ws_part, xhat,
                       uqkv, o, xhat, nullptr, 0, st);
    if (r) return r;
    src = dst;
  }
  return MTGR_OK;
}

extern "C" {

int mtgr_hstu_layer_bwd(const mtgr_layer_params* p, const void* x_in, const mtgr_layer_saved* saved,
                        const void* dx_out, void* dx_in, const mtgr_layer_grads* grads,
                        const mtgr_layer_bwd_extras* extras, const int32_t* offsets, const uint8_t* group_ids,
                        const int64_t* timestamps, int32_t B, int64_t T, int32_t max_len, float attn_scale,
                        int dt, void* workspace, size_t ws_bytes, mtgr_stream_t stream) {
  int r = layer_param_checks(p, dt);
  if (r) return r;
  if (!jagged_ok(offsets, group_ids, timestamps, B, T) || max_len < 0) return MTGR_ERR_INVALID_ARG;
  if (!saved || !grads) return MTGR_ERR_INVALID_ARG;
  if (!grads->W_uqkv || !grads->gamma1 || !grads->beta1 || !grads->gamma2 || !grads->beta2 || !grads->W_o)
    return MTGR_ERR_INVALID_ARG;
  const int d = p->d;
  if (T > 0 && (!x_in || !dx_out || !dx_in || !saved->xhat || !saved->mean1 || !saved->rstd1 || !saved->zgrad ||
                !saved->uqkv || !saved->o || !saved->mean2 || !saved->rstd2 || !saved->y))
    return MTGR_ERR_INVALID_ARG;
  if (!vec_ok(x_in, d, dt) || !vec_ok(dx_out, d, dt) || !vec_ok(dx_in, d, dt)) return MTGR_ERR_INVALID_ARG;
  if (ws_bytes < layer_bwd_ws(B, T, max_len, d, p->H, dt) || (T > 0 && !workspace))
    return MTGR_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = S(stream);
  const int G = p->G;
  if (T > 0 && B > 0) {
    r = validate_jagged(offsets, group_ids, B, T, kLayerGroups, true, max_len, st);
    if (r) return r;
  }
  if (T == 0 || B == 0) {
    r = launch_fill_f32(grads->W_uqkv, (int64_t)4 * d * d, 0.f, st);
    if (!r) r = launch_fill_f32(grads->W_o, (int64_t)d * d, 0.f, st);
    if (!r) r = launch_fill_f32(grads->gamma1, (int64_t)G * d, 0.f, st);
    if (!r) r = launch_fill_f32(grads->beta1, (int64_t)G * d, 0.f, st);
    if (!r) r = launch_fill_f32(grads->gamma2, (int64_t)G * d, 0.f, st);
    if (!r) r = launch_fill_f32(grads->beta2, (int64_t)G * d, 0.f, st);
    if (!r && grads->b_uqkv) r = launch_fill_f32(grads->b_uqkv, (int64_t)4 * d, 0.f, st);
    if (!r && grads->b_o) r = launch_fill_f32(grads->b_o, (int64_t)d, 0.f, st);
    return r;
  }
  const size_t e = elt(dt);
  Carver cv{(char*)workspace, ws_bytes};
  void* ws_prep = cv.take(attn_ws(B, T));
  void* ws_dy = cv.take((size_t)T * d * e);
  void* ws_do = cv.take((size_t)T * d * e);
  void* ws_dz = cv.take((size_t)T * 4 * d * e);
  size_t rbytes = gln_bwd_workspace_bytes(T, d, kMaxG), cbytes = colsum_workspace_bytes(T, 4 * d);
  void* ws_red = cv.take(rbytes > cbytes ? rbytes : cbytes);
  const size_t dsb = ds_ws(B, T, max_len, p->H, dt);
  void* ws_ds = dsb ? cv.take(dsb) : nullptr;
  if (!cv.ok) return MTGR_ERR_WORKSPACE_TOO_SMALL;
  PrepView pv;
  {
    ProfScope ps("prep", st);
    r = launch_prep(offsets, group_ids, B, T, ws_prep, st, &pv);
  }
  if (r) return r;
  const bool want_dact = extras && extras->d_uqkv;
  void* dO = (extras && extras->d_o) ? extras->d_o : ws_do;
  // gradients w.r.t. SiLU(z) go to the caller's buffer when asked for,
  // otherwise straight into dz with SiLU' applied by the producers
  void* dact = want_dact ? extras->d_uqkv : ws_dz;
  const char* zb = (const char*)saved->zgrad;
  const char* ub = (const char*)saved->uqkv;
  char* db = (char*)dact;
  // a6 backward: dy = dx_out W_o ; dW_o = dx_out^T y ; db_o = colsum(dx_out)
  GemmEpiArgs ep = {};
  ep.kind = EPI_STORE; ep.C = ws_dy; ep.ldc = d;
  {
    ProfScope ps("gemm_dy", st);
    r = launch_gemm(dt, dx_out, d, true, p->W_o, d, false, (int)T, d, d, ep, 1, st);
  }
  if (r) return r;
  GemmEpiArgs ew = {};
  ew.kind = EPI_F32_ATOMIC; ew.C = grads->W_o; ew.ldc = d;
  {
    ProfScope ps("gemm_dW_o", st);
    r = launch_gemm(dt, dx_out, d, false, saved->y, d, false, d, d, (int)T, ew, splits_for(d, d, (int)T), st);
  }
  if (r) return r;
  if (grads->b_o) {
    r = launch_colsum(dt, dx_out, d, T, d, grads->b_o, ws_red, st);
    if (r) return r;
  }
  // a5 backward: dU = dy * GLN2(o) [* SiLU'(z_u)], dO = GLN2'(dy * U)
  {
    ProfScope ps("gln2_gate_bwd", st);
    r = launch_gln_bwd(dt, ws_dy, d, saved->o, d, saved->mean2, saved->rstd2, p->gamma2, p->beta2, group_ids, T,
                     d, G, dO, d, nullptr, 0, ub, 4 * d, db, 4 * d, want_dact ? nullptr : zb, 4 * d,
                       grads->gamma2, grads->beta2, ws_red, st);
  }
  if (r) return r;
  // a7: attention backward into the Q, K, V blocks
  AttnArgs a = {};
  a.q = ub + (size_t)d * e; a.k = ub + (size_t)2 * d * e; a.v = ub + (size_t)3 * d * e; a.ldqkv = 4 * d;
  a.d_o = dO; a.lddo = d;
  a.dq = db + (size_t)d * e; a.dk = db + (size_t)2 * d * e; a.dv = db + (size_t)3 * d * e; a.lddqkv = 4 * d;
  if (!want_dact) {
    a.zq = zb + (size_t)d * e; a.zk = zb + (size_t)2 * d * e; a.zv = zb + (size_t)3 * d * e; a.ldz = 4 * d;
  }
  a.ts = timestamps; a.B = B; a.T = T; a.H = p->H; a.dh = p->dh; a.alpha = p->alpha; a.scale = attn_scale;
  set_ds(a, ws_ds, max_len, dt);
  r = launch_attn_bwd(dt, a, pv, st);
  if (r) return r;
  if (want_dact) {
    if (hipMemcpyAsync(ws_dz, dact, (size_t)T * 4 * d * e, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return MTGR_ERR_HIP;
    r = launch_silu_grad_mul(dt, ws_dz, 4 * d, saved->zgrad, 4 * d, T, 4 * d, st);
    if (r) return r;
  }
  // a3 backward: dxhat = dz W_uqkv ; dW_uqkv = dz^T xhat ; db_uqkv = colsum(dz)
  GemmEpiArgs ex = {};
  ex.kind = EPI_STORE; ex.C = ws_dy; ex.ldc = d;
  {
    ProfScope ps("gemm_dxhat", st);
    r = launch_gemm(dt, ws_dz, 4 * d, true, p->W_uqkv, d, false, (int)T, d, 4 * d, ex, 1, st);
  }
  if (r) return r;
  GemmEpiArgs eu = {};
  eu.kind = EPI_F32_ATOMIC; eu.C = grads->W_uqkv; eu.ldc = d;
  {
    ProfScope ps("gemm_dW_uqkv", st);
    r = launch_gemm(dt, ws_dz, 4 * d, false, saved->xhat, d, false, 4 * d, d, (int)T, eu,
                    splits_for(4 * d, d, (int)T), st);
  }
  if (r) return r;
  if (grads->b_uqkv) {
    r = launch_colsum(dt, ws_dz, 4 * d, T, 4 * d, grads->b_uqkv, ws_red, st);
    if (r) return r;
  }
  // a2 backward with the residual: dx = GLN1'(dxhat) + dx_out
  ProfScope ps("gln1_bwd", st);
  return launch_gln_bwd(dt, ws_dy, d, x_in, d, saved->mean1, saved->rstd1, p->gamma1, p->beta1, group_ids, T, d,
                        G, dx_in, d, dx_out, d, nullptr, 0, nullptr, 0, nullptr, 0, grads->gamma1, grads->beta1,
                        ws_red, st);
}

}  // extern "C"
