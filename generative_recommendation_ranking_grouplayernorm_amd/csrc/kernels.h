// Host-side launchers of the gfx950 kernels (C++ linkage, used by api.cpp).
#pragma once

#include "common.h"

namespace mtgr {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Brackets the launches of one named kernel step with HIP events on stream
// `s` when timing is switched on (mtgr_profile_enable); a no-op otherwise.
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t s);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  const char* name_;
  hipStream_t stream_;
  void* begin_;
};
// True while mtgr_profile_enable(1) is in effect.
bool profiling_enabled();

// mtgr_hstu_stack_fwd / mtgr_candidate_head_fwd on a HIP stream; with
// check_meta false the validation-mode device check is skipped (the graph
// entry points run it before capture and before every replay instead).
int stack_fwd_run(const mtgr_layer_params* layers, int32_t L, const void* x_in, void* x_out,
                  const int32_t* offsets, const uint8_t* group_ids, const int64_t* timestamps, int32_t B, int64_t T,
                  float attn_scale, int dt, void* workspace, size_t ws_bytes, hipStream_t st, bool check_meta);
int head_fwd_run(const mtgr_head_params* p, const void* x, int64_t ld_x, const int32_t* offsets,
                 const uint8_t* group_ids, int32_t B, int64_t T, int64_t n_cand, float* logits, int dt,
                 void* workspace, size_t ws_bytes, hipStream_t stream, bool check_meta);

// Host-side argument checks of mtgr_hstu_attn_fwd other than its workspace.
int attn_fwd_arg_checks(const void* q, const void* k, const void* v, int64_t ld_qkv, const void* o, int64_t ld_o,
                        const int32_t* offsets, const uint8_t* group_ids, const int64_t* timestamps, int32_t B,
                        int64_t T, int32_t H, int32_t dh, int dt);

// Host-side argument checks of mtgr_hstu_stack_fwd (MTGR_OK or a status).
int stack_fwd_validate(const mtgr_layer_params* layers, int32_t L, const void* x_in, void* x_out,
                       const int32_t* offsets, const uint8_t* group_ids, const int64_t* timestamps, int32_t B,
                       int64_t T, int dt, const void* workspace, size_t ws_bytes);

// Rows per attention tile: queries per forward / dQ workgroup, keys per
// dK/dV workgroup.
constexpr int ATTN_QTILE = 128;   // forward and dQ
constexpr int ATTN_KTILE = 128;   // dK/dV

// ---- a1: segments and tile lists -----------------------------------------
struct TileList {
  int32_t* ntiles;   // [1] number of valid entries
  int2* tiles;       // (user, first row) of each tile, longest users first
  int64_t max_tiles; // host-side upper bound on *ntiles
};
struct PrepView {
  int32_t* seg;      // [B, 5]
  TileList q;        // ATTN_QTILE-row tiles
  TileList k;        // ATTN_KTILE-row tiles
  int64_t* tprefix;  // [B + 1] exclusive prefix of ceil(L / 128)^2
};
int64_t max_tiles(int B, int64_t T, int rows_per_tile);
size_t prep_workspace_bytes(int B, int64_t T);
int launch_prep(const int32_t* offsets, const uint8_t* group_ids, int B, int64_t T, void* ws,
                hipStream_t stream, PrepView* out);
int launch_seg_only(const int32_t* offsets, const uint8_t* group_ids, int B, int64_t T, int32_t* seg,
                    hipStream_t stream);
// Device check of jagged metadata (validation mode): offsets[0] = 0,
// non-decreasing, offsets[B] = T; every group id < G; with `ordered`, group
// ids non-decreasing inside each user; with max_len > 0, no row longer than
// max_len.  Reads offsets[0..B] (when B > 0) and group_ids[0..T) only.
// MTGR_OK when validation is off or the metadata passes, MTGR_ERR_VALIDATION
// when it fails; synchronises `stream` when on.
int validate_jagged(const int32_t* offsets, const uint8_t* group_ids, int B, int64_t T, int G, bool ordered,
                    int max_len, hipStream_t stream);
bool validation_enabled();
void set_validation(int on);

// ---- Stochastic Length sampling and the token-budget cut -----------------
int64_t sl_max_blocks(int B, int64_t T);
size_t sl_workspace_bytes(int B, int64_t T);
int launch_stochastic_length(const int32_t* offsets, const uint8_t* g, const int64_t* ts, const void* x,
                             int64_t ldx_bytes, int row_bytes, int B, int64_t T, const float* u, int s_keep,
                             int64_t budget, int32_t* offsets_out, uint8_t* g_out, int64_t* ts_out, void* x_out,
                             int64_t ldo_bytes, int64_t* fit_out, void* ws, hipStream_t stream);

// ---- candidate head and loss ----------------------------------------------
struct HeadArgs {
  const int32_t* offsets; const uint8_t* group_ids; int B; int64_t T; int64_t n_cand;
  const void* x; int64_t ldx;
  int d, h, nt;
  const void* W1; const void* b1; const void* W2; const void* b2;
  bool train;           // loss and backward too
  const float* labels;  // [n_cand, nt] when train
  float* logits;        // [n_cand, nt] or NULL
  float* loss;          // [1]
  void* dx; int64_t lddx;
  float* dW1; float* db1; float* dW2; float* db2;
};
struct HeadWs {
  int32_t* seg; int32_t* cand_off;
  char* xc; char* z1; char* hc; char* dz1;
  float* dz; float* loss_k;
  char* dxc; char* red;
  size_t bytes;
};
HeadWs head_carve(void* ws, int B, int64_t n_cand, int d, int h, int nt, int dt);
size_t head_workspace_bytes(int B, int64_t n_cand, int d, int h, int nt, int dt);
int head_split(int M, int N, int K);
int launch_head(int dt, const HeadArgs& a, void* ws, hipStream_t stream);
// Host-side argument checks shared by the head entry points.
int head_validate(const mtgr_head_params* p, const void* x, int64_t ld_x, const int32_t* offsets,
                  const uint8_t* group_ids, int32_t B, int64_t T, int64_t n_cand, int dt);

// ---- a2/a5: group norm rows ---------------------------------------------
// y = GLN(x) (mode plain) or y = GLN(x) * u (mode gate).
// Group ids at or above G read the last parameter row (G - 1).
int launch_gln_fwd(int dt, const void* x, int64_t ldx, void* y, int64_t ldy, const void* gamma,
                   const void* beta, const uint8_t* g, int64_t T, int d, int G, float eps, float* mean,
                   float* rstd, const void* u, int64_t ldu, hipStream_t stream);
// Row inputs given as fp32 partial sums (split-K products, split-key
// attention): x[row, col] = round_T(sum_{s < n} part[s * plane + row * ldp +
// col] (+ bias[col]) (+ resid[row * ldr + col])), the planes added in order,
// then the bias, then the residual.  When xs is set, x is also stored there
// (xs may alias resid: each element is read before it is written, by the
// same thread).
struct PartialRows {
  const float* part; int n; int64_t plane; int64_t ldp;
  const void* bias; const void* resid; int64_t ldr;
  void* xs; int64_t ldxs;
};
// launch_gln_fwd with x taken from partial sums.
int launch_gln_fwd_part(int dt, const PartialRows& in, void* y, int64_t ldy, const void* gamma, const void* beta,
                        const uint8_t* g, int64_t T, int d, int G, float eps, float* mean, float* rstd,
                        const void* u, int64_t ldu, hipStream_t stream);
// Only the sum: xs = x (in.xs must be set).
int launch_partial_reduce(int dt, const PartialRows& in, int64_t T, int d, hipStream_t stream);
// Backward.  Plain: dx = GLN'(dy) [+ resid].  Gate (u != NULL): the forward
// was y = GLN(x) * u, so du = dy * GLN(x) [* gu if gu != NULL, gu = SiLU'(zu)] and
// dx = GLN'(dy * u).  dgamma/dbeta fp32 [G, d] overwritten.
size_t gln_bwd_workspace_bytes(int64_t T, int d, int G);
int launch_gln_bwd(int dt, const void* dy, int64_t lddy, const void* x, int64_t ldx, const float* mean,
                   const float* rstd, const void* gamma, const void* beta, const uint8_t* g,
                   int64_t T, int d, int G, void* dx, int64_t lddx, const void* resid,
                   int64_t ldr, const void* u, int64_t ldu, void* du, int64_t lddu,
                   const void* zu, int64_t ldzu, float* dgamma, float* dbeta, void* ws,
                   hipStream_t stream);

// ---- GEMM ----------------------------------------------------------------
// C[m, n] = sum_k A(m, k) * B(n, k).
//   a_kcontig: A(m,k) = A[m*lda + k], else A[k*lda + m]
//   b_kcontig: B(n,k) = B[n*ldb + k], else B[k*ldb + n]
enum GemmEpi {
  EPI_STORE = 0,       // C = acc                                  (dtype dt)
  EPI_BIAS_SILU = 1,   // z = acc + bias; Z = z or SiLU'(z) (if given); C = SiLU(z)
  EPI_BIAS_RESID = 2,  // C = acc + bias + R
  EPI_F32_STORE = 3,   // Cf = acc (fp32)
  EPI_F32_ATOMIC = 4,  // Cf += acc (fp32, for split-K)
  EPI_F32_PLANES = 5   // Cf[split * plane + m * ldc + n] = acc (split-K, one fp32 plane per split)
};
struct GemmEpiArgs {
  int kind;
  void* C;
  int64_t ldc;
  const void* bias;  // [N] or NULL
  void* Z;           // pre-activation out (EPI_BIAS_SILU) or NULL
  int64_t ldz;
  int zgrad;         // 1: Z receives SiLU'(z) instead of z
  const void* R;     // residual (EPI_BIAS_RESID)
  int64_t ldr;
  int64_t plane;     // elements between split planes (EPI_F32_PLANES)
};
// K splits for an EPI_F32_PLANES product of short batches: enough 128 x 128
// tile jobs for one per compute unit, each at least two K steps deep.
int gemm_plane_splits(int M, int N, int K);
int launch_gemm(int dt, const void* A, int64_t lda, bool a_kcontig, const void* B, int64_t ldb,
                bool b_kcontig, int M, int N, int K, const GemmEpiArgs& ep, int splits,
                hipStream_t stream);
int launch_fill_f32(float* p, int64_t n, float v, hipStream_t stream);
// Column sums of a [T, N] matrix into fp32 out[N] (bias gradients).
int launch_colsum(int dt, const void* X, int64_t ldx, int64_t T, int N, float* out, void* ws,
                  hipStream_t stream);
size_t colsum_workspace_bytes(int64_t T, int N);
// x[t, n] *= SiLU'(z[t, n]) for n < N (in place on x).
int launch_silu_grad_mul(int dt, void* x, int64_t ldx, const void* z, int64_t ldz, int64_t T, int N,
                         hipStream_t stream);

// ---- a4/a7: attention ----------------------------------------------------
struct AttnArgs {
  const void* q; const void* k; const void* v; int64_t ldqkv;
  void* o; int64_t ldo;
  const void* d_o; int64_t lddo;
  void* dq; void* dk; void* dv; int64_t lddqkv;
  // optional SiLU derivatives at the pre-activations: when set, the
  // backward writes dq * zq (likewise dk, dv), zq/zk/zv at row stride ldz.
  const void* zq; const void* zk; const void* zv; int64_t ldz;
  const int64_t* ts;
  int B; int64_t T; int H; int dh;
  float alpha, scale;
  // backward only: dS buffer of ds_cap tile pairs per head (32 KB each in
  // 16-bit types).  When set, the dK/dV kernel stores dS there and dQ
  // streams it; when NULL, dQ recomputes S and dA.
  void* ds; int64_t ds_cap;
  // forward only: fp32 partial sums of nsplit key runs ([nsplit][T][H dh],
  // O itself is then not written: the caller adds the planes), or NULL for
  // one workgroup per (query tile, head) writing O
  float* part; int nsplit;
};
// Key runs per (query tile, head) of the 16-bit forward: more than one only
// when the batch has too few query tiles to give every compute unit two
// workgroups.  attn_fwd_part_bytes: the partial-sum storage that needs.
constexpr int ATTN_MAX_SPLITS = 4;
int attn_fwd_splits(int dt, int B, int64_t T, int H);
size_t attn_fwd_part_bytes(int dt, int B, int64_t T, int H, int dh);
// Bytes of dS storage that a batch of B rows, T tokens and rows of at most
// max_len tokens can need: H * 32 KB per 128 x 128 tile pair, with
// sum_b ceil(L_b / 128)^2 <= min(B ceil(M / 128)^2, (M T + 254 T + 16129 B) / 16384).
size_t attn_ds_bytes(int B, int64_t T, int max_len, int H);
constexpr size_t DS_TILE_BYTES = 32768;  // one 128-query x 128-key tile of 16-bit dS
int launch_attn_fwd(int dt, const AttnArgs& a, const PrepView& pv, hipStream_t stream);
int launch_attn_bwd(int dt, const AttnArgs& a, const PrepView& pv, hipStream_t stream);

}  // namespace mtgr
