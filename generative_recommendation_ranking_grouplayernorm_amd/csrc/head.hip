// Candidate head and discriminative loss after the last layer.
//
// zzxanthony blog "MTGR：工业级生成式推荐框架" 5.4 and 7: the candidate tokens'
// outputs go through an MLP to logits; 6 and fun-rec "MTGR：混合范式建模"
// 7.3.1: the loss is discriminative and taken at candidate positions only;
// paper-daily 它解决什么问题: a click rate and a conversion rate per exposed
// candidate.  Read as: logits = Linear2(SiLU(Linear1(x_c))) with one logit per
// task, loss = mean over candidates of the summed per-task binary
// cross-entropy.
//
// Launch sequence (training): segments; one workgroup numbers the candidate
// tokens (exclusive scan of the per-user counts); one wave per candidate
// gathers its row; the hidden layer is a GEMM with a bias + SiLU epilogue
// that keeps the pre-activation; one wave per candidate computes the logits,
// its loss term, dlogits and dZ1 = (dlogits W2) * SiLU'(z1); sums over the
// candidates in fixed order (64-candidate chunks, then the chunks) give dW2,
// db2, db1 and the loss; the GEMMs of the layer give dW1 and dX_c = dZ1 W1;
// one wave per token row writes dx (its candidate's row of dX_c, zeros
// elsewhere).
#include "kernels.h"

namespace mtgr {

constexpr int HEAD_PLAN_THREADS = 1024;

// cand_off[b] = candidates of users before b (exclusive scan of n_c), and
// cand_off[B] = all of them.
__global__ __launch_bounds__(HEAD_PLAN_THREADS) void head_plan_kernel(const int32_t* __restrict__ seg, int B,
                                                                      int32_t* __restrict__ cand_off) {
  __shared__ int32_t scan[HEAD_PLAN_THREADS];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int b0 = 0; b0 < B; b0 += HEAD_PLAN_THREADS) {
    const int b = b0 + tid;
    const int n = b < B ? seg[(int64_t)b * 5 + 4] - seg[(int64_t)b * 5 + 3] : 0;
    scan[tid] = n;
    __syncthreads();
    for (int off = 1; off < HEAD_PLAN_THREADS; off <<= 1) {
      const int add = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const int incl = carry_s + scan[tid];
    if (b < B) cand_off[b] = incl - n;
    __syncthreads();
    if (tid == HEAD_PLAN_THREADS - 1) carry_s = incl;
    __syncthreads();
  }
  if (tid == 0) cand_off[B] = carry_s;
}

// largest b with off[b] <= k (off non-decreasing, off[0] = 0 <= k < off[B])
__device__ __forceinline__ int head_user_of(const int32_t* off, int B, int64_t k) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= k) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Xc[k] = x[row of candidate k]; rows past the metadata's candidate count
// (a caller error) are zero-filled.
__global__ __launch_bounds__(256) void head_gather_kernel(const int32_t* __restrict__ seg,
                                                          const int32_t* __restrict__ cand_off, int B, int64_t n_cand,
                                                          const char* __restrict__ x, int64_t ldx_bytes,
                                                          int row_bytes, char* __restrict__ xc) {
  const int64_t k = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (k >= n_cand) return;
  char* dst = xc + k * (int64_t)row_bytes;
  if (k >= cand_off[B]) {
    for (int c = lane * 16; c < row_bytes; c += 1024) *(uint4*)(dst + c) = make_uint4(0, 0, 0, 0);
    return;
  }
  const int b = head_user_of(cand_off, B, k);
  const int64_t row = seg[(int64_t)b * 5 + 3] + (k - cand_off[b]);
  const char* src = x + row * ldx_bytes;
  for (int c = lane * 16; c < row_bytes; c += 1024) *(uint4*)(dst + c) = *(const uint4*)(src + c);
}

// One wave per candidate k: logits z_t = H[k] . W2[t] + b2[t].  With labels:
// loss_k = sum_t softplus(z_t) - y_t z_t, dz_t = (sigmoid(z_t) - y_t) / n,
// dZ1[k] = (sum_t dz_t W2[t]) * SiLU'(Z1[k]).
template <typename T, int NT, bool TRAIN>
__global__ __launch_bounds__(256) void head_out_kernel(const T* __restrict__ Hc, const T* __restrict__ Z1,
                                                       const T* __restrict__ W2, const T* __restrict__ b2, int h,
                                                       int64_t n_cand, const float* __restrict__ labels,
                                                       float* __restrict__ logits, float* __restrict__ dz_out,
                                                       float* __restrict__ loss_k, T* __restrict__ dZ1) {
  const int64_t k = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (k >= n_cand) return;
  const T* hr = Hc + k * h;
  float acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.f;
  for (int j = lane; j < h; j += 64) {
    const float hv = to_f32(hr[j]);
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] += hv * to_f32(W2[(int64_t)t * h + j]);
  }
  float z[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) z[t] = warp_sum(acc[t]) + (b2 ? to_f32(b2[t]) : 0.f);
  if (lane == 0 && logits) {
#pragma unroll
    for (int t = 0; t < NT; ++t) logits[k * NT + t] = z[t];
  }
  if (!TRAIN) return;
  const float inv_n = 1.0f / (float)n_cand;
  float dz[NT];
  float lk = 0.f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float y = labels[k * NT + t];
    // softplus(z) = max(z, 0) + log1p(exp(-|z|)); sigmoid from the same exp
    const float e = expf(-fabsf(z[t]));
    lk += fmaxf(z[t], 0.f) + log1pf(e) - y * z[t];
    const float sg = z[t] >= 0.f ? 1.0f / (1.0f + e) : e / (1.0f + e);
    dz[t] = (sg - y) * inv_n;
  }
  if (lane == 0) {
    loss_k[k] = lk;
#pragma unroll
    for (int t = 0; t < NT; ++t) dz_out[k * NT + t] = dz[t];
  }
  const T* zr = Z1 + k * h;
  T* dr = dZ1 + k * h;
  for (int j = lane; j < h; j += 64) {
    float dh = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) dh += dz[t] * to_f32(W2[(int64_t)t * h + j]);
    const float zz = to_f32(zr[j]);
    const float s = 1.0f / (1.0f + expf(-zz));
    dr[j] = from_f32<T>(dh * s * (1.0f + zz * (1.0f - s)));
  }
}

// Sums over the candidates, in two fixed-order stages.  Stage 1: workgroup
// (b, c) takes 256 outputs and candidates [64 c, 64 c + 64), writing its
// part of partial row c
//   [dW2 (nt x h) | db2 (nt) | db1 (h) | loss (1)]
// with dW2[t][j] = sum dz[k][t] H[k][j], db2[t] = sum dz[k][t],
// db1[j] = sum dZ1[k][j], loss = sum loss_k.  Stage 2 adds the partial rows
// in order.
constexpr int HEAD_CHUNK = 64;

__host__ __device__ inline int head_red_width(int h, int nt) { return nt * h + nt + h + 1; }

template <typename T, int NT>
__global__ __launch_bounds__(256) void head_grad_partials_kernel(const T* __restrict__ Hc,
                                                                 const float* __restrict__ dz,
                                                                 const T* __restrict__ dZ1,
                                                                 const float* __restrict__ loss_k, int h,
                                                                 int64_t n_cand, float* __restrict__ part) {
  // blockIdx.x: 256 consecutive outputs; blockIdx.y: the candidate chunk
  const int64_t k0 = (int64_t)blockIdx.y * HEAD_CHUNK;
  const int64_t k1 = min(k0 + HEAD_CHUNK, n_cand);
  const int width = head_red_width(h, NT);
  const int o = blockIdx.x * 256 + threadIdx.x;
  if (o >= width) return;
  float acc = 0.f;
  if (o < NT * h) {
    const int t = o / h, j = o - t * h;
#pragma unroll 8
    for (int64_t k = k0; k < k1; ++k) acc += dz[k * NT + t] * to_f32(Hc[k * h + j]);
  } else if (o < NT * h + NT) {
    const int t = o - NT * h;
    for (int64_t k = k0; k < k1; ++k) acc += dz[k * NT + t];
  } else if (o < NT * h + NT + h) {
    const int j = o - NT * h - NT;
#pragma unroll 8
    for (int64_t k = k0; k < k1; ++k) acc += to_f32(dZ1[k * h + j]);
  } else {
    for (int64_t k = k0; k < k1; ++k) acc += loss_k[k];
  }
  part[(int64_t)blockIdx.y * width + o] = acc;
}

__global__ __launch_bounds__(256) void head_grad_reduce_kernel(const float* __restrict__ part, int nchunks, int h,
                                                               int nt, int64_t n_cand, float* __restrict__ dW2,
                                                               float* __restrict__ db2, float* __restrict__ db1,
                                                               float* __restrict__ loss) {
  const int width = head_red_width(h, nt);
  const int o = blockIdx.x * 256 + threadIdx.x;
  if (o >= width) return;
  float acc = 0.f;
  for (int c = 0; c < nchunks; ++c) acc += part[(int64_t)c * width + o];
  if (o < nt * h) dW2[o] = acc;
  else if (o < nt * h + nt) { if (db2) db2[o - nt * h] = acc; }
  else if (o < nt * h + nt + h) { if (db1) db1[o - nt * h - nt] = acc; }
  else *loss = acc / (float)n_cand;
}

// dx[r] = dXc[candidate ordinal of r] for candidate rows, zeros elsewhere.
__global__ __launch_bounds__(256) void head_expand_kernel(const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ seg,
                                                          const int32_t* __restrict__ cand_off, int B, int64_t T,
                                                          int64_t n_cand, const char* __restrict__ dxc, int row_bytes,
                                                          char* __restrict__ dx, int64_t lddx_bytes) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= T) return;
  char* dst = dx + r * lddx_bytes;
  int64_t k = -1;
  if (B > 0 && r < offsets[B]) {
    const int b = head_user_of(offsets, B, r);
    const int c0 = seg[(int64_t)b * 5 + 3];
    if (r >= c0) k = cand_off[b] + (r - c0);
  }
  if (k >= 0 && k < n_cand) {
    const char* src = dxc + k * (int64_t)row_bytes;
    for (int c = lane * 16; c < row_bytes; c += 1024) *(uint4*)(dst + c) = *(const uint4*)(src + c);
  } else {
    for (int c = lane * 16; c < row_bytes; c += 1024) *(uint4*)(dst + c) = make_uint4(0, 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
HeadWs head_carve(void* ws, int B, int64_t n_cand, int d, int h, int nt, int dt) {
  const size_t e = dt == MTGR_F32 ? 4 : 2;
  HeadWs w = {};
  size_t off = 0;
  char* base = (char*)ws;
  auto take = [&](size_t n) -> char* {
    const size_t at = off;
    off += align_up(n, 256);
    return base ? base + at : nullptr;
  };
  w.seg = (int32_t*)take((size_t)B * 5 * 4);
  w.cand_off = (int32_t*)take((size_t)(B + 1) * 4);
  w.xc = take((size_t)n_cand * d * e);
  w.z1 = take((size_t)n_cand * h * e);
  w.hc = take((size_t)n_cand * h * e);
  w.dz1 = take((size_t)n_cand * h * e);
  w.dz = (float*)take((size_t)n_cand * nt * 4);
  w.loss_k = (float*)take((size_t)n_cand * 4);
  w.dxc = take((size_t)n_cand * d * e);
  w.red = take((size_t)((n_cand + HEAD_CHUNK - 1) / HEAD_CHUNK) * head_red_width(h, nt) * sizeof(float));
  w.bytes = off;
  return w;
}

size_t head_workspace_bytes(int B, int64_t n_cand, int d, int h, int nt, int dt) {
  return head_carve(nullptr, B, n_cand, d, h, nt, dt).bytes;
}

template <typename T, int NT>
static void head_out_launch(const HeadWs& w, const void* W2, const void* b2, int h, int64_t n_cand,
                            const float* labels, float* logits, bool train, hipStream_t st) {
  const dim3 grid((unsigned)((n_cand + 3) / 4));
  if (train)
    hipLaunchKernelGGL((head_out_kernel<T, NT, true>), grid, dim3(256), 0, st, (const T*)w.hc, (const T*)w.z1,
                       (const T*)W2, (const T*)b2, h, n_cand, labels, logits, w.dz, w.loss_k, (T*)w.dz1);
  else
    hipLaunchKernelGGL((head_out_kernel<T, NT, false>), grid, dim3(256), 0, st, (const T*)w.hc, (const T*)w.z1,
                       (const T*)W2, (const T*)b2, h, n_cand, labels, logits, w.dz, w.loss_k, (T*)w.dz1);
}

template <typename T>
static int head_out_dispatch(int nt, const HeadWs& w, const void* W2, const void* b2, int h, int64_t n_cand,
                             const float* labels, float* logits, bool train, hipStream_t st) {
  switch (nt) {
    case 1: head_out_launch<T, 1>(w, W2, b2, h, n_cand, labels, logits, train, st); break;
    case 2: head_out_launch<T, 2>(w, W2, b2, h, n_cand, labels, logits, train, st); break;
    case 3: head_out_launch<T, 3>(w, W2, b2, h, n_cand, labels, logits, train, st); break;
    case 4: head_out_launch<T, 4>(w, W2, b2, h, n_cand, labels, logits, train, st); break;
    default: return MTGR_ERR_UNSUPPORTED;
  }
  MTGR_LAUNCH_CHECK();
  return MTGR_OK;
}

template <typename T>
static int head_sums(int nt, const HeadWs& w, int h, int64_t n_cand, float* dW2, float* db2, float* db1, float* loss,
                     hipStream_t st) {
  const int nchunks = (int)((n_cand + HEAD_CHUNK - 1) / HEAD_CHUNK);
  const dim3 grid((unsigned)((head_red_width(h, nt) + 255) / 256), (unsigned)nchunks);
  float* part = (float*)w.red;
  switch (nt) {
    case 1: hipLaunchKernelGGL((head_grad_partials_kernel<T, 1>), grid, dim3(256), 0, st, (const T*)w.hc, w.dz, (const T*)w.dz1, w.loss_k, h, n_cand, part); break;
    case 2: hipLaunchKernelGGL((head_grad_partials_kernel<T, 2>), grid, dim3(256), 0, st, (const T*)w.hc, w.dz, (const T*)w.dz1, w.loss_k, h, n_cand, part); break;
    case 3: hipLaunchKernelGGL((head_grad_partials_kernel<T, 3>), grid, dim3(256), 0, st, (const T*)w.hc, w.dz, (const T*)w.dz1, w.loss_k, h, n_cand, part); break;
    case 4: hipLaunchKernelGGL((head_grad_partials_kernel<T, 4>), grid, dim3(256), 0, st, (const T*)w.hc, w.dz, (const T*)w.dz1, w.loss_k, h, n_cand, part); break;
    default: return MTGR_ERR_UNSUPPORTED;
  }
  const int width = head_red_width(h, nt);
  hipLaunchKernelGGL(head_grad_reduce_kernel, dim3((unsigned)((width + 255) / 256)), dim3(256), 0, st, part, nchunks,
                     h, nt, n_cand, dW2, db2, db1, loss);
  MTGR_LAUNCH_CHECK();
  return MTGR_OK;
}

int launch_head(int dt, const HeadArgs& a, void* ws, hipStream_t st) {
  const size_t e = dt == MTGR_F32 ? 4 : 2;
  const HeadWs w = head_carve(ws, a.B, a.n_cand, a.d, a.h, a.nt, dt);
  int r = launch_seg_only(a.offsets, a.group_ids, a.B, a.T, w.seg, st);
  if (r) return r;
  {
    ProfScope ps("head_gather", st);
    hipLaunchKernelGGL(head_plan_kernel, dim3(1), dim3(HEAD_PLAN_THREADS), 0, st, w.seg, a.B, w.cand_off);
    if (a.n_cand > 0)
      hipLaunchKernelGGL(head_gather_kernel, dim3((unsigned)((a.n_cand + 3) / 4)), dim3(256), 0, st, w.seg,
                         w.cand_off, a.B, a.n_cand, (const char*)a.x, a.ldx * (int64_t)e, (int)(a.d * e),
                         (char*)w.xc);
    MTGR_LAUNCH_CHECK();
  }
  const bool train = a.train;
  if (a.n_cand > 0) {
    // hidden layer: Z1 = Xc W1^T + b1 (kept), H = SiLU(Z1)
    GemmEpiArgs ep = {};
    ep.kind = EPI_BIAS_SILU;
    ep.C = w.hc; ep.ldc = a.h; ep.bias = a.b1; ep.Z = w.z1; ep.ldz = a.h;
    {
      ProfScope ps("head_hidden", st);
      r = launch_gemm(dt, w.xc, a.d, true, a.W1, a.d, true, (int)a.n_cand, a.h, a.d, ep, 1, st);
    }
    if (r) return r;
    ProfScope ps("head_out", st);
    switch (dt) {
      case MTGR_F32: r = head_out_dispatch<float>(a.nt, w, a.W2, a.b2, a.h, a.n_cand, a.labels, a.logits, train, st); break;
      case MTGR_BF16: r = head_out_dispatch<bf16_t>(a.nt, w, a.W2, a.b2, a.h, a.n_cand, a.labels, a.logits, train, st); break;
      default: r = head_out_dispatch<f16_t>(a.nt, w, a.W2, a.b2, a.h, a.n_cand, a.labels, a.logits, train, st); break;
    }
    if (r) return r;
  }
  if (!train) return MTGR_OK;
  // head weight gradients and the loss
  if (a.n_cand > 0) {
    {
      ProfScope ps("head_sums", st);
      switch (dt) {
        case MTGR_F32: r = head_sums<float>(a.nt, w, a.h, a.n_cand, a.dW2, a.db2, a.db1, a.loss, st); break;
        case MTGR_BF16: r = head_sums<bf16_t>(a.nt, w, a.h, a.n_cand, a.dW2, a.db2, a.db1, a.loss, st); break;
        default: r = head_sums<f16_t>(a.nt, w, a.h, a.n_cand, a.dW2, a.db2, a.db1, a.loss, st); break;
      }
    }
    if (r) return r;
    {
      // dW1 = dZ1^T Xc (fp32, split over the candidates)
      ProfScope ps2("head_dW1", st);
      GemmEpiArgs ew = {};
      ew.kind = EPI_F32_ATOMIC;
      ew.C = a.dW1; ew.ldc = a.d;
      r = launch_gemm(dt, w.dz1, a.h, false, w.xc, a.d, false, a.h, a.d, (int)a.n_cand, ew,
                      head_split(a.h, a.d, (int)a.n_cand), st);
      if (r) return r;
    }
    {
      // dXc = dZ1 W1
      ProfScope ps3("head_dX", st);
      GemmEpiArgs ex = {};
      ex.kind = EPI_STORE;
      ex.C = w.dxc; ex.ldc = a.d;
      r = launch_gemm(dt, w.dz1, a.h, true, a.W1, a.d, false, (int)a.n_cand, a.d, a.h, ex, 1, st);
      if (r) return r;
    }
  } else {
    // no candidates: zero loss and gradients
    r = launch_fill_f32(a.dW2, (int64_t)a.nt * a.h, 0.f, st);
    if (!r && a.db2) r = launch_fill_f32(a.db2, a.nt, 0.f, st);
    if (!r) r = launch_fill_f32(a.dW1, (int64_t)a.h * a.d, 0.f, st);
    if (!r && a.db1) r = launch_fill_f32(a.db1, a.h, 0.f, st);
    if (!r) r = launch_fill_f32(a.loss, 1, 0.f, st);
    if (r) return r;
  }
  if (a.T > 0) {
    ProfScope ps("head_expand", st);
    hipLaunchKernelGGL(head_expand_kernel, dim3((unsigned)((a.T + 3) / 4)), dim3(256), 0, st, a.offsets, w.seg,
                       w.cand_off, a.B, a.T, a.n_cand, (const char*)w.dxc, (int)(a.d * e), (char*)a.dx,
                       a.lddx * (int64_t)e);
    MTGR_LAUNCH_CHECK();
  }
  return MTGR_OK;
}

// Split-K of dW1 over the candidates: about one 256 x 256 tile job per
// compute unit, each split at least 256 candidates deep.
int head_split(int M, int N, int K) {
  const int tiles = ((M + 255) / 256) * ((N + 255) / 256);
  int s = (256 + tiles - 1) / tiles;
  const int maxs = K / 256 > 0 ? K / 256 : 1;
  if (s > maxs) s = maxs;
  return s < 1 ? 1 : s;
}

}  // namespace mtgr
