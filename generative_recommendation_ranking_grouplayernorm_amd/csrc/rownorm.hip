// a2 / a5: Group LayerNorm forward and backward, the norm-then-gate step
// GLN2(O) * U, and small reductions (bias gradients, SiLU' products).
//
// Group LayerNorm: fun-rec 7.3.3 formula (x - mu) / sigma * gamma_g + beta_g,
// read as statistics per token over its d features and affine parameters per
// token group (paper-daily 模型怎么搭: each token class has its own norm
// parameters).  The gate order (normalise the aggregate, then multiply by U)
// follows paper-daily 模型怎么搭.
//
// All kernels are HBM-bound row sweeps: one 64-lane wave per token row, 16-byte
// vector accesses, statistics in fp32 from values held in registers.
#include "kernels.h"

namespace mtgr {

// ---- 8-element vector access ---------------------------------------------
__device__ __forceinline__ void load8(const float* p, float* o) {
  float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
template <typename H>
__device__ __forceinline__ void load8_16(const H* p, float* o) {
  uint4 r = *(const uint4*)p;
  uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = from_bits16<H>((uint16_t)(w[i] & 0xffff));
    o[2 * i + 1] = from_bits16<H>((uint16_t)(w[i] >> 16));
  }
}
// Streaming (non-temporal) variant for rows read once: cached reads of them
// push the next kernel's inputs out of the caches.
template <typename H>
__device__ __forceinline__ void load8_16_nt(const H* p, float* o) {
  const u32x4_t r = __builtin_nontemporal_load((const u32x4_t*)p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = from_bits16<H>((uint16_t)(r[i] & 0xffff));
    o[2 * i + 1] = from_bits16<H>((uint16_t)(r[i] >> 16));
  }
}
__device__ __forceinline__ void load8_nt(const float* p, float* o) { load8(p, o); }
__device__ __forceinline__ void load8_nt(const bf16_t* p, float* o) { load8_16_nt(p, o); }
__device__ __forceinline__ void load8_nt(const f16_t* p, float* o) { load8_16_nt(p, o); }
__device__ __forceinline__ void load8(const bf16_t* p, float* o) { load8_16(p, o); }
__device__ __forceinline__ void load8(const f16_t* p, float* o) { load8_16(p, o); }

__device__ __forceinline__ void store8(float* p, const float* v) {
  *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
  *(float4*)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
template <typename H>
__device__ __forceinline__ void store8_16(H* p, const float* v) {
  uint4 r;
  r.x = pack2<H>(v[0], v[1]);
  r.y = pack2<H>(v[2], v[3]);
  r.z = pack2<H>(v[4], v[5]);
  r.w = pack2<H>(v[6], v[7]);
  *(uint4*)p = r;
}
__device__ __forceinline__ void store8(bf16_t* p, const float* v) { store8_16(p, v); }
__device__ __forceinline__ void store8(f16_t* p, const float* v) { store8_16(p, v); }

// 8 consecutive elements held raw in registers (loaded ahead, converted later).
template <typename T> struct Chunk8 {
  uint4 v;
  __device__ __forceinline__ void load(const T* p) { v = *(const uint4*)p; }
  // streaming (non-temporal) read of data used once
  __device__ __forceinline__ void load_nt(const T* p) {
    const u32x4_t r = __builtin_nontemporal_load((const u32x4_t*)p);
    v = make_uint4(r[0], r[1], r[2], r[3]);
  }
  __device__ __forceinline__ void get(float* o) const {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = from_bits16<T>((uint16_t)(w[i] & 0xffff));
      o[2 * i + 1] = from_bits16<T>((uint16_t)(w[i] >> 16));
    }
  }
};
template <> struct Chunk8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *(const float4*)p;
    b = *(const float4*)(p + 4);
  }
  __device__ __forceinline__ void load_nt(const float* p) { load(p); }
  __device__ __forceinline__ void get(float* o) const {
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};

// ---- forward ---------------------------------------------------------------
// NCH = number of 512-column chunks a lane covers (lane owns columns
// lane*8 + 512*i .. +7).
// Sum of partial planes (+ bias, + residual) for the 8 columns c..c+7 of
// row, rounded to T; stored to xs when given.
template <typename T>
__device__ __forceinline__ void partial_row8(const PartialRows& pr, int64_t row, int c, float* v) {
  const float* p = pr.part + row * pr.ldp + c;
  load8(p, v);
  for (int s = 1; s < pr.n; ++s) {
    float w[8];
    load8(p + s * pr.plane, w);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] += w[e];
  }
  if (pr.bias) {
    float b[8];
    load8((const T*)pr.bias + c, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] += b[e];
  }
  if (pr.resid) {
    float r[8];
    load8((const T*)pr.resid + row * pr.ldr + c, r);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] += r[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = to_f32(from_f32<T>(v[e]));
  if (pr.xs) store8((T*)pr.xs + row * pr.ldxs + c, v);
}

// NCH = number of 512-column chunks a lane covers (lane owns columns
// lane*8 + 512*i .. +7).  PART: x comes from fp32 partial sums (pr).
template <typename T, int NCH, bool GATE, bool PART>
__global__ __launch_bounds__(256) void gln_fwd_kernel(
    const T* x, int64_t ldx, T* y, int64_t ldy, const T* __restrict__ gamma,
    const T* __restrict__ beta, const uint8_t* __restrict__ g, int64_t nrows, int d, int G, float eps,
    float* __restrict__ mean_out, float* __restrict__ rstd_out, const T* __restrict__ u, int64_t ldu,
    PartialRows pr) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= nrows) return;
  float v[NCH][8];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane * 8 + i * 512;
    if (c < d) {
      if (PART) partial_row8<T>(pr, row, c, v[i]);
      else load8_nt(x + row * ldx + c, v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[i][e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = 0.f;
    }
  }
  const float inv_d = 1.0f / (float)d;
  const float mean = warp_sum(s) * inv_d;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane * 8 + i * 512;
    if (c < d) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float t = v[i][e] - mean;
        q += t * t;
      }
    }
  }
  const float var = warp_sum(q) * inv_d;
  const float rstd = 1.0f / sqrtf(var + eps);
  // a group id beyond the parameter rows (metadata outside the contract)
  // takes the last row: never a read past gamma / beta
  const int grp = min((int)g[row], G - 1);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane * 8 + i * 512;
    if (c < d) {
      float ga[8], be[8], out[8];
      load8(gamma + (int64_t)grp * d + c, ga);
      load8(beta + (int64_t)grp * d + c, be);
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = (v[i][e] - mean) * rstd * ga[e] + be[e];
      if (GATE) {
        float uu[8];
        load8_nt(u + row * ldu + c, uu);
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] *= uu[e];
      }
      store8(y + row * ldy + c, out);
    }
  }
  if (lane == 0 && mean_out) {
    mean_out[row] = mean;
    rstd_out[row] = rstd;
  }
}

template <typename T, bool GATE, bool PART>
static int gln_fwd_dispatch(const void* x, int64_t ldx, void* y, int64_t ldy, const void* gamma,
                            const void* beta, const uint8_t* g, int64_t T_, int d, int G, float eps,
                            float* mean, float* rstd, const void* u, int64_t ldu, const PartialRows& pr,
                            hipStream_t st) {
  dim3 grid((unsigned)((T_ + 3) / 4)), block(256);
  const int nch = (d + 511) / 512;
  const int n = nch <= 2 ? nch : nch <= 4 ? 4 : nch <= 8 ? 8 : 16;
#define GLN_FWD_CASE(N)                                                                                 \
  case N:                                                                                               \
    hipLaunchKernelGGL((gln_fwd_kernel<T, N, GATE, PART>), grid, block, 0, st, (const T*)x, ldx, (T*)y, \
                       ldy, (const T*)gamma, (const T*)beta, g, T_, d, G, eps, mean, rstd, (const T*)u, ldu, \
                       pr);                                                                             \
    break;
  switch (n) {
    GLN_FWD_CASE(1)
    GLN_FWD_CASE(2)
    GLN_FWD_CASE(4)
    GLN_FWD_CASE(8)
    default: GLN_FWD_CASE(16)
  }
#undef GLN_FWD_CASE
  MTGR_LAUNCH_CHECK();
  return MTGR_OK;
}

template <typename T>
__global__ __launch_bounds__(256) void partial_reduce_kernel(PartialRows pr, int64_t nrows, int d) {
  const int cpr = d / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= nrows * cpr) return;
  float v[8];
  partial_row8<T>(pr, idx / cpr, (int)(idx % cpr) * 8, v);
}

int launch_partial_reduce(int dt, const PartialRows& in, int64_t T_, int d, hipStream_t stream) {
  if (T_ <= 0) return MTGR_OK;
  if (!in.xs || !in.part || in.n < 1 || d % 8) return MTGR_ERR_INVALID_ARG;
  const int64_t n = T_ * (d / 8);
  const dim3 grid((unsigned)((n + 255) / 256));
  switch (dt) {
    case MTGR_F32: hipLaunchKernelGGL(partial_reduce_kernel<float>, grid, dim3(256), 0, stream, in, T_, d); break;
    case MTGR_BF16: hipLaunchKernelGGL(partial_reduce_kernel<bf16_t>, grid, dim3(256), 0, stream, in, T_, d); break;
    case MTGR_F16: hipLaunchKernelGGL(partial_reduce_kernel<f16_t>, grid, dim3(256), 0, stream, in, T_, d); break;
    default: return MTGR_ERR_UNSUPPORTED;
  }
  MTGR_LAUNCH_CHECK();
  return MTGR_OK;
}

int launch_gln_fwd(int dt, const void* x, int64_t ldx, void* y, int64_t ldy, const void* gamma,
                   const void* beta, const uint8_t* g, int64_t T_, int d, int G, float eps, float* mean,
                   float* rstd, const void* u, int64_t ldu, hipStream_t stream) {
  if (T_ <= 0) return MTGR_OK;
  const bool gate = u != nullptr;
  const PartialRows none = {};
#define GLN_FWD_DT(TY)                                                                                        \
  return gate ? gln_fwd_dispatch<TY, true, false>(x, ldx, y, ldy, gamma, beta, g, T_, d, G, eps, mean, rstd, \
                                                  u, ldu, none, stream)                                      \
              : gln_fwd_dispatch<TY, false, false>(x, ldx, y, ldy, gamma, beta, g, T_, d, G, eps, mean, rstd, \
                                                   u, ldu, none, stream);
  switch (dt) {
    case MTGR_F32: GLN_FWD_DT(float)
    case MTGR_BF16: GLN_FWD_DT(bf16_t)
    case MTGR_F16: GLN_FWD_DT(f16_t)
  }
#undef GLN_FWD_DT
  return MTGR_ERR_UNSUPPORTED;
}

int launch_gln_fwd_part(int dt, const PartialRows& in, void* y, int64_t ldy, const void* gamma, const void* beta,
                        const uint8_t* g, int64_t T_, int d, int G, float eps, float* mean, float* rstd,
                        const void* u, int64_t ldu, hipStream_t stream) {
  if (T_ <= 0) return MTGR_OK;
  if (!in.part || in.n < 1) return MTGR_ERR_INVALID_ARG;
  const bool gate = u != nullptr;
#define GLN_FWD_DT(TY)                                                                                             \
  return gate ? gln_fwd_dispatch<TY, true, true>(nullptr, 0, y, ldy, gamma, beta, g, T_, d, G, eps, mean, rstd, u, \
                                                 ldu, in, stream)                                                     \
              : gln_fwd_dispatch<TY, false, true>(nullptr, 0, y, ldy, gamma, beta, g, T_, d, G, eps, mean, rstd, u, \
                                                  ldu, in, stream);
  switch (dt) {
    case MTGR_F32: GLN_FWD_DT(float)
    case MTGR_BF16: GLN_FWD_DT(bf16_t)
    case MTGR_F16: GLN_FWD_DT(f16_t)
  }
#undef GLN_FWD_DT
  return MTGR_ERR_UNSUPPORTED;
}

// ---- backward ---------------------------------------------------------------
// The grid is sized to the blocks the GPU holds at once (one round, no tail),
// each block taking an equal share of the rows, 4 waves x consecutive rows.
// Partial gamma/beta sums: one [2][G][d] slice per block, at most
// GLN_BWD_MAX_BLOCKS blocks (and never fewer than 16 rows per block).
constexpr int GLN_BWD_MAX_BLOCKS = 2048;
constexpr int GLN_BWD_MIN_ROWS = 16;


// Per block: partial[blockIdx.x][0][G][d] = dgamma part, [1][G][d] = dbeta part.
// Each wave walks 16 consecutive rows; the group rarely changes along them,
// so the per-group sums stay in registers and are flushed to LDS (atomic
// adds) only on a change.
// EXACT: d == 512 NCH, so every lane owns full chunks (no per-lane tests).
template <typename T, int NCH, bool GATE, bool EXACT>
__global__ __launch_bounds__(256) void gln_bwd_kernel(
    const T* __restrict__ dy, int64_t lddy, const T* __restrict__ x, int64_t ldx,
    const float* __restrict__ mean, const float* __restrict__ rstd, const T* __restrict__ gamma,
    const T* __restrict__ beta, const uint8_t* __restrict__ g, int64_t nrows, int d, int G, T* dx,
    int64_t lddx, const T* __restrict__ resid, int64_t ldr, const T* __restrict__ u, int64_t ldu,
    T* du, int64_t lddu, const T* __restrict__ zu, int64_t ldzu, float* __restrict__ partial,
    int64_t rows_per_block) {
  extern __shared__ float acc[];  // [2][G][d]
  const int Gd = G * d;
  for (int i = threadIdx.x; i < 2 * Gd; i += blockDim.x) acc[i] = 0.f;
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t RPW = (rows_per_block + 3) / 4;
  const int64_t blk_end = min((int64_t)(blockIdx.x + 1) * rows_per_block, nrows);
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block + (int64_t)w * RPW;
  const int64_t r1 = min(r0 + RPW, blk_end);
  const float inv_d = 1.0f / (float)d;
  float ag[NCH][8], ab[NCH][8];
#pragma unroll
  for (int i = 0; i < NCH; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) ag[i][e] = ab[i][e] = 0.f;
  int cur = -1;
  auto flush = [&]() {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane * 8 + i * 512;
      if (EXACT || c < d) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          atomicAdd(&acc[cur * d + c + e], ag[i][e]);
          atomicAdd(&acc[Gd + cur * d + c + e], ab[i][e]);
          ag[i][e] = ab[i][e] = 0.f;
        }
      }
    }
  };
  // The streamed inputs of row + 1 are loaded (raw) while row is computed,
  // with non-temporal loads: each is read once, and cached reads of them
  // cost 6-8% of the kernels' time (layer step, same box).
  struct Raw {
    Chunk8<T> x[NCH], dy[NCH], u[NCH], zu[NCH], r[NCH];
    float mu, rs;
    int grp;
  };
  auto load_raw = [&](Raw& R, int64_t row) {
    R.mu = mean[row];
    R.rs = rstd[row];
    R.grp = min((int)g[row], G - 1);  // never an LDS slot past the G groups
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane * 8 + i * 512;
      if (EXACT || c < d) {
        R.x[i].load_nt(x + row * ldx + c);
        R.dy[i].load_nt(dy + row * lddy + c);
        if (GATE) {
          R.u[i].load_nt(u + row * ldu + c);
          if (zu) R.zu[i].load_nt(zu + row * ldzu + c);
        } else if (resid) {
          R.r[i].load_nt(resid + row * ldr + c);
        }
      }
    }
  };
  Chunk8<T> gam[NCH], bet[NCH];  // the current group's gamma / beta, reloaded on a change
  auto process = [&](const Raw& R, int64_t row) {
    const int grp = R.grp;
    if (grp != cur) {
      if (cur >= 0) flush();
      cur = grp;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = lane * 8 + i * 512;
        if (EXACT || c < d) {
          gam[i].load(gamma + (int64_t)grp * d + c);
          if (GATE) bet[i].load(beta + (int64_t)grp * d + c);
        }
      }
    }
    const float mu = R.mu, rs = R.rs;
    float n[NCH][8], e[NCH][8];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane * 8 + i * 512;
      if (EXACT || c < d) {
        float dyv[8], ga[8];
        R.x[i].get(n[i]);
        R.dy[i].get(dyv);
        gam[i].get(ga);
#pragma unroll
        for (int k = 0; k < 8; ++k) n[i][k] = (n[i][k] - mu) * rs;
        if (GATE) {
          float uu[8], be[8], duv[8];
          R.u[i].get(uu);
          bet[i].get(be);
#pragma unroll
          for (int k = 0; k < 8; ++k) duv[k] = dyv[k] * (n[i][k] * ga[k] + be[k]);
          if (zu) {
            float gg[8];  // SiLU'(z_u)
            R.zu[i].get(gg);
#pragma unroll
            for (int k = 0; k < 8; ++k) duv[k] *= gg[k];
          }
          store8(du + row * lddu + c, duv);
#pragma unroll
          for (int k = 0; k < 8; ++k) dyv[k] *= uu[k];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          ag[i][k] += dyv[k] * n[i][k];
          ab[i][k] += dyv[k];
          e[i][k] = dyv[k] * ga[k];
          s1 += e[i][k];
          s2 += e[i][k] * n[i][k];
        }
      }
    }
    s1 = warp_sum(s1) * inv_d;
    s2 = warp_sum(s2) * inv_d;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane * 8 + i * 512;
      if (EXACT || c < d) {
        float out[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) out[k] = rs * (e[i][k] - s1 - n[i][k] * s2);
        if (!GATE && resid) {
          float rv[8];
          R.r[i].get(rv);
#pragma unroll
          for (int k = 0; k < 8; ++k) out[k] += rv[k];
        }
        store8(dx + row * lddx + c, out);
      }
    }
  };
  // three row buffers used in turn (no loaded register is ever copied): the
  // rows two and three ahead are in flight while a row is computed
  Raw ra, rb, rc;
  if (r0 < r1) load_raw(ra, r0);
  if (r0 + 1 < r1) load_raw(rb, r0 + 1);
  for (int64_t row = r0; row < r1; row += 3) {
    if (row + 2 < r1) load_raw(rc, row + 2);
    process(ra, row);
    if (row + 1 >= r1) break;
    if (row + 3 < r1) load_raw(ra, row + 3);
    process(rb, row + 1);
    if (row + 2 >= r1) break;
    if (row + 4 < r1) load_raw(rb, row + 4);
    process(rc, row + 2);
  }
  if (cur >= 0) flush();
  __syncthreads();
  float* dst = partial + (int64_t)blockIdx.x * 2 * Gd;
  for (int i = threadIdx.x; i < 2 * Gd; i += blockDim.x) dst[i] = acc[i];
}

// out[i] = sum over nparts of partial[p][i], i < n, then split into
// out_a = out[0 .. na), out_b = out[na .. n).  64 columns per workgroup,
// 16 groups of parts summed in parallel and combined through LDS.
__global__ __launch_bounds__(1024) void reduce_partials_kernel(const float* __restrict__ partial, int nparts, int n,
                                                               float* __restrict__ out_a, float* __restrict__ out_b,
                                                               int na) {
  __shared__ float red[16][65];
  const int cl = threadIdx.x & 63, rg = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + cl;
  float s = 0.f;
  if (i < n) {
#pragma unroll 8
    for (int p = rg; p < nparts; p += 16) s += partial[(int64_t)p * n + i];
  }
  red[rg][cl] = s;
  __syncthreads();
  if (rg != 0 || i >= n) return;
  float t = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) t += red[r][cl];
  if (i < na) {
    if (out_a) out_a[i] = t;
  } else if (out_b) {
    out_b[i - na] = t;
  }
}

static int64_t gln_bwd_block_bound(int64_t T_) {
  const int64_t b = (T_ + GLN_BWD_MIN_ROWS - 1) / GLN_BWD_MIN_ROWS;
  return b < 1 ? 1 : (b > GLN_BWD_MAX_BLOCKS ? GLN_BWD_MAX_BLOCKS : b);
}

size_t gln_bwd_workspace_bytes(int64_t T_, int d, int G) {
  return align_up((size_t)gln_bwd_block_bound(T_) * 2 * G * d * sizeof(float), 256);
}

// Compute units of the current device (cached per device).
static int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

template <typename T, bool GATE>
static int gln_bwd_dispatch(const void* dy, int64_t lddy, const void* x, int64_t ldx, const float* mean,
                            const float* rstd, const void* gamma, const void* beta, const uint8_t* g,
                            int64_t T_, int d, int G, void* dx, int64_t lddx, const void* resid,
                            int64_t ldr, const void* u, int64_t ldu, void* du, int64_t lddu,
                            const void* zu, int64_t ldzu, float* partial, int* nparts, hipStream_t st) {
  const size_t lds = (size_t)2 * G * d * sizeof(float);
  const int nch = (d + 511) / 512;
  const int N = nch <= 1 ? 1 : nch <= 2 ? 2 : nch <= 4 ? 4 : 8;
  const bool exact = d == N * 512;
  using KernelFn = decltype(&gln_bwd_kernel<T, 1, GATE, true>);
#define GLN_BWD_SEL(NN) (exact ? (KernelFn)gln_bwd_kernel<T, NN, GATE, true> : (KernelFn)gln_bwd_kernel<T, NN, GATE, false>)
  const KernelFn fn = N == 1 ? GLN_BWD_SEL(1) : N == 2 ? GLN_BWD_SEL(2) : N == 4 ? GLN_BWD_SEL(4) : GLN_BWD_SEL(8);
#undef GLN_BWD_SEL
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)fn, 256, lds) != hipSuccess || per_cu < 1)
    per_cu = 1;
  int64_t nblk = (int64_t)per_cu * device_cu_count();
  const int64_t bound = gln_bwd_block_bound(T_);
  if (nblk > bound) nblk = bound;
  const int64_t rpb = (T_ + nblk - 1) / nblk;
  nblk = (T_ + rpb - 1) / rpb;
  *nparts = (int)nblk;
  const T* dyp = (const T*)dy;
  const T* xp = (const T*)x;
  hipLaunchKernelGGL(fn, dim3((unsigned)nblk), dim3(256), lds, st, dyp, lddy, xp, ldx, mean, rstd,
                     (const T*)gamma, (const T*)beta, g, T_, d, G, (T*)dx, lddx, (const T*)resid, ldr,
                     (const T*)u, ldu, (T*)du, lddu, (const T*)zu, ldzu, partial, rpb);
  MTGR_LAUNCH_CHECK();
  return MTGR_OK;
}

int launch_gln_bwd(int dt, const void* dy, int64_t lddy, const void* x, int64_t ldx, const float* mean,
                   const float* rstd, const void* gamma, const void* beta, const uint8_t* g,
                   int64_t T_, int d, int G, void* dx, int64_t lddx, const void* resid,
                   int64_t ldr, const void* u, int64_t ldu, void* du, int64_t lddu,
                   const void* zu, int64_t ldzu, float* dgamma, float* dbeta, void* ws,
                   hipStream_t stream) {
  const int Gd = G * d;
  if (T_ <= 0) {
    if (dgamma) { int r = launch_fill_f32(dgamma, Gd, 0.f, stream); if (r) return r; }
    if (dbeta) { int r = launch_fill_f32(dbeta, Gd, 0.f, stream); if (r) return r; }
    return MTGR_OK;
  }
  float* partial = (float*)ws;
  const bool gate = u != nullptr;
  int r = MTGR_ERR_UNSUPPORTED;
  int nparts = 0;
#define GLN_BWD_CALL(TT, GG)                                                                         \
  gln_bwd_dispatch<TT, GG>(dy, lddy, x, ldx, mean, rstd, gamma, beta, g, T_, d, G, dx, lddx, resid, \
                           ldr, u, ldu, du, lddu, zu, ldzu, partial, &nparts, stream)
  switch (dt) {
    case MTGR_F32: r = gate ? GLN_BWD_CALL(float, true) : GLN_BWD_CALL(float, false); break;
    case MTGR_BF16: r = gate ? GLN_BWD_CALL(bf16_t, true) : GLN_BWD_CALL(bf16_t, false); break;
    case MTGR_F16: r = gate ? GLN_BWD_CALL(f16_t, true) : GLN_BWD_CALL(f16_t, false); break;
  }
#undef GLN_BWD_CALL
  if (r) return r;
  hipLaunchKernelGGL(reduce_partials_kernel, dim3((2 * Gd + 63) / 64), dim3(1024), 0, stream, partial,
                     nparts, 2 * Gd, dgamma, dbeta, Gd);
  MTGR_LAUNCH_CHECK();
  return MTGR_OK;
}

// ---- small helpers ----------------------------------------------------------
__global__ void fill_f32_kernel(float* p, int64_t n, float v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

int launch_fill_f32(float* p, int64_t n, float v, hipStream_t stream) {
  if (n <= 0) return MTGR_OK;
  hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n, v);
  MTGR_LAUNCH_CHECK();
  return MTGR_OK;
}

constexpr int COLSUM_ROWS = 256;

template <typename T>
__global__ void colsum_partial_kernel(const T* __restrict__ X, int64_t ldx, int64_t nrows, int N,
                                      float* __restrict__ partial) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= N) return;
  const int64_t r0 = (int64_t)blockIdx.y * COLSUM_ROWS;
  const int64_t r1 = r0 + COLSUM_ROWS < nrows ? r0 + COLSUM_ROWS : nrows;
  float s = 0.f;
  for (int64_t r = r0; r < r1; ++r) s += to_f32(X[r * ldx + c]);
  partial[(int64_t)blockIdx.y * N + c] = s;
}

size_t colsum_workspace_bytes(int64_t T_, int N) {
  const int64_t nb = (T_ + COLSUM_ROWS - 1) / COLSUM_ROWS;
  return align_up((size_t)(nb > 0 ? nb : 1) * N * sizeof(float), 256);
}

int launch_colsum(int dt, const void* X, int64_t ldx, int64_t T_, int N, float* out, void* ws,
                  hipStream_t stream) {
  if (T_ <= 0) return launch_fill_f32(out, N, 0.f, stream);
  const int nb = (int)((T_ + COLSUM_ROWS - 1) / COLSUM_ROWS);
  float* partial = (float*)ws;
  dim3 grid((N + 255) / 256, nb);
  switch (dt) {
    case MTGR_F32: hipLaunchKernelGGL(colsum_partial_kernel<float>, grid, dim3(256), 0, stream, (const float*)X, ldx, T_, N, partial); break;
    case MTGR_BF16: hipLaunchKernelGGL(colsum_partial_kernel<bf16_t>, grid, dim3(256), 0, stream, (const bf16_t*)X, ldx, T_, N, partial); break;
    case MTGR_F16: hipLaunchKernelGGL(colsum_partial_kernel<f16_t>, grid, dim3(256), 0, stream, (const f16_t*)X, ldx, T_, N, partial); break;
    default: return MTGR_ERR_UNSUPPORTED;
  }
  MTGR_LAUNCH_CHECK();
  hipLaunchKernelGGL(reduce_partials_kernel, dim3((N + 63) / 64), dim3(1024), 0, stream, partial, nb, N,
                     out, (float*)nullptr, N);
  MTGR_LAUNCH_CHECK();
  return MTGR_OK;
}

// x *= g elementwise (g: the saved SiLU derivative)
template <typename T>
__global__ void silu_grad_mul_kernel(T* x, int64_t ldx, const T* __restrict__ g, int64_t ldg,
                                     int64_t nrows, int N) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = nrows * (int64_t)N;
  if (i >= total) return;
  const int64_t r = i / N;
  const int c = (int)(i - r * N);
  x[r * ldx + c] = from_f32<T>(to_f32(x[r * ldx + c]) * to_f32(g[r * ldg + c]));
}

int launch_silu_grad_mul(int dt, void* x, int64_t ldx, const void* z, int64_t ldz, int64_t T_, int N,
                         hipStream_t stream) {
  const int64_t total = T_ * (int64_t)N;
  if (total <= 0) return MTGR_OK;
  dim3 grid((unsigned)((total + 255) / 256));
  switch (dt) {
    case MTGR_F32: hipLaunchKernelGGL(silu_grad_mul_kernel<float>, grid, dim3(256), 0, stream, (float*)x, ldx, (const float*)z, ldz, T_, N); break;
    case MTGR_BF16: hipLaunchKernelGGL(silu_grad_mul_kernel<bf16_t>, grid, dim3(256), 0, stream, (bf16_t*)x, ldx, (const bf16_t*)z, ldz, T_, N); break;
    case MTGR_F16: hipLaunchKernelGGL(silu_grad_mul_kernel<f16_t>, grid, dim3(256), 0, stream, (f16_t*)x, ldx, (const f16_t*)z, ldz, T_, N); break;
    default: return MTGR_ERR_UNSUPPORTED;
  }
  MTGR_LAUNCH_CHECK();
  return MTGR_OK;
}

}  // namespace mtgr
