// GEMMs of the layer: the fused UQKV projection with bias + SiLU in the
// epilogue (a3; paper-daily 模型怎么搭: one linear layer followed by SiLU gives
// U, Q, K, V), the output projection with bias + residual (a6), and the
// backward products (data gradients and fp32 weight gradients).
//
// bf16 / f16: 256x256 output tile per 512-thread workgroup, 8 waves in 2x4,
// each wave 128x64 = 4x2 MFMA 32x32x16 tiles; K staged through LDS 64 deep,
// double-buffered, one barrier per K step.  Operands stored K-contiguous are
// read with 16-byte LDS loads; operands stored M/N-contiguous (the transposed
// products of the backward) are read with gfx950's LDS transpose load, so no
// operand is ever transposed in memory.
// f32: a plain LDS-tiled FMA kernel (small parity workloads only).
#include "kernels.h"

namespace mtgr {

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }
// 16-bit outputs: the hardware reciprocal (1 ulp) is far below the output rounding
__device__ __forceinline__ float silu_fast(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Staged epilogue of 8 consecutive outputs (m, n..n+7), N % 8 == 0.
constexpr int G_EPI_PITCH = 72;  // floats per staged row

template <typename T>
__device__ __forceinline__ void load8_t(const T* p, float* o) {
  const uint4 r = *(const uint4*)p;
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = from_bits16<T>((uint16_t)(w[i] & 0xffff));
    o[2 * i + 1] = from_bits16<T>((uint16_t)(w[i] >> 16));
  }
}

template <typename T>
__device__ __forceinline__ void store8_t(T* p, const float* v) {
  uint4 r;
  r.x = pack2<T>(v[0], v[1]);
  r.y = pack2<T>(v[2], v[3]);
  r.z = pack2<T>(v[4], v[5]);
  r.w = pack2<T>(v[6], v[7]);
  *(uint4*)p = r;
}

template <typename T, int EPI>
__device__ __forceinline__ void epi_row8(const GemmEpiArgs& ep, int m, int n, float* v) {
  if (EPI == EPI_BIAS_SILU || EPI == EPI_BIAS_RESID) {
    if (ep.bias) {
      float bb[8];
      load8_t<T>((const T*)ep.bias + n, bb);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += bb[e];
    }
  }
  if (EPI == EPI_BIAS_SILU) {
    float z[8];
    // round z to T first so forward and backward see the same pre-activation
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = to_f32(from_f32<T>(v[e]));
    if (ep.Z) store8_t<T>((T*)ep.Z + (int64_t)m * ep.ldz + n, z);
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = silu_fast(z[e]);
    store8_t<T>((T*)ep.C + (int64_t)m * ep.ldc + n, z);
  } else if (EPI == EPI_BIAS_RESID) {
    float r[8];
    load8_t<T>((const T*)ep.R + (int64_t)m * ep.ldr + n, r);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] += r[e];
    store8_t<T>((T*)ep.C + (int64_t)m * ep.ldc + n, v);
  } else {
    store8_t<T>((T*)ep.C + (int64_t)m * ep.ldc + n, v);
  }
}

template <typename T, int EPI>
__device__ __forceinline__ void epi_apply(const GemmEpiArgs& ep, int m, int n, float acc) {
  if (EPI == EPI_STORE) {
    ((T*)ep.C)[(int64_t)m * ep.ldc + n] = from_f32<T>(acc);
  } else if (EPI == EPI_BIAS_SILU) {
    float z = acc + (ep.bias ? to_f32(((const T*)ep.bias)[n]) : 0.f);
    T zr = from_f32<T>(z);
    if (ep.Z) ((T*)ep.Z)[(int64_t)m * ep.ldz + n] = zr;
    // SiLU of the stored (rounded) pre-activation, so that forward and
    // backward see the same z.
    float zq = to_f32(zr);
    ((T*)ep.C)[(int64_t)m * ep.ldc + n] = from_f32<T>(silu_f(zq));
  } else if (EPI == EPI_BIAS_RESID) {
    float r = acc + (ep.bias ? to_f32(((const T*)ep.bias)[n]) : 0.f) +
              to_f32(((const T*)ep.R)[(int64_t)m * ep.ldr + n]);
    ((T*)ep.C)[(int64_t)m * ep.ldc + n] = from_f32<T>(r);
  } else if (EPI == EPI_F32_STORE) {
    ((float*)ep.C)[(int64_t)m * ep.ldc + n] = acc;
  } else {
    atomicAdd(&((float*)ep.C)[(int64_t)m * ep.ldc + n], acc);
  }
}

// ---------------------------------------------------------------------------
// MFMA kernel: 256 x 256 output tile, 512 threads = 8 waves as 2 (M) x 4 (N),
// each wave 128 x 64 = 4 x 2 MFMA 32x32x16 tiles; K staged 64 deep through
// LDS, double-buffered with register prefetch, one barrier per K step.
// Global reads are buffer loads whose range check zero-fills rows past the
// matrix edge; advancing a K step changes only scalar registers.
// ---------------------------------------------------------------------------
constexpr int G_BM = 256, G_BN = 256, G_BK = 64;
constexpr int G_KC_PITCH = G_BK + 8;    // K-contiguous tile [256][72]
constexpr int G_MN_PITCH = G_BM + 16;   // M/N-contiguous tile [64][272]
constexpr int G_TILE_ELEMS = G_BM * G_KC_PITCH;  // >= G_BK * G_MN_PITCH
static_assert(G_BK * G_MN_PITCH <= G_TILE_ELEMS, "tile size");

// Buffer resource over one operand's K step.  K-contiguous: rows r0.. (the
// M or N index), columns k0..; M/N-contiguous: rows k0.. (the K index),
// columns r0...  Reads beyond the valid rows return zeros.
template <bool KC>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_rsrc(const uint16_t* P, int64_t ld, int r0, int R, int k0,
                                                         int kend) {
  if (KC) return make_rsrc(P + (int64_t)r0 * ld + k0, (int)((int64_t)(R - r0) * ld * 2 - (int64_t)k0 * 2));
  return make_rsrc(P + (int64_t)k0 * ld + r0, (int)((int64_t)(kend - k0) * ld * 2 - (int64_t)r0 * 2));
}

template <bool KC>
__device__ __forceinline__ int gemm_voff(int64_t ld, int c) {
  if (KC) return ((c >> 3) * (int)ld + (c & 7) * 8) * 2;
  return ((c >> 5) * (int)ld + (c & 31) * 8) * 2;
}

template <bool KC>
__device__ __forceinline__ void gemm_swrite(uint16_t* s, int c, uint4 v) {
  if (KC) *(uint4*)(s + (c >> 3) * G_KC_PITCH + (c & 7) * 8) = v;
  else *(uint4*)(s + (c >> 5) * G_MN_PITCH + (c & 31) * 8) = v;
}

// MFMA operand for 32 rows starting at r0 (within the tile), k-step ks.
template <bool KC>
__device__ __forceinline__ op8 gemm_operand(const uint16_t* s, int r0, int ks, int lane) {
  op8 o;
  if (KC) {
    const int row = r0 + (lane & 31), kk = ks * 16 + 8 * (lane >> 5);
    o.v = *(const u32x4_t*)(s + row * G_KC_PITCH + kk);
  } else {
    const int G = lane >> 4, i = lane & 15;
    const int kr = ks * 16 + 8 * (G >> 1) + (i >> 2);
    const int col = r0 + 16 * (G & 1) + 4 * (i & 3);
    uint2 lo = lds_read_tr16(s + kr * G_MN_PITCH + col);
    uint2 hi = lds_read_tr16(s + (kr + 4) * G_MN_PITCH + col);
    o.v[0] = lo.x; o.v[1] = lo.y; o.v[2] = hi.x; o.v[3] = hi.y;
  }
  return o;
}

// Scheduling hint for one K step (four 16-deep slices, eight MFMAs each, R
// LDS reads feeding each slice): the reads of slice s + 1 are spread between
// the MFMAs of slice s, so that operands arrive before they are needed.
template <int R, int I>
__device__ __forceinline__ void gemm_pipeline_slot() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA I of the slice
  constexpr int n = (R * (I + 1)) / 8 - (R * I) / 8;
  if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x100, n, 0);  // DS reads
  if constexpr (I + 1 < 8) gemm_pipeline_slot<R, I + 1>();
}
template <int R>
__device__ __forceinline__ void gemm_pipeline() {
  __builtin_amdgcn_sched_group_barrier(0x100, R, 0);  // DS reads of slice 0
  gemm_pipeline_slot<R, 0>();
  gemm_pipeline_slot<R, 0>();
  gemm_pipeline_slot<R, 0>();
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
}

// Workgroup L -> (row job, N tile).  Workgroups run round-robin on the 8
// XCDs; every N tile of one row job goes to the same XCD so that the A rows
// are fetched once into that XCD's L2.
__device__ __forceinline__ bool gemm_tile_of(int L, int NT, int R, int& rr, int& nt) {
  const int x = L & 7, r = L >> 3;
  nt = r % NT;
  rr = (r / NT) * 8 + x;
  return rr < R;
}

template <typename T, bool AK, bool BKC, int EPI>
__global__ __launch_bounds__(512, 1) void gemm_mfma_kernel(const uint16_t* __restrict__ A, int64_t lda,
                                                           const uint16_t* __restrict__ B, int64_t ldb,
                                                           int M, int N, int K, int k_per_split, int MT,
                                                           int NT, int R, GemmEpiArgs ep) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][2 * G_TILE_ELEMS];
  int rr, nt;
  if (!gemm_tile_of(blockIdx.x, NT, R, rr, nt)) return;
  const int mt = rr % MT, split = rr / MT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int m0 = mt * G_BM, n0 = nt * G_BN;
  const int kbeg = split * k_per_split;
  const int kend = min(K, kbeg + k_per_split);
  const int nk = kend > kbeg ? (kend - kbeg + G_BK - 1) / G_BK : 0;
  if (EPI == EPI_F32_ATOMIC && nk == 0) return;

  f32x16_t acc[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[t][u][j] = 0.f;

  int va[4], vb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    va[i] = gemm_voff<AK>(lda, tid + 512 * i);
    vb[i] = gemm_voff<BKC>(ldb, tid + 512 * i);
  }
  uint4 ra[4], rb[4];
  auto gload = [&](int k0) {
    const __amdgpu_buffer_rsrc_t sa = gemm_rsrc<AK>(A, lda, m0, M, k0, kend);
    const __amdgpu_buffer_rsrc_t sb = gemm_rsrc<BKC>(B, ldb, n0, N, k0, kend);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = buf_load16(sa, va[i]);
      rb[i] = buf_load16(sb, vb[i]);
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gemm_swrite<AK>(smem[buf], tid + 512 * i, ra[i]);
      gemm_swrite<BKC>(smem[buf] + G_TILE_ELEMS, tid + 512 * i, rb[i]);
    }
  };
  if (nk > 0) {
    gload(kbeg);
    swrite(0);
  }
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const int buf = it & 1;
    const bool more = it + 1 < nk;
    if (more) gload(kbeg + (it + 1) * G_BK);
    const uint16_t* sa = smem[buf];
    const uint16_t* sb = smem[buf] + G_TILE_ELEMS;
#pragma unroll
    for (int ks = 0; ks < G_BK / 16; ++ks) {
      op8 a[4], b[2];
#pragma unroll
      for (int t = 0; t < 4; ++t) a[t] = gemm_operand<AK>(sa, wm * 128 + t * 32, ks, lane);
#pragma unroll
      for (int u = 0; u < 2; ++u) b[u] = gemm_operand<BKC>(sb, wn * 64 + u * 32, ks, lane);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u) acc[t][u] = mfma32<T>(a[t], b[u], acc[t][u]);
    }
    gemm_pipeline<4 * (AK ? 1 : 2) + 2 * (BKC ? 1 : 2)>();
    if (more) swrite(buf ^ 1);
    __syncthreads();
  }
  if constexpr (EPI == EPI_F32_STORE || EPI == EPI_F32_ATOMIC) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int m = m0 + wm * 128 + t * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
          const int n = n0 + wn * 64 + u * 32 + (lane & 31);
          if (m < M && n < N) epi_apply<T, EPI>(ep, m, n, acc[t][u][j]);
        }
  } else {
    // 16-bit outputs: stage each wave's tile through its own LDS region (64
    // rows at a time, fp32) and write whole 128-byte row segments.
    float* st = (float*)&smem[0][0] + wave * (64 * G_EPI_PITCH);
    const int wr0 = m0 + wm * 128, wc0 = n0 + wn * 64;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int r = tt * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
            st[r * G_EPI_PITCH + u * 32 + (lane & 31)] = acc[2 * half + tt][u][j];
          }
      // lane -> 8 consecutive columns of one row; 8 rows per pass
      const int cc = (lane & 7) * 8;
      const int n = wc0 + cc;
#pragma unroll
      for (int pass = 0; pass < 8; ++pass) {
        const int r = pass * 8 + (lane >> 3);
        const int m = wr0 + half * 64 + r;
        if (m < M && n < N) {
          float v[8];
          const float4 a = *(const float4*)&st[r * G_EPI_PITCH + cc];
          const float4 b = *(const float4*)&st[r * G_EPI_PITCH + cc + 4];
          v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
          epi_row8<T, EPI>(ep, m, n, v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Plain kernel (f32)
// ---------------------------------------------------------------------------
template <typename T, bool AK, bool BKC, int EPI>
__global__ __launch_bounds__(256) void gemm_simple_kernel(const T* __restrict__ A, int64_t lda,
                                                          const T* __restrict__ B, int64_t ldb, int M,
                                                          int N, int K, int k_per_split,
                                                          GemmEpiArgs ep) {
  __shared__ float As[16][17], Bs[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m = blockIdx.y * 16 + ty, n = blockIdx.x * 16 + tx;
  const int kbeg = blockIdx.z * k_per_split;
  const int kend = min(K, kbeg + k_per_split);
  float acc = 0.f;
  for (int k0 = kbeg; k0 < kend; k0 += 16) {
    const int am = blockIdx.y * 16 + ty, bn = blockIdx.x * 16 + ty, kk = k0 + tx;
    float av = 0.f, bv = 0.f;
    if (am < M && kk < kend) av = to_f32(AK ? A[(int64_t)am * lda + kk] : A[(int64_t)kk * lda + am]);
    if (bn < N && kk < kend) bv = to_f32(BKC ? B[(int64_t)bn * ldb + kk] : B[(int64_t)kk * ldb + bn]);
    As[ty][tx] = av;
    Bs[ty][tx] = bv;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 16; ++q) acc += As[ty][q] * Bs[tx][q];
    __syncthreads();
  }
  if (EPI == EPI_F32_ATOMIC && kend <= kbeg) return;
  if (m < M && n < N) epi_apply<T, EPI>(ep, m, n, acc);
}

template <typename T, bool AK, bool BKC, int EPI>
static void gemm_launch_t(const void* A, int64_t lda, const void* B, int64_t ldb, int M, int N, int K,
                          int splits, const GemmEpiArgs& ep, hipStream_t st) {
  int kps = (K + splits - 1) / splits;
  if constexpr (sizeof(T) == 2) {
    kps = (kps + G_BK - 1) / G_BK * G_BK;
    const int MT = (M + G_BM - 1) / G_BM, NT = (N + G_BN - 1) / G_BN, R = MT * splits;
    const unsigned grid = (unsigned)((R + 7) / 8 * 8 * NT);
    hipLaunchKernelGGL((gemm_mfma_kernel<T, AK, BKC, EPI>), dim3(grid), dim3(512), 0, st, (const uint16_t*)A,
                       lda, (const uint16_t*)B, ldb, M, N, K, kps, MT, NT, R, ep);
  } else {
    dim3 grid((N + 15) / 16, (M + 15) / 16, splits);
    hipLaunchKernelGGL((gemm_simple_kernel<T, AK, BKC, EPI>), grid, dim3(256), 0, st, (const T*)A, lda,
                       (const T*)B, ldb, M, N, K, kps, ep);
  }
}

template <typename T, int EPI>
static void gemm_launch_layout(const void* A, int64_t lda, bool ak, const void* B, int64_t ldb, bool bk,
                               int M, int N, int K, int splits, const GemmEpiArgs& ep, hipStream_t st) {
  if (ak && bk) gemm_launch_t<T, true, true, EPI>(A, lda, B, ldb, M, N, K, splits, ep, st);
  else if (ak && !bk) gemm_launch_t<T, true, false, EPI>(A, lda, B, ldb, M, N, K, splits, ep, st);
  else if (!ak && !bk) gemm_launch_t<T, false, false, EPI>(A, lda, B, ldb, M, N, K, splits, ep, st);
  else gemm_launch_t<T, false, true, EPI>(A, lda, B, ldb, M, N, K, splits, ep, st);
}

template <typename T>
static void gemm_launch_epi(const void* A, int64_t lda, bool ak, const void* B, int64_t ldb, bool bk,
                            int M, int N, int K, int splits, const GemmEpiArgs& ep, hipStream_t st) {
  switch (ep.kind) {
    case EPI_STORE: gemm_launch_layout<T, EPI_STORE>(A, lda, ak, B, ldb, bk, M, N, K, splits, ep, st); break;
    case EPI_BIAS_SILU: gemm_launch_layout<T, EPI_BIAS_SILU>(A, lda, ak, B, ldb, bk, M, N, K, splits, ep, st); break;
    case EPI_BIAS_RESID: gemm_launch_layout<T, EPI_BIAS_RESID>(A, lda, ak, B, ldb, bk, M, N, K, splits, ep, st); break;
    case EPI_F32_STORE: gemm_launch_layout<T, EPI_F32_STORE>(A, lda, ak, B, ldb, bk, M, N, K, splits, ep, st); break;
    default: gemm_launch_layout<T, EPI_F32_ATOMIC>(A, lda, ak, B, ldb, bk, M, N, K, splits, ep, st); break;
  }
}

int launch_gemm(int dt, const void* A, int64_t lda, bool a_kcontig, const void* B, int64_t ldb,
                bool b_kcontig, int M, int N, int K, const GemmEpiArgs& ep, int splits,
                hipStream_t stream) {
  if (M <= 0 || N <= 0) return MTGR_OK;
  if (splits < 1) splits = 1;
  if (ep.kind == EPI_F32_ATOMIC) {
    // split-K partial sums land in a zeroed output
    int r = launch_fill_f32((float*)ep.C, (int64_t)M * ep.ldc, 0.f, stream);
    if (r) return r;
  }
  switch (dt) {
    case MTGR_F32: gemm_launch_epi<float>(A, lda, a_kcontig, B, ldb, b_kcontig, M, N, K, splits, ep, stream); break;
    case MTGR_BF16: gemm_launch_epi<bf16_t>(A, lda, a_kcontig, B, ldb, b_kcontig, M, N, K, splits, ep, stream); break;
    case MTGR_F16: gemm_launch_epi<f16_t>(A, lda, a_kcontig, B, ldb, b_kcontig, M, N, K, splits, ep, stream); break;
    default: return MTGR_ERR_UNSUPPORTED;
  }
  MTGR_LAUNCH_CHECK();
  return MTGR_OK;
}

}  // namespace mtgr
