// GEMMs of the layer: the fused UQKV projection with bias + SiLU in the
// epilogue (a3; paper-daily 模型怎么搭: one linear layer followed by SiLU gives
// U, Q, K, V), the output projection with bias + residual (a6), and the
// backward products (data gradients and fp32 weight gradients).
//
// bf16 / f16: 256x256 output tile per 512-thread workgroup, 8 waves in 2x4,
// each wave 128x64 = 4x2 MFMA 32x32x16 tiles (128x128 tiles of 4 waves for
// short batches); K staged through LDS 64 deep by buffer-to-LDS loads,
// double-buffered, one barrier per K step.  Operands stored K-contiguous are
// read with 16-byte LDS loads; operands stored M/N-contiguous (the transposed
// products of the backward) are read with gfx950's LDS transpose load, so no
// operand is ever transposed in memory.
// f32: a plain LDS-tiled FMA kernel (small parity workloads only).
#include "kernels.h"

namespace mtgr {


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

// NT: a streaming (non-temporal) store, for large outputs.
template <typename T, bool NT = false>
__device__ __forceinline__ void store8_t(T* p, const float* v) {
  u32x4_t r;
  r[0] = pack2<T>(v[0], v[1]);
  r[1] = pack2<T>(v[2], v[3]);
  r[2] = pack2<T>(v[4], v[5]);
  r[3] = pack2<T>(v[6], v[7]);
  if constexpr (NT) __builtin_nontemporal_store(r, (u32x4_t*)p);
  else *(u32x4_t*)p = r;
}

// bb: the 8 bias values of columns n..n+7 (zeros without a bias); rr: the
// raw residual row segment (EPI_BIAS_RESID), both loaded by the caller ahead
// of the stores.
template <typename T, int EPI, bool NT>
__device__ __forceinline__ void epi_row8(const GemmEpiArgs& ep, int m, int n, float* v, const float* bb,
                                         const uint4& rr) {
  if ((EPI == EPI_BIAS_SILU || EPI == EPI_BIAS_RESID) && ep.bias) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] += bb[e];
  }
  if (EPI == EPI_BIAS_SILU) {
    float z[8], sg[8];
    // z rounded to T first (two values per conversion), so that SiLU and its
    // derivative are those of the value a consumer of z would see; 16-bit
    // outputs take the hardware reciprocal (1 ulp), far below their rounding
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const uint32_t w = pack2<T>(v[e], v[e + 1]);
      z[e] = from_bits16<T>((uint16_t)(w & 0xffff));
      z[e + 1] = from_bits16<T>((uint16_t)(w >> 16));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sg[e] = __builtin_amdgcn_rcpf(1.0f + __expf(-z[e]));
    if (ep.Z) {
      float zo[8];
      // z itself, or SiLU'(z) = sigma + SiLU(z) (1 - sigma)
#pragma unroll
      for (int e = 0; e < 8; ++e) zo[e] = ep.zgrad ? __builtin_fmaf(z[e] * sg[e], 1.0f - sg[e], sg[e]) : z[e];
      store8_t<T, NT>((T*)ep.Z + (int64_t)m * ep.ldz + n, zo);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] *= sg[e];
    store8_t<T, NT>((T*)ep.C + (int64_t)m * ep.ldc + n, z);
  } else if (EPI == EPI_BIAS_RESID) {
    const uint32_t w[4] = {rr.x, rr.y, rr.z, rr.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] += from_bits16<T>((uint16_t)(w[e] & 0xffff));
      v[2 * e + 1] += from_bits16<T>((uint16_t)(w[e] >> 16));
    }
    store8_t<T, NT>((T*)ep.C + (int64_t)m * ep.ldc + n, v);
  } else {
    store8_t<T, NT>((T*)ep.C + (int64_t)m * ep.ldc + n, v);
  }
}

template <typename T, int EPI>
__device__ __forceinline__ void epi_apply(const GemmEpiArgs& ep, int m, int n, float acc) {
  if (EPI == EPI_STORE) {
    ((T*)ep.C)[(int64_t)m * ep.ldc + n] = from_f32<T>(acc);
  } else if (EPI == EPI_BIAS_SILU) {
    float z = acc + (ep.bias ? to_f32(((const T*)ep.bias)[n]) : 0.f);
    // SiLU (and its derivative) of z rounded to T, the value a consumer of
    // z would see
    const float zq = to_f32(from_f32<T>(z));
    const float sg = 1.0f / (1.0f + __expf(-zq));
    if (ep.Z) ((T*)ep.Z)[(int64_t)m * ep.ldz + n] = from_f32<T>(ep.zgrad ? sg * (1.0f + zq * (1.0f - sg)) : zq);
    ((T*)ep.C)[(int64_t)m * ep.ldc + n] = from_f32<T>(zq * sg);
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
// MFMA kernel.  Output tile BM x BN per workgroup of WAVES_M x WAVES_N waves,
// each wave TM x TN MFMA 32x32x16 tiles; K staged 64 deep through LDS,
// double-buffered, one barrier per K step.  Tiles go from memory straight to
// LDS (buffer loads with the LDS destination), so loading the next K step
// costs the waves no registers and no LDS write instructions: the LDS writes
// happen while the MFMAs of the current step run (writing the tiles from
// registers at the end of each step took 20-30% of the products' time).  The
// range check of the buffer loads zero-fills rows past the matrix edge;
// advancing a K step changes only scalar registers.
//   large: 256 x 256, 8 waves as 2 x 4, 128 x 64 per wave (every batch of
//          more than a few thousand rows);
//   small: 128 x 128, 4 waves as 2 x 2, 64 x 64 per wave, two workgroups per
//          compute unit (forward products of short batches, such as one
//          serving request, where the large tiles would leave most compute
//          units idle).
// ---------------------------------------------------------------------------
constexpr int G_BK = 64;
constexpr int G_KC_PITCH = G_BK + 8;  // K-contiguous rows: 64 + 8 halves

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int MIN_BLOCKS_, bool STREAM_OUT_>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, MIN_BLOCKS = MIN_BLOCKS_;
  // 16-bit outputs stored non-temporally.  The large tiles serve long
  // batches, whose outputs (100 MB and more) would otherwise push the next
  // kernels' inputs out of the 256 MB last-level cache (the UQKV projection
  // of the 65,536-token layer runs 5% faster); the small tiles serve short
  // batches, whose outputs the next kernel reads from the cache.
  static constexpr bool STREAM_OUT = STREAM_OUT_;
  static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
  static constexpr int TM = BM / WAVES_M / 32, TN = BN / WAVES_N / 32;
};
using GemmLarge = GemmCfg<256, 256, 2, 4, 1, true>;
using GemmSmall = GemmCfg<128, 128, 2, 2, 2, false>;

// LDS tile of one operand with ROWS rows (its M or N extent), unpadded rows
// of 16-byte chunks under an XOR swizzle.  K-contiguous: [ROWS][64], chunk c
// (of 8) of row r at c ^ kc_swz(r), so that the 16 rows of a quarter-wave's
// operand read (one chunk each) and the 2 rows x 8 chunks of a quarter-wave's
// write land on distinct bank groups.  M/N-contiguous: [64][ROWS], chunk c of
// K row r at c ^ mn_swz(r), so that a half-wave's transpose read (4 K rows x
// 4 chunks, 8 bytes per lane) covers 16 distinct chunk positions and each of
// its quarter-waves (4 rows x 2 chunks) 8 distinct positions modulo 8.  With
// padded pitches (72 / ROWS + 16 elements) both kinds of reads collided, the
// transposed ones on most accesses.  The allocation keeps the padded size,
// which the epilogue's fp32 staging needs (64 rows x 72 floats per wave,
// NW / 4 waves per tile object).
template <int ROWS>
struct GTile {
  static constexpr int KC_ELEMS = ROWS * G_KC_PITCH;
  static constexpr int MN_ELEMS = G_BK * (ROWS + 16);
  static constexpr int ELEMS = KC_ELEMS > MN_ELEMS ? KC_ELEMS : MN_ELEMS;
};
__device__ __forceinline__ int kc_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int mn_swz(int r) { return (4 * (r & 3)) ^ (r & 2); }

// Buffer resource over one operand's K step.  K-contiguous: rows r0.. (the
// M or N index), columns k0..; M/N-contiguous: rows k0.. (the K index),
// columns r0...  Reads beyond the valid rows return zeros.  A step reads at
// most ROWS (K-contiguous) or G_BK (M/N-contiguous) rows, so the range ends
// there: its byte size fits 32 bits for any number of tokens.
template <bool KC, int ROWS>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_rsrc(const uint16_t* P, int64_t ld, int r0, int R, int k0,
                                                         int kend) {
  if (KC)
    return make_rsrc(P + (int64_t)r0 * ld + k0, (int)((int64_t)min(R - r0, ROWS) * ld * 2 - (int64_t)k0 * 2));
  return make_rsrc(P + (int64_t)k0 * ld + r0, (int)((int64_t)min(kend - k0, G_BK) * ld * 2 - (int64_t)r0 * 2));
}

// Tiles reach LDS by buffer-to-LDS loads: one wave instruction fills 1 KB of
// LDS, lane l's 16 bytes landing at byte 16 l, so the tile's 1 KB block j
// (8 K-contiguous rows, or 1024 / (2 ROWS) M/N-contiguous K rows) is one
// instruction, and the swizzle is applied to the global address each lane
// reads: the lane at LDS chunk position p of row r fetches the row's chunk
// p ^ swz(r).  The byte offset returned is relative to the step's buffer
// resource (gemm_rsrc).
template <bool KC, int ROWS>
__device__ __forceinline__ int gemm_dma_voff(int64_t ld, int j, int lane) {
  constexpr int CPR = KC ? 8 : ROWS / 8;  // 16-byte chunks per LDS row
  constexpr int RPB = 64 / CPR;           // LDS rows per 1 KB block
  const int row = j * RPB + lane / CPR, p = lane % CPR;
  const int ch = p ^ (KC ? kc_swz(row) : mn_swz(row));
  return (row * (int)ld + ch * 8) * 2;
}

__device__ __forceinline__ void gemm_dma16(__amdgpu_buffer_rsrc_t r, uint16_t* lds_block, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_block, 16, voff, 0, 0, 0);
}

// Wait until this wave's buffer-to-LDS loads have written LDS (vmcnt = 0;
// gfx9 encoding with the other counters at their maxima).
__device__ __forceinline__ void gemm_wait_dma() { __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8)); }

// MFMA operand for 32 rows starting at r0 (within the tile), k-step ks.
template <bool KC, int ROWS>
__device__ __forceinline__ op8 gemm_operand(const uint16_t* s, int r0, int ks, int lane) {
  op8 o;
  if (KC) {
    const int row = r0 + (lane & 31), ch = 2 * ks + (lane >> 5);
    o.v = *(const u32x4_t*)(s + row * G_BK + 8 * (ch ^ kc_swz(row)));
  } else {
    const int G = lane >> 4, i = lane & 15;
    const int kr = ks * 16 + 8 * (G >> 1) + (i >> 2);
    const int col = r0 + 16 * (G & 1) + 4 * (i & 3);
    // rows kr and kr + 4 share kr % 4, so both reads use one swizzle
    const uint16_t* p = s + kr * ROWS + 8 * ((col >> 3) ^ mn_swz(kr)) + (col & 7);
    uint2 lo = lds_read_tr16(p);
    uint2 hi = lds_read_tr16(p + 4 * ROWS);
    o.v[0] = lo.x; o.v[1] = lo.y; o.v[2] = hi.x; o.v[3] = hi.y;
  }
  return o;
}

// Scheduling hint for one K step (four 16-deep slices of NM MFMAs each, R
// LDS reads feeding each slice): the reads of slice s + 1 are spread between
// the MFMAs of slice s, so that operands arrive before they are needed.
template <int R, int NM, int I>
__device__ __forceinline__ void gemm_pipeline_slot() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA I of the slice
  constexpr int n = (R * (I + 1)) / NM - (R * I) / NM;
  if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x100, n, 0);  // DS reads
  if constexpr (I + 1 < NM) gemm_pipeline_slot<R, NM, I + 1>();
}
template <int R, int NM>
__device__ __forceinline__ void gemm_pipeline() {
  __builtin_amdgcn_sched_group_barrier(0x100, R, 0);  // DS reads of slice 0
  gemm_pipeline_slot<R, NM, 0>();
  gemm_pipeline_slot<R, NM, 0>();
  gemm_pipeline_slot<R, NM, 0>();
  __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
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

template <typename T, bool AK, bool BKC, int EPI, typename C>
__global__ __launch_bounds__(C::THREADS, C::MIN_BLOCKS) void gemm_mfma_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb, int M, int N, int K,
    int k_per_split, int MT, int NT, int R, GemmEpiArgs ep) {
  constexpr int BM = C::BM, BN = C::BN, TM = C::TM, TN = C::TN, NTH = C::THREADS, NW = NTH / 64;
  constexpr int A_ELEMS = GTile<BM>::ELEMS, B_ELEMS = GTile<BN>::ELEMS;
  // 1 KB buffer-to-LDS blocks per wave and K step
  constexpr int A_LOADS = BM * G_BK * 2 / 1024 / NW, B_LOADS = BN * G_BK * 2 / 1024 / NW;
  static_assert(A_LOADS * NW * 1024 == BM * G_BK * 2 && B_LOADS * NW * 1024 == BN * G_BK * 2, "load split");
  static_assert(TN % 2 == 0 && TM % 2 == 0, "epilogue stages 64 x 64 blocks");
  static_assert(A_ELEMS == B_ELEMS && (NW / 4) * 64 * G_EPI_PITCH * 4 <= A_ELEMS * 2, "epilogue staging fits");
  // The operand tiles of the two K-step buffers are separate LDS objects, so
  // that the compiler can tell the reads of one buffer from the loads in
  // flight into the other and need not wait for those loads before a read.
  __shared__ __attribute__((aligned(16))) uint16_t sa0[A_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t sb0[B_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t sa1[A_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t sb1[B_ELEMS];
  int rr, nt;
  if (!gemm_tile_of(blockIdx.x, NT, R, rr, nt)) return;
  const int mt = rr % MT, split = rr / MT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int m0 = mt * BM, n0 = nt * BN;
  const int kbeg = split * k_per_split;
  const int kend = min(K, kbeg + k_per_split);
  const int nk = kend > kbeg ? (kend - kbeg + G_BK - 1) / G_BK : 0;
  if (EPI == EPI_F32_ATOMIC && nk == 0) return;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int u = 0; u < TN; ++u)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[t][u][j] = 0.f;

  int va[A_LOADS], vb[B_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) va[i] = gemm_dma_voff<AK, BM>(lda, i * NW + wave, lane);
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) vb[i] = gemm_dma_voff<BKC, BN>(ldb, i * NW + wave, lane);
  auto mma = [&](const uint16_t* sa, const uint16_t* sb) {
#pragma unroll
    for (int ks = 0; ks < G_BK / 16; ++ks) {
      op8 a[TM], b[TN];
#pragma unroll
      for (int t = 0; t < TM; ++t) a[t] = gemm_operand<AK, BM>(sa, wm * (TM * 32) + t * 32, ks, lane);
#pragma unroll
      for (int u = 0; u < TN; ++u) b[u] = gemm_operand<BKC, BN>(sb, wn * (TN * 32) + u * 32, ks, lane);
#pragma unroll
      for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int u = 0; u < TN; ++u) acc[t][u] = mfma32<T>(a[t], b[u], acc[t][u]);
    }
    gemm_pipeline<TM * (AK ? 1 : 2) + TN * (BKC ? 1 : 2), TM * TN>();
  };
  // K step at k0 into one buffer (loads in flight until gemm_wait_dma)
  auto dma = [&](uint16_t* s_a, uint16_t* s_b, int k0) {
    const __amdgpu_buffer_rsrc_t sa = gemm_rsrc<AK, BM>(A, lda, m0, M, k0, kend);
    const __amdgpu_buffer_rsrc_t sb = gemm_rsrc<BKC, BN>(B, ldb, n0, N, k0, kend);
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) gemm_dma16(sa, s_a + (i * NW + wave) * 512, va[i]);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) gemm_dma16(sb, s_b + (i * NW + wave) * 512, vb[i]);
  };
  // Step it computes from one buffer while step it + 1 loads into the other
  // (freed by the barrier that ended step it - 1); the loop is unrolled by
  // two so that each half names its buffers statically.
  if (nk > 0) dma(sa0, sb0, kbeg);
  gemm_wait_dma();
  __syncthreads();
  for (int it = 0; it < nk; it += 2) {
    if (it + 1 < nk) dma(sa1, sb1, kbeg + (it + 1) * G_BK);
    mma(sa0, sb0);
    gemm_wait_dma();
    __syncthreads();
    if (it + 1 < nk) {
      if (it + 2 < nk) dma(sa0, sb0, kbeg + (it + 2) * G_BK);
      mma(sa1, sb1);
      gemm_wait_dma();
      __syncthreads();
    }
  }
  if constexpr (EPI == EPI_F32_STORE || EPI == EPI_F32_ATOMIC || EPI == EPI_F32_PLANES) {
    float* planeC = (float*)ep.C + (EPI == EPI_F32_PLANES ? (int64_t)split * ep.plane : 0);
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
      for (int u = 0; u < TN; ++u)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int m = m0 + wm * (TM * 32) + t * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
          const int n = n0 + wn * (TN * 32) + u * 32 + (lane & 31);
          if (m < M && n < N) {
            if (EPI == EPI_F32_PLANES) planeC[(int64_t)m * ep.ldc + n] = acc[t][u][j];
            else epi_apply<T, EPI>(ep, m, n, acc[t][u][j]);
          }
        }
  } else {
    // 16-bit outputs: stage each wave's tile through its own LDS region (64
    // rows at a time, fp32) and write whole 128-byte row segments.  The bias
    // and residual values a lane needs are loaded before any store: the
    // compiler cannot move a load past a store that may alias it, so loads
    // inside the store loop would each wait a full memory round trip.
    const int sq = wave / (NW / 4);
    uint16_t* const sbase = sq == 0 ? sa0 : sq == 1 ? sb0 : sq == 2 ? sa1 : sb1;
    float* st = (float*)sbase + (wave % (NW / 4)) * (64 * G_EPI_PITCH);
    const int wr0 = m0 + wm * (TM * 32), wc0 = n0 + wn * (TN * 32);
    const int cc = (lane & 7) * 8;
    // 64-column blocks of the wave's tile
    float bb[TN / 2][8];
#pragma unroll
    for (int cb = 0; cb < TN / 2; ++cb) {
      const int n = wc0 + cb * 64 + cc;
#pragma unroll
      for (int e = 0; e < 8; ++e) bb[cb][e] = 0.f;
      if ((EPI == EPI_BIAS_SILU || EPI == EPI_BIAS_RESID) && ep.bias && n < N) load8_t<T>((const T*)ep.bias + n, bb[cb]);
    }
#pragma unroll
    for (int cb = 0; cb < TN / 2; ++cb) {
      const int n = wc0 + cb * 64 + cc;
#pragma unroll
      for (int half = 0; half < TM / 2; ++half) {
        uint4 rr[8];
#pragma unroll
        for (int pass = 0; pass < 8; ++pass) {
          rr[pass] = make_uint4(0, 0, 0, 0);
          if (EPI == EPI_BIAS_RESID) {
            const int m = wr0 + half * 64 + pass * 8 + (lane >> 3);
            if (m < M && n < N) {  // read once: non-temporal
            const u32x4_t t = __builtin_nontemporal_load((const u32x4_t*)((const T*)ep.R + (int64_t)m * ep.ldr + n));
            rr[pass] = make_uint4(t[0], t[1], t[2], t[3]);
          }
          }
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int r = tt * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
              st[r * G_EPI_PITCH + u * 32 + (lane & 31)] = acc[2 * half + tt][2 * cb + u][j];
            }
        // lane -> 8 consecutive columns of one row; 8 rows per pass
#pragma unroll
        for (int pass = 0; pass < 8; ++pass) {
          const int r = pass * 8 + (lane >> 3);
          const int m = wr0 + half * 64 + r;
          if (m < M && n < N) {
            float v[8];
            const float4 a = *(const float4*)&st[r * G_EPI_PITCH + cc];
            const float4 b = *(const float4*)&st[r * G_EPI_PITCH + cc + 4];
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
            epi_row8<T, EPI, C::STREAM_OUT>(ep, m, n, v, bb[cb], rr[pass]);
          }
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

template <typename T, bool AK, bool BKC, int EPI, typename C>
static void gemm_launch_cfg(const void* A, int64_t lda, const void* B, int64_t ldb, int M, int N, int K, int kps,
                            int splits, const GemmEpiArgs& ep, hipStream_t st) {
  const int MT = (M + C::BM - 1) / C::BM, NT = (N + C::BN - 1) / C::BN, R = MT * splits;
  const unsigned grid = (unsigned)((R + 7) / 8 * 8 * NT);
  hipLaunchKernelGGL((gemm_mfma_kernel<T, AK, BKC, EPI, C>), dim3(grid), dim3(C::THREADS), 0, st,
                     (const uint16_t*)A, lda, (const uint16_t*)B, ldb, M, N, K, kps, MT, NT, R, ep);
}

// Products whose large-tile grid would not give every compute unit a
// workgroup use the small tiles (only the forward layout, both operands
// K-contiguous, has them).
constexpr int G_SMALL_BELOW = 256;

template <typename T, bool AK, bool BKC, int EPI>
static void gemm_launch_t(const void* A, int64_t lda, const void* B, int64_t ldb, int M, int N, int K,
                          int splits, const GemmEpiArgs& ep, hipStream_t st) {
  int kps = (K + splits - 1) / splits;
  if constexpr (sizeof(T) == 2) {
    kps = (kps + G_BK - 1) / G_BK * G_BK;
    const int64_t large = (int64_t)((M + 255) / 256) * ((N + 255) / 256) * splits;
    if constexpr (AK && BKC) {
      if (large < G_SMALL_BELOW) {
        gemm_launch_cfg<T, AK, BKC, EPI, GemmSmall>(A, lda, B, ldb, M, N, K, kps, splits, ep, st);
        return;
      }
    }
    gemm_launch_cfg<T, AK, BKC, EPI, GemmLarge>(A, lda, B, ldb, M, N, K, kps, splits, ep, st);
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
    case EPI_F32_PLANES: gemm_launch_layout<T, EPI_F32_PLANES>(A, lda, ak, B, ldb, bk, M, N, K, splits, ep, st); break;
    default: gemm_launch_layout<T, EPI_F32_ATOMIC>(A, lda, ak, B, ldb, bk, M, N, K, splits, ep, st); break;
  }
}

int gemm_plane_splits(int M, int N, int K) {
  const int64_t tiles = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
  int s = (int)((256 + tiles - 1) / tiles);
  const int maxs = K / (2 * G_BK);
  if (s > maxs) s = maxs;
  if (s > 4) s = 4;
  return s < 1 ? 1 : s;
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
