// a1: jagged segments and the tile work list.
//
// A user row is [U | S | R | C] (blog "MTGR：工业级生成式推荐框架" section 4;
// fun-rec 7.3.1), so with non-decreasing group ids the group starts are
// lower bounds of 1, 2, 3 in the user's slice of group_ids.
#include <stdlib.h>

#include <mutex>

#include "kernels.h"

namespace mtgr {

__device__ __forceinline__ int lower_bound_u8(const uint8_t* g, int lo, int hi, int value) {
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if ((int)g[mid] < value) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Row [lo, hi) of user b, clamped into [0, T]: offsets outside the contract
// (decreasing, negative, past T) then give wrong rows but never rows outside
// the batch, so no later kernel indexes outside its buffers.
__device__ __forceinline__ void user_rows(const int32_t* __restrict__ offsets, int b, int64_t T, int& lo, int& hi) {
  const int t = (int)T;
  lo = min(max(offsets[b], 0), t);
  hi = min(max(offsets[b + 1], lo), t);
}

__global__ void seg_kernel(const int32_t* __restrict__ offsets, const uint8_t* __restrict__ g,
                           int B, int64_t T, int32_t* __restrict__ seg) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int lo, hi;
  user_rows(offsets, b, T, lo, hi);
  seg[b * 5 + 0] = lo;
  seg[b * 5 + 1] = lower_bound_u8(g, lo, hi, 1);
  seg[b * 5 + 2] = lower_bound_u8(g, lo, hi, 2);
  seg[b * 5 + 3] = lower_bound_u8(g, lo, hi, 3);
  seg[b * 5 + 4] = hi;
}

// Everything the attention launches need, in one workgroup: segments of
// every user, the 128-row tile list (longest users first) and the
// exclusive prefix of n_t^2.  Per-user values are recomputed where needed
// rather than kept, so any B works with fixed shared memory.  Group ids of
// batches up to PREP_G_LDS tokens are first copied to LDS, so that the
// binary searches for the group starts wait on LDS rather than on a chain
// of dependent global loads.
constexpr int PREP_G_LDS = 128 * 1024;
static_assert(ATTN_QTILE == 128 && ATTN_KTILE == 128, "query and key tile lists are one list");

__global__ __launch_bounds__(1024) void prep_all_kernel(const int32_t* __restrict__ offsets,
                                                        const uint8_t* __restrict__ g, int B,
                                                        int32_t* __restrict__ seg,
                                                        int32_t* __restrict__ order_scratch,
                                                        int2* __restrict__ tiles, int32_t* __restrict__ ntiles,
                                                        int64_t* __restrict__ tprefix, int64_t T,
                                                        int64_t tile_cap) {
  __shared__ int hist[1024];
  __shared__ int warp_i[16];
  __shared__ long long warp_l[16];
  __shared__ int carry_i;
  __shared__ long long carry_l;
  __shared__ __attribute__((aligned(16))) uint8_t gs[PREP_G_LDS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool in_lds = T <= PREP_G_LDS;
  hist[tid] = 0;
  if (in_lds) {
    if (((uintptr_t)g & 15) == 0) {
      for (int i = 16 * tid; i < T; i += 16 * 1024) {
        if (i + 16 <= T) *(uint4*)(gs + i) = *(const uint4*)(g + i);
        else for (int j = i; j < T; ++j) gs[j] = g[j];
      }
    } else {
      for (int i = tid; i < T; i += 1024) gs[i] = g[i];
    }
  }
  __syncthreads();
  // segments and the histogram of tile counts
  const uint8_t* gsrc = in_lds ? (const uint8_t*)gs : g;
  for (int b = tid; b < B; b += 1024) {
    int lo, hi;
    user_rows(offsets, b, T, lo, hi);
    seg[b * 5 + 0] = lo;
    seg[b * 5 + 1] = lower_bound_u8(gsrc, lo, hi, 1);
    seg[b * 5 + 2] = lower_bound_u8(gsrc, lo, hi, 2);
    seg[b * 5 + 3] = lower_bound_u8(gsrc, lo, hi, 3);
    seg[b * 5 + 4] = hi;
    const int c = (hi - lo + 127) / 128;
    atomicAdd(&hist[min(c, 1023)], 1);
  }
  __syncthreads();
  {
    // exclusive prefix over the buckets from the largest count down: thread
    // t holds bucket 1023 - t
    const int c = 1023 - tid;
    const int h = hist[c];
    int v = h;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(v, off, 64);
      if (lane >= off) v += t;
    }
    if (lane == 63) warp_i[w] = v;
    __syncthreads();
    int before = 0;
    for (int k = 0; k < w; ++k) before += warp_i[k];
    hist[c] = before + v - h;
    if (tid == 0) {
      carry_i = 0;
      carry_l = 0;
    }
  }
  __syncthreads();
  for (int b = tid; b < B; b += 1024) {
    int lo, hi;
    user_rows(offsets, b, T, lo, hi);
    const int c = min((hi - lo + 127) / 128, 1023);
    order_scratch[atomicAdd(&hist[c], 1)] = b;
  }
  __syncthreads();
  // tile list in sorted order and the n_t^2 prefix in user order, one
  // 1024-user chunk at a time
  for (int base = 0; base < B; base += 1024) {
    const int i = base + tid;
    const int bs = i < B ? order_scratch[i] : 0;
    int blo = 0, bhi = 0;
    if (i < B) user_rows(offsets, bs, T, blo, bhi);
    const int cnt = (bhi - blo + 127) / 128;
    long long sq = 0;
    if (i < B) {
      int ilo, ihi;
      user_rows(offsets, i, T, ilo, ihi);
      const long long nt = (ihi - ilo + 127) / 128;
      sq = nt * nt;
    }
    int v = cnt;
    long long vl = sq;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(v, off, 64);
      const long long tl = __shfl_up(vl, off, 64);
      if (lane >= off) { v += t; vl += tl; }
    }
    if (lane == 63) { warp_i[w] = v; warp_l[w] = vl; }
    __syncthreads();
    if (tid < 64) {
      int si = tid < 16 ? warp_i[tid] : 0;
      long long sl = tid < 16 ? warp_l[tid] : 0;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const int t = __shfl_up(si, off, 64);
        const long long tl = __shfl_up(sl, off, 64);
        if (tid >= off) { si += t; sl += tl; }
      }
      if (tid < 16) { warp_i[tid] = si; warp_l[tid] = sl; }
    }
    __syncthreads();
    const int excl = carry_i + (w > 0 ? warp_i[w - 1] : 0) + v - cnt;
    const long long exl = carry_l + (w > 0 ? warp_l[w - 1] : 0) + vl - sq;
    if (i < B) {
      const int lo = blo;
      // overlapping rows (offsets outside the contract) could ask for more
      // tiles than the list holds: those are dropped
      for (int t = 0; t < cnt && excl + t < tile_cap; ++t) tiles[excl + t] = make_int2(bs, lo + t * 128);
      tprefix[i] = exl;
    }
    __syncthreads();
    if (tid == 1023) {
      carry_i = excl + cnt;
      carry_l = exl + sq;
    }
    __syncthreads();
  }
  if (tid == 0) {
    *ntiles = (int)min((int64_t)carry_i, tile_cap);
    tprefix[B] = carry_l;
  }
}

int64_t max_tiles(int B, int64_t T, int rows_per_tile) {
  return (T + rows_per_tile - 1) / rows_per_tile + B;
}

size_t prep_workspace_bytes(int B, int64_t T) {
  size_t n = 0;
  n += align_up((size_t)B * 5 * sizeof(int32_t), 256);      // seg
  n += 256;                                                    // tile counts
  n += align_up((size_t)B * sizeof(int32_t), 256);           // order scratch
  n += align_up((size_t)max_tiles(B, T, ATTN_QTILE) * sizeof(int2), 256);
  n += align_up((size_t)max_tiles(B, T, ATTN_KTILE) * sizeof(int2), 256);
  n += align_up((size_t)(B + 1) * sizeof(int64_t), 256);    // dS tile prefix
  return n;
}

int launch_prep(const int32_t* offsets, const uint8_t* group_ids, int B, int64_t T, void* ws,
                hipStream_t stream, PrepView* out) {
  char* p = (char*)ws;
  out->seg = (int32_t*)p;
  p += align_up((size_t)B * 5 * sizeof(int32_t), 256);
  out->q.ntiles = (int32_t*)p;
  out->k.ntiles = (int32_t*)p + 1;
  p += 256;
  int32_t* order = (int32_t*)p;
  p += align_up((size_t)B * sizeof(int32_t), 256);
  out->q.tiles = (int2*)p;
  out->q.max_tiles = max_tiles(B, T, ATTN_QTILE);
  p += align_up((size_t)out->q.max_tiles * sizeof(int2), 256);
  out->k.tiles = (int2*)p;
  out->k.max_tiles = max_tiles(B, T, ATTN_KTILE);
  p += align_up((size_t)out->k.max_tiles * sizeof(int2), 256);
  out->tprefix = (int64_t*)p;
  // query and key tiles are both 128 rows: one list serves both
  out->k.tiles = out->q.tiles;
  out->k.ntiles = out->q.ntiles;
  hipLaunchKernelGGL(prep_all_kernel, dim3(1), dim3(1024), 0, stream, offsets, group_ids, B, out->seg, order,
                     out->q.tiles, out->q.ntiles, out->tprefix, T, out->q.max_tiles);
  MTGR_LAUNCH_CHECK();
  return MTGR_OK;
}

int launch_seg_only(const int32_t* offsets, const uint8_t* group_ids, int B, int64_t T, int32_t* seg,
                    hipStream_t stream) {
  if (B <= 0) return MTGR_OK;
  hipLaunchKernelGGL(seg_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, offsets, group_ids, B, T, seg);
  MTGR_LAUNCH_CHECK();
  return MTGR_OK;
}

// ---------------------------------------------------------------------------
// Validation mode: a device check of the jagged metadata before any other
// launch of an entry point.  The result is one flag word of static device
// memory (bit 0: offsets, bit 1: a group id >= G, bit 2: group ids
// decreasing inside a user, bit 3: a row longer than max_len), read back by
// the host after a stream synchronisation.
// ---------------------------------------------------------------------------
static __device__ __align__(16) uint32_t validate_flag[4];

// True when token t starts a user, i.e. t == offsets[b] for some b in
// [0, B] (binary search; offsets that are not sorted fail the offsets test
// anyway).
__device__ __forceinline__ bool is_user_start(const int32_t* __restrict__ offsets, int B, int64_t t) {
  int lo = 0, hi = B;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)offsets[mid] < t) lo = mid + 1; else hi = mid;
  }
  return (int64_t)offsets[lo] == t;
}

__global__ __launch_bounds__(256) void validate_clear_kernel(uint32_t* flag) {
  if (threadIdx.x == 0) flag[0] = 0;
}

__global__ __launch_bounds__(256) void validate_kernel(const int32_t* __restrict__ offsets,
                                                       const uint8_t* __restrict__ g, int B, int64_t T, int G,
                                                       int ordered, int max_len, uint32_t* flag) {
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t bad = 0;
  if (offsets) {
    for (int64_t b = i0; b <= B; b += stride) {
      const int64_t v = offsets[b];
      if (b == 0 && v != 0) bad |= 1;
      if (b == B && v != T) bad |= 1;
      if (b < B) {
        const int64_t w = offsets[b + 1];
        if (w < v) bad |= 1;
        else if (max_len > 0 && w - v > max_len) bad |= 8;
      }
    }
  }
  for (int64_t t = i0; t < T; t += stride) {
    const int gt = g[t];
    if (gt >= G) bad |= 2;
    if (ordered && t + 1 < T) {
      const int gn = g[t + 1];
      if (gn < gt && !(offsets && is_user_start(offsets, B, t + 1))) bad |= 4;
    }
  }
  if (bad) atomicOr(flag, bad);
}

namespace {
std::mutex g_validate_mu;
int g_validate_on = -1;              // -1: MTGR_VALIDATE not read yet
uint32_t* g_flag_addr[64] = {};      // device address of validate_flag, per device

int validate_state() {
  if (g_validate_on < 0) {
    const char* e = getenv("MTGR_VALIDATE");
    g_validate_on = (e && e[0] && !(e[0] == '0' && e[1] == 0)) ? 1 : 0;
  }
  return g_validate_on;
}
}  // namespace

bool validation_enabled() {
  std::lock_guard<std::mutex> lk(g_validate_mu);
  return validate_state() != 0;
}

void set_validation(int on) {
  std::lock_guard<std::mutex> lk(g_validate_mu);
  g_validate_on = on ? 1 : 0;
}

int validate_jagged(const int32_t* offsets, const uint8_t* group_ids, int B, int64_t T, int G, bool ordered,
                    int max_len, hipStream_t stream) {
  // One validated call at a time per process: the flag word is shared, and
  // each call has synchronised its stream before the lock is released.
  std::lock_guard<std::mutex> lk(g_validate_mu);
  if (!validate_state()) return MTGR_OK;
  if (B <= 0 && T <= 0) return MTGR_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return MTGR_ERR_HIP;
  if (cs != hipStreamCaptureStatusNone) return MTGR_ERR_UNSUPPORTED;  // it synchronises
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MTGR_ERR_HIP;
  if (!g_flag_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(validate_flag)) != hipSuccess || !p) return MTGR_ERR_HIP;
    g_flag_addr[dev] = (uint32_t*)p;
  }
  uint32_t* flag = g_flag_addr[dev];
  hipLaunchKernelGGL(validate_clear_kernel, dim3(1), dim3(64), 0, stream, flag);
  MTGR_LAUNCH_CHECK();
  const int64_t n = (T > B ? T : (int64_t)B + 1);
  const int64_t blocks = (n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048;
  hipLaunchKernelGGL(validate_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, B > 0 ? offsets : nullptr,
                     group_ids, B > 0 ? B : 0, T, G, ordered ? 1 : 0, max_len, flag);
  MTGR_LAUNCH_CHECK();
  uint32_t host = 0;
  if (hipMemcpyAsync(&host, flag, sizeof(host), hipMemcpyDeviceToHost, stream) != hipSuccess) return MTGR_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return MTGR_ERR_HIP;
  return host ? MTGR_ERR_VALIDATION : MTGR_OK;
}

}  // namespace mtgr
