// a1: jagged segments and the tile work list.
//
// A user row is [U | S | R | C] (blog "MTGR：工业级生成式推荐框架" section 4;
// fun-rec 7.3.1), so with non-decreasing group ids the group starts are
// lower bounds of 1, 2, 3 in the user's slice of group_ids.
#include "kernels.h"

namespace mtgr {

__device__ __forceinline__ int lower_bound_u8(const uint8_t* g, int lo, int hi, int value) {
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if ((int)g[mid] < value) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__global__ void seg_kernel(const int32_t* __restrict__ offsets, const uint8_t* __restrict__ g,
                           int B, int32_t* __restrict__ seg) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int lo = offsets[b], hi = offsets[b + 1];
  seg[b * 5 + 0] = lo;
  seg[b * 5 + 1] = lower_bound_u8(g, lo, hi, 1);
  seg[b * 5 + 2] = lower_bound_u8(g, lo, hi, 2);
  seg[b * 5 + 3] = lower_bound_u8(g, lo, hi, 3);
  seg[b * 5 + 4] = hi;
}

// One workgroup: exclusive scan of per-user tile counts, then every user
// writes (user, first row) of each of its ROWS_PER_TILE-row tiles.  The
// list is ordered by descending user length so that the longest rows start
// first (a longest-processing-time-first schedule across the workgroups).
__global__ __launch_bounds__(1024) void tile_list_kernel(const int32_t* __restrict__ offsets, int B,
                                                         int rows_per_tile,
                                                         int32_t* __restrict__ order_scratch,
                                                         int2* __restrict__ tiles,
                                                         int32_t* __restrict__ ntiles) {
  __shared__ int warp_sums[16];
  __shared__ int carry;
  const int tid = threadIdx.x;
  // Counting sort of users by tile count, descending.  Tile counts are
  // bounded by the longest row / rows_per_tile; bucket at that granularity.
  __shared__ int hist[1024];
  for (int i = tid; i < 1024; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  for (int b = tid; b < B; b += blockDim.x) {
    int n = offsets[b + 1] - offsets[b];
    int c = (n + rows_per_tile - 1) / rows_per_tile;
    atomicAdd(&hist[min(c, 1023)], 1);
  }
  __syncthreads();
  if (tid == 0) {
    // exclusive prefix over buckets from the largest count down
    int run = 0;
    for (int c = 1023; c >= 0; --c) {
      int h = hist[c];
      hist[c] = run;
      run += h;
    }
  }
  __syncthreads();
  // Stable placement is not needed: any order inside a bucket is fine.
  for (int b = tid; b < B; b += blockDim.x) {
    int n = offsets[b + 1] - offsets[b];
    int c = min((n + rows_per_tile - 1) / rows_per_tile, 1023);
    int pos = atomicAdd(&hist[c], 1);
    order_scratch[pos] = b;
  }
  __syncthreads();
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < B; base += blockDim.x) {
    int i = base + tid;
    int b = i < B ? order_scratch[i] : 0;
    int cnt = 0;
    if (i < B) {
      int n = offsets[b + 1] - offsets[b];
      cnt = (n + rows_per_tile - 1) / rows_per_tile;
    }
    // block-wide inclusive scan of cnt
    int v = cnt;
    const int lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int t = __shfl_up(v, off, 64);
      if (lane >= off) v += t;
    }
    if (lane == 63) warp_sums[w] = v;
    __syncthreads();
    if (tid < 64) {
      int s = tid < (int)(blockDim.x >> 6) ? warp_sums[tid] : 0;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        int t = __shfl_up(s, off, 64);
        if (tid >= off) s += t;
      }
      if (tid < 16) warp_sums[tid] = s;
    }
    __syncthreads();
    int excl = carry + (w > 0 ? warp_sums[w - 1] : 0) + v - cnt;
    if (i < B) {
      int lo = offsets[b];
      for (int t = 0; t < cnt; ++t) tiles[excl + t] = make_int2(b, lo + t * rows_per_tile);
    }
    __syncthreads();
    if (tid == blockDim.x - 1) carry = excl + cnt;
    __syncthreads();
  }
  if (tid == 0) *ntiles = carry;
}

// One workgroup: exclusive prefix over users (in user order) of n_t^2,
// n_t = ceil(L / 128); out[B] is the total.  n_t^2 is the number of
// 128 x 128 (query, key) tile pairs a user's backward keeps dS for, so the
// prefix places each user's dS tiles in one packed buffer.
__global__ __launch_bounds__(1024) void tile_square_prefix_kernel(const int32_t* __restrict__ offsets, int B,
                                                                  int64_t* __restrict__ out) {
  __shared__ long long warp_sums[16];
  __shared__ long long carry;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < B; base += 1024) {
    const int b = base + tid;
    long long v0 = 0;
    if (b < B) {
      const long long nt = (offsets[b + 1] - offsets[b] + 127) / 128;
      v0 = nt * nt;
    }
    long long v = v0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long t = __shfl_up(v, off, 64);
      if (lane >= off) v += t;
    }
    if (lane == 63) warp_sums[w] = v;
    __syncthreads();
    if (tid < 64) {
      long long s = tid < 16 ? warp_sums[tid] : 0;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const long long t = __shfl_up(s, off, 64);
        if (tid >= off) s += t;
      }
      if (tid < 16) warp_sums[tid] = s;
    }
    __syncthreads();
    const long long excl = carry + (w > 0 ? warp_sums[w - 1] : 0) + v - v0;
    if (b < B) out[b] = excl;
    __syncthreads();
    if (tid == 1023) carry = excl + v0;
    __syncthreads();
  }
  if (tid == 0) out[B] = carry;
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
  if (B > 0) {
    hipLaunchKernelGGL(seg_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, offsets, group_ids, B,
                       out->seg);
    MTGR_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(tile_list_kernel, dim3(1), dim3(1024), 0, stream, offsets, B, ATTN_QTILE, order,
                     out->q.tiles, out->q.ntiles);
  MTGR_LAUNCH_CHECK();
  hipLaunchKernelGGL(tile_list_kernel, dim3(1), dim3(1024), 0, stream, offsets, B, ATTN_KTILE, order,
                     out->k.tiles, out->k.ntiles);
  MTGR_LAUNCH_CHECK();
  hipLaunchKernelGGL(tile_square_prefix_kernel, dim3(1), dim3(1024), 0, stream, offsets, B, out->tprefix);
  MTGR_LAUNCH_CHECK();
  return MTGR_OK;
}

int launch_seg_only(const int32_t* offsets, const uint8_t* group_ids, int B, int32_t* seg,
                    hipStream_t stream) {
  if (B <= 0) return MTGR_OK;
  hipLaunchKernelGGL(seg_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, offsets, group_ids, B, seg);
  MTGR_LAUNCH_CHECK();
  return MTGR_OK;
}

}  // namespace mtgr
