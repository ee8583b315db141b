// Stochastic Length sampling in front of the training path, and the cut of
// the shortened users to a token budget.
//
// paper-daily "MTGR：美团外卖生成式推荐Scaling Law落地实践", section
// 计算量涨了 65 倍，训练成本怎么压住: training replaces a long user sequence by a
// randomly drawn segment of it (online scoring keeps the full sequence).
// Read here as: the history S of each user keeps a contiguous window of
// s_keep tokens starting at floor(u * (n_s - s_keep + 1)) (float32 product)
// for the user's uniform draw u; profile, real-time and candidate tokens stay.
// Batches are sized by token count (zzxanthony blog 11.3): the training batch
// is the longest prefix of shortened users within the budget.
//
// Two launches after the segment kernel: one workgroup plans (window start
// and new length per user, an exclusive scan into the new offsets, the
// budget cut, and a list of 32-row copy blocks of the users within the
// budget); then one workgroup per block copies its rows (features, group
// id, timestamp) from their source rows.
#include "kernels.h"

namespace mtgr {

constexpr int SL_PLAN_THREADS = 1024;
constexpr int SL_BLK = 32;  // output rows per copy block

__device__ __forceinline__ int sl_window_start(float u, int n_s, int s_keep) {
  const int m = n_s - s_keep;
  if (m <= 0) return 0;
  const float prod = u * (float)(m + 1);
  const int st = (int)floorf(prod);
  return min(max(st, 0), m);
}

// New length of user b and (through *first) its first kept history row.
__device__ __forceinline__ int sl_user_len(const int32_t* seg, const float* u, int b, int s_keep, int* first) {
  const int* s = seg + (int64_t)b * 5;
  const int n_s = s[2] - s[1];
  *first = s[1] + (n_s > s_keep ? sl_window_start(u[b], n_s, s_keep) : 0);
  return (s[1] - s[0]) + min(n_s, s_keep) + (s[4] - s[2]);
}

// Inclusive scan of v over the workgroup's threads (Hillis-Steele in LDS).
__device__ __forceinline__ int sl_block_scan(int v, int32_t* scan) {
  const int tid = threadIdx.x;
  scan[tid] = v;
  __syncthreads();
  for (int off = 1; off < SL_PLAN_THREADS; off <<= 1) {
    const int add = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  const int r = scan[tid];
  __syncthreads();
  return r;
}

// One workgroup.  Pass 1: window start and new length per user, their
// exclusive scan into offsets_out, the budget cut into fit_out.  Pass 2: the
// copy blocks of the fitting users, SL_BLK output rows each:
// blocks[k] = {user, first output row, rows}, and the block count.
__global__ __launch_bounds__(SL_PLAN_THREADS) void sl_plan_kernel(const int32_t* __restrict__ seg,
                                                                  const float* __restrict__ u, int B, int s_keep,
                                                                  int64_t budget, int32_t* __restrict__ starts,
                                                                  int32_t* __restrict__ offsets_out,
                                                                  int64_t* __restrict__ fit_out,
                                                                  int4* __restrict__ blocks,
                                                                  int32_t* __restrict__ nblocks) {
  __shared__ int32_t scan[SL_PLAN_THREADS];
  __shared__ int32_t carry_s, fit_s, fit_tok_s;
  const int tid = threadIdx.x;
  if (tid == 0) {
    carry_s = 0;
    fit_s = 0;
    fit_tok_s = 0;
  }
  __syncthreads();
  for (int b0 = 0; b0 < B; b0 += SL_PLAN_THREADS) {
    const int b = b0 + tid;
    int len = 0, first = 0;
    if (b < B) {
      len = sl_user_len(seg, u, b, s_keep, &first);
      starts[b] = first;
    }
    const int incl = carry_s + sl_block_scan(len, scan);
    if (b < B) {
      offsets_out[b] = incl - len;
      // users b' <= b fit when the tokens through b' stay within the budget
      if ((int64_t)incl <= budget) {
        atomicMax(&fit_s, b + 1);
        atomicMax(&fit_tok_s, incl);
      }
    }
    __syncthreads();
    if (tid == SL_PLAN_THREADS - 1) carry_s = incl;
    __syncthreads();
  }
  const int fit = fit_s;
  if (tid == 0) {
    offsets_out[B] = carry_s;
    fit_out[0] = fit;
    fit_out[1] = fit_tok_s;
  }
  // pass 2 (lengths recomputed from the read-only inputs); blocks[k] =
  // {user, first output row, rows, user position of the first row}
  __syncthreads();
  if (tid == 0) carry_s = 0;
  __shared__ int32_t row_carry_s;
  if (tid == 0) row_carry_s = 0;
  __syncthreads();
  for (int b0 = 0; b0 < fit; b0 += SL_PLAN_THREADS) {
    const int b = b0 + tid;
    int len = 0, first = 0;
    if (b < fit) len = sl_user_len(seg, u, b, s_keep, &first);
    const int nb = (len + SL_BLK - 1) / SL_BLK;
    const int blk_incl = carry_s + sl_block_scan(nb, scan);
    const int row_incl = row_carry_s + sl_block_scan(len, scan);
    if (b < fit) {
      const int k0 = blk_incl - nb, r0 = row_incl - len;
      for (int j = 0; j < nb; ++j)
        blocks[k0 + j] = make_int4(b, r0 + j * SL_BLK, min(SL_BLK, len - j * SL_BLK), j * SL_BLK);
    }
    __syncthreads();
    if (tid == SL_PLAN_THREADS - 1) {
      carry_s = blk_incl;
      row_carry_s = row_incl;
    }
    __syncthreads();
  }
  if (tid == 0) *nblocks = carry_s;
}

// Workgroup k copies block k: up to SL_BLK consecutive output rows of one
// user.  The source row of output position p in the user:
//   p < n_u              : profile row s0 + p
//   p < n_u + keep       : history row first + (p - n_u)
//   else                 : real-time / candidate row s2 + (p - n_u - keep)
// Each thread moves CH 16-byte chunks per round, all loads of a round issued
// before its stores; loads and stores are non-temporal (streamed once, kept
// out of the caches: measured 1.6x faster than cached accesses).
template <int CH>
__global__ __launch_bounds__(256) void sl_copy_kernel(const int32_t* __restrict__ seg,
                                                      const int32_t* __restrict__ starts,
                                                      const int4* __restrict__ blocks,
                                                      const int32_t* __restrict__ nblocks, int s_keep,
                                                      const uint8_t* __restrict__ g, const int64_t* __restrict__ ts,
                                                      const char* __restrict__ x, int64_t ldx_bytes, int row_bytes,
                                                      uint8_t* __restrict__ g_out, int64_t* __restrict__ ts_out,
                                                      char* __restrict__ x_out, int64_t ldo_bytes) {
  if ((int)blockIdx.x >= *nblocks) return;
  const int4 blk = blocks[blockIdx.x];
  const int b = blk.x, r0 = blk.y, nr = blk.z;
  const int* s = seg + (int64_t)b * 5;
  const int s0 = s[0], n_u = s[1] - s[0], s2 = s[2];
  const int keep = min(s[2] - s[1], s_keep);
  const int first = starts[b];
  const int tid = threadIdx.x;
  const int cpr = row_bytes >> 4;            // chunks per row
  const int total = nr * cpr;
  auto src_of = [&](int pos) -> int64_t {
    if (pos < n_u) return s0 + pos;
    if (pos < n_u + keep) return first + (pos - n_u);
    return s2 + (pos - n_u - keep);
  };
  const int pbase = blk.w;  // user position of the block's first row
  for (int c0 = 0; c0 < total; c0 += 256 * CH) {
    u32x4_t v[CH];
    int64_t dst[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = c0 + tid + 256 * i;
      dst[i] = -1;
      if (c < total) {
        const int row = c / cpr, col = (c - row * cpr) << 4;
        v[i] = __builtin_nontemporal_load((const u32x4_t*)(x + src_of(pbase + row) * ldx_bytes + col));
        dst[i] = (int64_t)(r0 + row) * ldo_bytes + col;
      }
    }
#pragma unroll
    for (int i = 0; i < CH; ++i)
      if (dst[i] >= 0) __builtin_nontemporal_store(v[i], (u32x4_t*)(x_out + dst[i]));
  }
  if (tid < nr) {
    const int64_t sr = src_of(pbase + tid);
    g_out[r0 + tid] = g[sr];
    ts_out[r0 + tid] = ts[sr];
  }
}

int64_t sl_max_blocks(int B, int64_t T) { return (T + SL_BLK - 1) / SL_BLK + B; }

size_t sl_workspace_bytes(int B, int64_t T) {
  return align_up((size_t)B * 5 * sizeof(int32_t), 256) + align_up((size_t)B * sizeof(int32_t), 256) + 256 +
         align_up((size_t)sl_max_blocks(B, T) * sizeof(int4), 256);
}

int launch_stochastic_length(const int32_t* offsets, const uint8_t* g, const int64_t* ts, const void* x,
                             int64_t ldx_bytes, int row_bytes, int B, int64_t T, const float* u, int s_keep,
                             int64_t budget, int32_t* offsets_out, uint8_t* g_out, int64_t* ts_out, void* x_out,
                             int64_t ldo_bytes, int64_t* fit_out, void* ws, hipStream_t st) {
  char* w = (char*)ws;
  int32_t* seg = (int32_t*)w;
  w += align_up((size_t)B * 5 * sizeof(int32_t), 256);
  int32_t* starts = (int32_t*)w;
  w += align_up((size_t)B * sizeof(int32_t), 256);
  int32_t* nblocks = (int32_t*)w;
  w += 256;
  int4* blocks = (int4*)w;
  int r = launch_seg_only(offsets, g, B, T, seg, st);
  if (r) return r;
  // never more than T rows fit, whatever the metadata (the output capacity)
  const int64_t cut = budget < T ? budget : T;
  hipLaunchKernelGGL(sl_plan_kernel, dim3(1), dim3(SL_PLAN_THREADS), 0, st, seg, u, B, s_keep, cut, starts,
                     offsets_out, fit_out, blocks, nblocks);
  MTGR_LAUNCH_CHECK();
  if (T <= 0 || B <= 0) return MTGR_OK;
  // at most sl_max_blocks(B, T) blocks; the ones past the count return at once
  hipLaunchKernelGGL(sl_copy_kernel<8>, dim3((unsigned)sl_max_blocks(B, T)), dim3(256), 0, st, seg, starts, blocks,
                     nblocks, s_keep, g, ts, (const char*)x, ldx_bytes, row_bytes, g_out, ts_out, (char*)x_out,
                     ldo_bytes);
  MTGR_LAUNCH_CHECK();
  return MTGR_OK;
}

}  // namespace mtgr
