// a4 / a7: jagged SiLU attention under MTGR's dynamic mask, forward and
// backward.
//
// Per user b and head h:  O_i = c * sum_j M_ij * SiLU(alpha <q_i, k_j>) v_j,
// no softmax (marovi summary, Métodos; paper-daily 模型怎么搭).  Mask rules
// (fun-rec 7.3.4 rules 1-3; blog section 9): U/S keys are visible to every
// token; a real-time key j is visible to a real-time or candidate query i
// when t_j < t_i, and to itself; a candidate key is visible only to itself.
//
// With the row laid out [U | S | R | C], the mask needs only the segment
// starts and the timestamps: key tiles entirely inside U+S are full (no
// per-element test), static-only query tiles stop at the end of S
// (history -> real-time blocks skipped), candidate keys are visited only by
// query tiles that contain candidates (candidate x candidate blocks skipped
// except for the diagonal), and the per-element test runs in registers.
//
// bf16 / f16 kernels use MFMA 32x32x16.  The score tile is computed
// transposed, S^T = K Q^T, so that each lane holds one query and 16 keys:
// that register layout is directly the A operand of P V (with the K index
// permuted identically on both operands), so P never leaves registers.
// V (and K, Q, dO in the backward) are read as B operands with the LDS
// transpose load.  The backward recomputes S; dK/dV are accumulated per
// key tile (key-major kernel) and dQ per query tile (query-major kernel), so
// no atomics are needed.
#include "kernels.h"

namespace mtgr {

__device__ __forceinline__ float silu_grad_from(float s, float sg) { return sg * (1.0f + s * (1.0f - sg)); }

// Visibility of key kj for query qi inside one user, both absolute token
// indices; s_end = start of R, r_end = start of C, hi = end of the row.
__device__ __forceinline__ bool mask_visible(int qi, int kj, int s_end, int r_end, int hi, int64_t tq,
                                             const int64_t* __restrict__ ts) {
  if (kj < s_end) return true;                                   // U / S key
  if (kj < r_end) return qi >= s_end && (ts[kj] < tq || kj == qi);  // real-time key
  return kj == qi && kj < hi;                                    // candidate key
}

// Same test with both timestamps at hand (tiles keep them in LDS), without
// branches: U/S keys are seen by all; a real-time key by real-time and
// candidate queries with a later timestamp, and by itself; a candidate key
// only by itself.  Rows beyond the user's end carry zero Q/K/V/dO, so their
// products vanish without a test.
__device__ __forceinline__ bool visible_ts(int qi, int kj, int s_end, int r_end, int64_t tq, int64_t tk) {
  const bool rt = qi >= s_end && (tk < tq || kj == qi);
  return kj < s_end || (kj < r_end ? rt : kj == qi);
}

// Key range a query tile [q0, q_last] needs: static queries stop at the end
// of S, real-time queries at the end of R, candidates at themselves.
__device__ __forceinline__ int key_end_for(int q_last, int s_end, int r_end) {
  if (q_last < s_end) return s_end;
  if (q_last < r_end) return r_end;
  return q_last + 1;
}

// The 64-key tiles (counted from the row start lo) that a query tile
// [q0, q_last] visits: every tile up to the end of R, then, for a tile of
// candidates, only the tiles of its own rows: a candidate key is visible
// only to itself, so candidate x candidate blocks off the diagonal are
// skipped.  Visit it (0 <= it < n) is tile tile(it).
struct KeyRuns {
  int na, b0, n;
  __device__ __forceinline__ int tile(int it) const { return it < na ? it : b0 + (it - na); }
};
__device__ __forceinline__ KeyRuns key_runs(int lo, int q0, int q_last, int s_end, int r_end) {
  const int kv_end = key_end_for(q_last, s_end, r_end);
  const int nall = (kv_end - lo + 63) >> 6;
  const int na = min(nall, (min(r_end, kv_end) - lo + 63) >> 6);
  const int b0 = max(na, (max(q0, r_end) - lo) >> 6);
  return {na, b0, na + max(0, nall - b0)};
}

constexpr int A_BQ = 128;  // queries per forward / dQ workgroup (4 waves x 32)
constexpr int A_BK = 64;   // keys per LDS tile (forward / dQ)
constexpr int A_BKW = 128; // keys per dK/dV workgroup (4 waves x 32)
constexpr int A_BQB = 64;  // queries per LDS tile (dK/dV)

template <int DH> struct AttnPitch {
  static constexpr int B128 = DH + 8;   // rows read 16 bytes per lane
  static constexpr int TR = DH + 16;    // rows read with the transpose load
};

// Load a [64 x DH] tile (rows r0.., columns col0..) into registers; rows at or
// beyond rlim read as zero.
template <int DH>
__device__ __forceinline__ void tile_gload(uint4* r, const uint16_t* __restrict__ P, int64_t ld, int r0,
                                           int rlim, int col0, int tid) {
  constexpr int CPR = DH / 8;                 // 16-byte chunks per row
  constexpr int CH = 64 * CPR / 256;          // chunks per thread
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid + 256 * i;
    const int row = c / CPR, col = (c % CPR) * 8;
    const int gr = r0 + row;
    r[i] = gr < rlim ? *(const uint4*)(P + (int64_t)gr * ld + col0 + col) : make_uint4(0, 0, 0, 0);
  }
}
template <int DH, int PITCH>
__device__ __forceinline__ void tile_swrite(uint16_t* s, const uint4* r, int tid) {
  constexpr int CPR = DH / 8;
  constexpr int CH = 64 * CPR / 256;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid + 256 * i;
    const int row = c / CPR, col = (c % CPR) * 8;
    *(uint4*)(s + row * PITCH + col) = r[i];
  }
}

// B operand (column = l32 of a 32-wide column block at col0, 16 K rows
// starting at k16 with the permuted order) read with the transpose load
// from a row-major [rows][PITCH] tile.
template <int PITCH>
__device__ __forceinline__ op8 tr_operand(const uint16_t* s, int k16, int col0, int lane) {
  const int G = lane >> 4, i = lane & 15, g = lane >> 5;
  const int row = k16 + 4 * g + (i >> 2);
  const int col = col0 + 16 * (G & 1) + 4 * (i & 3);
  uint2 lo = lds_read_tr16(s + row * PITCH + col);
  uint2 hi = lds_read_tr16(s + (row + 8) * PITCH + col);
  op8 o;
  o.v[0] = lo.x; o.v[1] = lo.y; o.v[2] = hi.x; o.v[3] = hi.y;
  return o;
}

// A operand: row r0 + l32 of a row-major tile, 8 columns at 16*ks + 8*g.
template <int PITCH>
__device__ __forceinline__ op8 row_operand(const uint16_t* s, int r0, int ks, int lane) {
  op8 o;
  o.v = *(const u32x4_t*)(s + (r0 + (lane & 31)) * PITCH + 16 * ks + 8 * (lane >> 5));
  return o;
}

// Pack accumulator values v[t][j] (t = 32-row subtile, j = MFMA output index)
// into the A operand of k-step u (16 rows 16u..16u+15 of the 64).
template <typename T>
__device__ __forceinline__ op8 pack_kstep(const float (&v)[2][16], int u) {
  const int t = u >> 1, j0 = (u & 1) * 8;
  op8 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o.v[e] = pack2<T>(v[t][j0 + 2 * e], v[t][j0 + 2 * e + 1]);
  return o;
}

// Scheduling hint for a run of N MFMAs each fed by one LDS read: keep AHEAD
// reads in flight ahead of the MFMA that consumes them, so that a wave does
// not stall on LDS latency before every MFMA.  Only orders instructions.
// As pipeline_lds_mfma for NM MFMAs fed by two LDS reads each (transposed
// operands): AHEAD reads first, then one MFMA per two reads.
template <int NM, int AHEAD>
__device__ __forceinline__ void pipeline_lds2_mfma() {
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);  // DS reads
#pragma unroll
  for (int i = 0; i < NM - AHEAD / 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD / 2, 0);
}

template <int N, int AHEAD>
__device__ __forceinline__ void pipeline_lds_mfma() {
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);  // DS reads
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

// ---------------------------------------------------------------------------
// workgroup -> (tile, head), XCD-aware
// ---------------------------------------------------------------------------
// Workgroups are dispatched round-robin over the 8 XCDs (workgroup L runs on
// XCD L % 8), each XCD with its own L2.  Mapping the head to L % 8 puts every
// query tile of one (user, head) on the same XCD, so its K/V rows are fetched
// from HBM once and then served from that XCD's L2.
__device__ __forceinline__ void xcd_tile_head(int L, int H, int& tile, int& head) {
  if ((H & 7) == 0) {
    const int x = L & 7, r = L >> 3, hg = H >> 3;
    head = x + 8 * (r % hg);
    tile = r / hg;
  } else if ((8 % H) == 0) {
    const int x = L & 7, r = L >> 3, per = 8 / H;
    head = x % H;
    tile = r * per + x / H;
  } else {
    head = L % H;
    tile = L / H;
  }
}

inline unsigned xcd_grid(int64_t max_tiles, int H) {
  if ((H & 7) == 0) return (unsigned)(max_tiles * H);
  if ((8 % H) == 0) {
    const int64_t per = 8 / H;
    return (unsigned)(((max_tiles + per - 1) / per) * 8);
  }
  return (unsigned)(max_tiles * H);
}

// Buffer resource over rows [r0, rlim) of a row-major [.., ld] 16-bit array,
// starting at column col0: rows at or beyond rlim read as zero.  The row
// range is wave-uniform, so advancing a tile changes only scalar registers.
// No caller reads more than 128 rows from one resource, so the range stops
// there: its byte size stays a small 32-bit value for any row length.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* P, int64_t ld, int r0, int rlim,
                                                         int col0) {
  return make_rsrc(P + (int64_t)r0 * ld + col0, (int)((int64_t)min(max(rlim - r0, 0), 128) * ld * 2));
}

// Timestamp of token r0 + lane, or 0 at or beyond rlim, as a range-checked
// buffer load: no select on the loaded value, so the load stays in flight
// until the value is used.
__device__ __forceinline__ int64_t ts_load(const int64_t* ts, int r0, int rlim, int lane) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(ts + r0, min(max(rlim - r0, 0), 64) * 8);
  return __builtin_bit_cast(int64_t, __builtin_amdgcn_raw_buffer_load_b64(r, lane * 8, 0, 0));
}

// Tile load: thread chunks c = tid + 256 i, row c / (DH/8), 8 columns.
template <int DH, int ROWS>
__device__ __forceinline__ void tile_gload_rows(uint4* r, const uint16_t* __restrict__ P, int64_t ld, int r0,
                                                int rlim, int col0, int tid) {
  constexpr int CPR = DH / 8;
  constexpr int CH = ROWS * CPR / 256;
  const __amdgpu_buffer_rsrc_t rs = rows_rsrc(P, ld, r0, rlim, col0);
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid + 256 * i;
    const int row = c / CPR, col = (c % CPR) * 8;
    r[i] = buf_load16(rs, (row * (int)ld + col) * 2);
  }
}
template <int DH, int ROWS, int PITCH>
__device__ __forceinline__ void tile_swrite_rows(uint16_t* s, const uint4* r, int tid) {
  constexpr int CPR = DH / 8;
  constexpr int CH = ROWS * CPR / 256;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid + 256 * i;
    const int row = c / CPR, col = (c % CPR) * 8;
    *(uint4*)(s + row * PITCH + col) = r[i];
  }
}

// ---------------------------------------------------------------------------
// V^T tiles in LDS
// ---------------------------------------------------------------------------
// The B operand of P V needs, per lane, 8 keys of one dh column.  With the
// keys of each 16-key group stored in the order pi(k) below, those 8 keys are
// contiguous, so the operand is one 16-byte LDS read instead of two transpose
// reads.  A [DH][64-key] tile is written from row-major global rows: each
// thread owns 4 consecutive keys x 8 dh, transposes them in registers and
// writes 8 eight-byte pieces; the lane -> (keys, dh chunk) assignment keeps
// every half-wave of the writes and every quarter-wave of the reads on
// distinct banks with a row pitch of 72 elements.
constexpr int VT_PITCH = 72;

__device__ __forceinline__ int key_perm(int k) {
  const int k16 = k & 15;
  return (k & ~15) + 8 * ((k16 >> 2) & 1) + 4 * (k16 >> 3) + (k16 & 3);
}

template <int DH>
struct VtLoad {
  uint4 x[4];
  int kq, c;
  bool on;
};

// Global loads of one 64-key V tile for V^T: 4 rows (keys 4kq..4kq+3) x 16
// bytes (dh 8c..8c+7).  tid < 256 (four waves), so c < 16: with DH = 128
// every thread has a chunk, which is stated at compile time so that the
// loads are not wrapped in lane-masked branches.
template <int DH>
__device__ __forceinline__ void vt_gload(VtLoad<DH>& L, const uint16_t* __restrict__ V, int64_t ld, int k0,
                                         int rlim, int col0, int tid) {
  const int lane = tid & 63, w = tid >> 6;
  L.kq = lane & 15;
  L.c = 4 * w + 2 * ((lane >> 5) & 1) + ((lane >> 4) & 1);
  L.on = DH / 8 >= 16 || L.c < DH / 8;
  const __amdgpu_buffer_rsrc_t rs = rows_rsrc(V, ld, k0, rlim, col0);
#pragma unroll
  for (int r = 0; r < 4; ++r)
    L.x[r] = L.on ? buf_load16(rs, ((4 * L.kq + r) * (int)ld + 8 * L.c) * 2) : make_uint4(0, 0, 0, 0);
}

template <int DH>
__device__ __forceinline__ void vt_swrite(uint16_t* s, const VtLoad<DH>& L) {
  if (!L.on) return;
  const uint32_t* x0 = (const uint32_t*)&L.x[0];
  const uint32_t* x1 = (const uint32_t*)&L.x[1];
  const uint32_t* x2 = (const uint32_t*)&L.x[2];
  const uint32_t* x3 = (const uint32_t*)&L.x[3];
  const int col = key_perm(4 * L.kq);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    // dh 8c + 2m (low halves) and 8c + 2m + 1 (high halves)
    uint2 lo, hi;
    lo.x = __builtin_amdgcn_perm(x1[m], x0[m], 0x05040100u);
    lo.y = __builtin_amdgcn_perm(x3[m], x2[m], 0x05040100u);
    hi.x = __builtin_amdgcn_perm(x1[m], x0[m], 0x07060302u);
    hi.y = __builtin_amdgcn_perm(x3[m], x2[m], 0x07060302u);
    *(uint2*)(s + (8 * L.c + 2 * m) * VT_PITCH + col) = lo;
    *(uint2*)(s + (8 * L.c + 2 * m + 1) * VT_PITCH + col) = hi;
  }
}

// B operand of P V from a V^T tile: column dh = col0 + l32, k-step u.
__device__ __forceinline__ op8 vt_operand(const uint16_t* s, int u, int col0, int lane) {
  op8 o;
  o.v = *(const u32x4_t*)(s + (col0 + (lane & 31)) * VT_PITCH + 16 * u + 8 * (lane >> 5));
  return o;
}

// ---------------------------------------------------------------------------
// Epilogue: one wave's 32-row accumulator tile to 16-bit rows
// ---------------------------------------------------------------------------
// acc[b] holds column 32 (cb0 + b) + l32 (relative to col0) of rows
// r0 + 8 (j >> 2) + 4 g + (j & 3).  out[row, col] = acc * scale, times
// z[row, col] (the SiLU derivative at the projection's pre-activation) when
// z is given; rows at or beyond rlim are not written.
// Two column blocks at a time pass through a wave-private LDS stage of
// 32 x 64 floats, so that z is read and out written 16 bytes per lane (all
// loads of a round issued before any is used) with the buffer range check
// doing the row bound.  The pitch of 72 floats puts the two lane halves of a
// stage write on different banks.
constexpr int EP_PITCH = 72;
constexpr int EP_FLOATS = 32 * EP_PITCH;  // per wave

template <typename T, int NB>
__device__ __forceinline__ void wave_store_rows(float* stage, const f32x16_t (&acc)[NB], int cb0, int lane,
                                                int r0, int rlim, float scale, uint16_t* out, int64_t ldo,
                                                int col0, const uint16_t* z, int64_t ldz) {
  constexpr int NBR = NB < 2 ? NB : 2;    // column blocks per round
  constexpr int CPR = NBR * 4;            // 8-column chunks per row
  constexpr int RPP = 64 / CPR;           // rows per pass
  constexpr int NP = 32 / RPP;            // passes per round
  const int l32 = lane & 31, g = lane >> 5;
  const __amdgpu_buffer_rsrc_t ro = rows_rsrc(out, ldo, r0, rlim, col0);
  const __amdgpu_buffer_rsrc_t rz = rows_rsrc(z ? z : out, ldz, r0, rlim, col0);
  const int pr = lane / CPR, pc = (lane % CPR) * 8;
#pragma unroll
  for (int b0 = 0; b0 < NB; b0 += NBR) {
#pragma unroll
    for (int b = 0; b < NBR; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        stage[(8 * (j >> 2) + 4 * g + (j & 3)) * EP_PITCH + 32 * b + l32] = acc[b0 + b][j] * scale;
    const int colb = 32 * (cb0 + b0) + pc;
    uint4 zz[NP];
    if (z) {
#pragma unroll
      for (int p = 0; p < NP; ++p)  // read once: non-temporal
        zz[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rz, ((p * RPP + pr) * (int)ldz + colb) * 2,
                                                                                0, 2 /* non-temporal */));
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int rr = p * RPP + pr;
      const f32x4_t a = *(const f32x4_t*)&stage[rr * EP_PITCH + pc];
      const f32x4_t c = *(const f32x4_t*)&stage[rr * EP_PITCH + pc + 4];
      float v[8] = {a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
      if (z) {
        const uint32_t zw[4] = {zz[p].x, zz[p].y, zz[p].z, zz[p].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= from_bits16<T>((uint16_t)(zw[e >> 1] >> (16 * (e & 1))));
      }
      u32x4_t o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack2<T>(v[2 * e], v[2 * e + 1]);
      buf_store16(ro, (rr * (int)ldo + colb) * 2, o);
    }
  }
}

// ---------------------------------------------------------------------------
// forward: 128 queries per workgroup (4 waves x 32), 64 keys per LDS stage,
// two workgroups per CU so that one wave's SiLU overlaps another's MFMAs.
// ---------------------------------------------------------------------------
constexpr int F_BQ = 128;
constexpr int F_BK = 64;

// As pipeline_lds_mfma, with NV vector-memory loads (the next tile's rows)
// issued one after each of the first MFMAs, so that the load issue overlaps
// the MFMAs instead of holding the wave at the top of the tile.
template <int N, int AHEAD, int NV>
__device__ __forceinline__ void pipeline_lds_mfma_vmem() {
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);  // DS reads
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    if (i < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

template <typename T, int DH, bool MASKED, int NV = 0>
__device__ __forceinline__ void fwd_tile(const uint16_t* Ks, const uint16_t* Vt, const int64_t* tsk,
                                         const op8 (&qop)[DH / 16], f32x16_t (&oacc)[DH / 32], int k0, int qi,
                                         int64_t tq, int s_end, int r_end, float kexp, int lane) {
  constexpr int KP = AttnPitch<DH>::B128;
  const int g = lane >> 5;
  f32x16_t sacc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) sacc[t] = mfma32<T>(row_operand<KP>(Ks, t * 32, 0, lane), qop[0], f32x16_t{});
#pragma unroll
  for (int s = 1; s < DH / 16; ++s)
#pragma unroll
    for (int t = 0; t < 2; ++t) sacc[t] = mfma32<T>(row_operand<KP>(Ks, t * 32, s, lane), qop[s], sacc[t]);
  if (NV > 0) pipeline_lds_mfma_vmem<DH / 8, 8, NV>();
  else pipeline_lds_mfma<DH / 8, 8>();
  float p[2][16];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float sv = sacc[t][j];
      float pv = sv * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(sv * kexp));
      if (MASKED) {
        const int kk = t * 32 + 8 * (j >> 2) + 4 * g + (j & 3);
        if (!visible_ts(qi, k0 + kk, s_end, r_end, tq, tsk[kk])) pv = 0.f;
      }
      p[t][j] = pv;
    }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const op8 pa = pack_kstep<T>(p, u);
#pragma unroll
    for (int c = 0; c < DH / 32; ++c) oacc[c] = mfma32<T>(pa, vt_operand(Vt, u, c * 32, lane), oacc[c]);
  }
  pipeline_lds_mfma<DH / 8, 8>();
}

// With nsplit > 1 (short batches), the key tiles of each (query tile, head)
// are shared out in nsplit contiguous runs, one workgroup each: workgroup
// L = split * base + L'.  Each writes its scaled fp32 partial sum to
// part[split][row][col] (rows of its query tile, zeros when its run is
// empty); the consumer of O adds the planes in split order.
template <typename T, int DH>
__global__ __launch_bounds__(256, 2) void attn_fwd_mfma(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    int64_t ldqkv, uint16_t* __restrict__ O, int64_t ldo, const int32_t* __restrict__ seg,
    const int64_t* __restrict__ ts, const int2* __restrict__ tiles, const int32_t* __restrict__ ntiles,
    int H, float kexp, float out_scale, int nsplit, int base, float* __restrict__ part, int64_t T_rows) {
  constexpr int KP = AttnPitch<DH>::B128;
  constexpr int NS = DH / 16, NC = DH / 32;
  struct Smem {
    uint16_t Ks[2][F_BK * KP];
    uint16_t Vt[2][DH * VT_PITCH];
    int64_t Tk[2][F_BK];  // key timestamps of the tile
  };
  __shared__ __attribute__((aligned(16))) union {
    Smem m;
    float ep[4 * EP_FLOATS];
  } sm;
  auto& Ks = sm.m.Ks;
  auto& Vt = sm.m.Vt;
  auto& Tk = sm.m.Tk;
  int tile, h, split = 0, L = blockIdx.x;
  if (nsplit > 1) {
    split = L / base;
    L -= split * base;
  }
  xcd_tile_head(L, H, tile, h);
  if (tile >= *ntiles) return;
  const int2 te = tiles[tile];
  const int b = te.x, q0 = te.y;
  const int lo = seg[b * 5 + 0], s_end = seg[b * 5 + 2], r_end = seg[b * 5 + 3], hi = seg[b * 5 + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), l32 = lane & 31, g = lane >> 5;
  const int q_last = min(q0 + F_BQ, hi) - 1;
  const KeyRuns kr = key_runs(lo, q0, q_last, s_end, r_end);
  const int qi = q0 + wave * 32 + l32;
  const bool qv = qi < hi;
  const int qr = qv ? qi : lo;
  const int64_t tq = ts[qr];
  const int hc = h * DH;

  op8 qop[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    u32x4_t v = *(const u32x4_t*)(Q + (int64_t)qr * ldqkv + hc + 16 * s + 8 * g);
    qop[s].v = qv ? v : u32x4_t{0, 0, 0, 0};
  }
  f32x16_t oacc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[c][j] = 0.f;

  constexpr int CH = F_BK * (DH / 8) / 256;
  uint4 rk[CH];
  VtLoad<DH> rv;
  int64_t rt = 0;
  const int nkt = kr.n;
  // this workgroup's run of key-tile visits [it0, it1)
  int it0 = 0, it1 = nkt;
  if (nsplit > 1) {
    const int per = (nkt + nsplit - 1) / nsplit;
    it0 = min(nkt, split * per);
    it1 = min(nkt, it0 + per);
  }
  // leading tiles made only of U/S keys need no mask test
  const int nfull = min(nkt, max(0, (s_end - lo) / F_BK));
  auto gload = [&](int k0) {
    tile_gload_rows<DH, F_BK>(rk, K, ldqkv, k0, hi, hc, tid);
    vt_gload<DH>(rv, V, ldqkv, k0, hi, hc, tid);
    rt = ts_load(ts, k0, hi, lane);  // every wave: no branch before the MFMAs
  };
  auto swrite = [&](int buf) {
    tile_swrite_rows<DH, F_BK, KP>(Ks[buf], rk, tid);
    vt_swrite<DH>(Vt[buf], rv);
    if (wave == 0) Tk[buf][lane] = rt;
  };
  if (it0 < it1) {
    gload(lo + kr.tile(it0) * F_BK);
    swrite(0);
  }
  __syncthreads();
  // the full tiles come first (tile(it) == it there)
  const int mid = max(it0, min(it1, nfull));
  for (int it = it0; it < mid; ++it) {
    const int buf = (it - it0) & 1, k0 = lo + it * F_BK;
    // unconditional, so that the loads share the MFMAs' scheduling region
    // and issue between them: past the run they fetch a tile nobody reads
    // (rows at or beyond the row end read as zero), written to the idle
    // buffer
    gload(lo + kr.tile(it + 1) * F_BK);
    fwd_tile<T, DH, false, 9>(Ks[buf], Vt[buf], Tk[buf], qop, oacc, k0, qi, tq, s_end, r_end, kexp, lane);
    swrite(buf ^ 1);
    __syncthreads();
  }
  for (int it = mid; it < it1; ++it) {
    const int buf = (it - it0) & 1, k0 = lo + kr.tile(it) * F_BK;
    const bool more = it + 1 < it1;
    if (more) gload(lo + kr.tile(it + 1) * F_BK);
    fwd_tile<T, DH, true>(Ks[buf], Vt[buf], Tk[buf], qop, oacc, k0, qi, tq, s_end, r_end, kexp, lane);
    if (more) swrite(buf ^ 1);
    __syncthreads();
  }
  if (nsplit > 1) {
    // fp32 partial: accumulator element (c, j) is column 32 c + l32 of row
    // 8 (j / 4) + 4 g + j % 4 of the wave's 32 rows
    float* pp = part + (int64_t)split * T_rows * (H * DH) + hc;
    const int r0 = q0 + wave * 32;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int row = r0 + 8 * (j >> 2) + 4 * g + (j & 3);
      if (row < hi) {
#pragma unroll
        for (int c = 0; c < NC; ++c) pp[(int64_t)row * (H * DH) + 32 * c + l32] = oacc[c][j] * out_scale;
      }
    }
    return;
  }
  wave_store_rows<T, NC>(sm.ep + wave * EP_FLOATS, oacc, 0, lane, q0 + wave * 32, hi, out_scale, O, ldo, hc,
                         nullptr, 0);
}

// ---------------------------------------------------------------------------
// Loads of a 64-row tile in "quad" form: each thread owns 4 consecutive rows
// x 8 columns, which serves both the row-major copy (A operands read 16 bytes
// per lane) and the transposed copy (B operands whose contraction index is the
// row).  Same lane assignment as vt_gload.
// ---------------------------------------------------------------------------
template <int DH>
__device__ __forceinline__ void quad_swrite_rows(uint16_t* s, const VtLoad<DH>& L) {
  constexpr int KP = AttnPitch<DH>::B128;
  if (!L.on) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) *(uint4*)(s + (4 * L.kq + r) * KP + 8 * L.c) = L.x[r];
}

// Row-major 64-row tile written from quads with a bank swizzle: for DH = 128
// a row is 256 unpadded bytes and its 16-byte chunk c sits at position
// c ^ ((r >> 2) ^ 4 (r & 3)) mod 16, which keeps both the quad writes (16
// lanes = 16 quads, one chunk) and the A-operand reads (16 consecutive rows,
// one chunk) on distinct banks; with a padded pitch the quad writes collide
// four ways.  DH = 64 keeps the padded pitch.
template <int DH> struct QuadRows {
  static constexpr int PITCH = DH == 128 ? 128 : DH + 8;  // elements per row
  static constexpr int SIZE = 64 * PITCH;
  static __device__ __forceinline__ int off(int row, int ch) {
    if (DH == 128) return row * 128 + 8 * (ch ^ (((row >> 2) ^ ((row & 3) << 2)) & 15));
    return row * PITCH + 8 * ch;
  }
};
template <int DH>
__device__ __forceinline__ void quad_swrite_swz(uint16_t* s, const VtLoad<DH>& L) {
  if (!L.on) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) *(uint4*)(s + QuadRows<DH>::off(4 * L.kq + r, L.c)) = L.x[r];
}
// Rows of a tile loaded by tile_gload_rows (thread chunks c = tid + 256 i,
// row c / (DH/8)) written to a QuadRows tile.
template <int DH, int ROWS>
__device__ __forceinline__ void tile_swrite_swz(uint16_t* s, const uint4* r, int tid) {
  constexpr int CPR = DH / 8;
  constexpr int CH = ROWS * CPR / 256;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid + 256 * i;
    *(uint4*)(s + QuadRows<DH>::off(c / CPR, c % CPR)) = r[i];
  }
}
// A operand from a QuadRows tile: row r0 + l32, 8 columns at 16 ks + 8 g.
template <int DH>
__device__ __forceinline__ op8 row_operand_swz(const uint16_t* s, int r0, int ks, int lane) {
  op8 o;
  o.v = *(const u32x4_t*)(s + QuadRows<DH>::off(r0 + (lane & 31), 2 * ks + (lane >> 5)));
  return o;
}

// B operand from a QuadRows tile read transposed (gfx950 LDS transpose
// load): column 32 c + l32 of the tile over contraction rows 16 u + 4 g +
// (j % 4) + 8 (j / 4) (g = lane / 32, j = 0..7: the permuted k order of
// pack_kstep), as two 4-row x 16-column quarter-wave blocks.  A lane's 8-byte
// piece never straddles a 16-byte chunk, so the row swizzle only moves whole
// chunks.  Lane i of quarter G reads row 16 u + 4 g + i / 4 + 8 h (h = 0, 1)
// at column 32 c + 16 (G % 2) + 4 (i % 4); with DH = 128 the swizzled chunk
// is 4 ((c ^ u ^ i / 4) % 4) + ((2 (G % 2) + (i % 4) / 2) ^ (g + 2 h)), so a
// lane needs only 8 base addresses, picked by (c ^ u) % 4 and h; u adds 16
// rows, an immediate offset.
template <int DH>
struct TrAddr {
  int a[4][2];
  __device__ __forceinline__ void init(int lane) {
    const int G = lane >> 4, i = lane & 15, q = i >> 2, g = G >> 1;
    const int chl = 2 * (G & 1) + ((i & 3) >> 1), sub = (i & 1) * 4;
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 4 * g + q + 8 * h;
        if (DH == 128) {
          a[v][h] = row * 128 + 8 * (4 * ((v ^ q) & 3) + (chl ^ (g + 2 * h))) + sub;
        } else {
          // padded rows: column 32 c + 16 (G % 2) + 4 (i % 4), no swizzle
          a[v][h] = row * QuadRows<DH>::PITCH + 16 * (G & 1) + 4 * (i & 3);
        }
      }
  }
  // operand (u, c) of tile s
  __device__ __forceinline__ op8 get(const uint16_t* s, int u, int c) const {
    const int v = DH == 128 ? ((c ^ u) & 3) : 0;
    const int imm = DH == 128 ? u * 16 * 128 : u * 16 * QuadRows<DH>::PITCH + 32 * c;
    const uint2 lo = lds_read_tr16(s + a[v][0] + imm);
    const uint2 hi = lds_read_tr16(s + a[v][1] + imm);
    op8 o;
    o.v[0] = lo.x; o.v[1] = lo.y; o.v[2] = hi.x; o.v[3] = hi.y;
    return o;
  }
};

// ---------------------------------------------------------------------------
// Elementwise SiLU terms of a 64 x 32 score tile (two 32 x 32 accumulators),
// with or without the mask test.  Kept as straight-line code per variant so
// that the exp / rcp chains of the 32 elements interleave.
// ---------------------------------------------------------------------------
// Transposed tile (rows = keys kk of the tile at k0, lane = query qi):
// f = M * SiLU'(alpha s) goes to the exchange buffer fx as f16 pairs.
template <bool MASKED>
__device__ __forceinline__ void silu_grad_rows_keys(const f32x16_t (&x)[2], uint32_t* fx, int lane, float kexp,
                                                    float alpha, int qi, int k0, int g, int s_end, int r_end,
                                                    int64_t tq, const int64_t* tsk) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float f[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = 2 * e + h;
        const float sr = x[t][j];
        const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(sr * kexp));
        // SiLU'(y) = sigma + y sigma (1 - sigma), y = alpha s
        f[h] = __builtin_fmaf(alpha * (sr * sg), 1.0f - sg, sg);
        if (MASKED) {
          const int kk = t * 32 + 8 * (j >> 2) + 4 * g + (j & 3);
          f[h] = visible_ts(qi, k0 + kk, s_end, r_end, tq, tsk[kk]) ? f[h] : 0.f;
        }
      }
      fx[(t * 8 + e) * 64 + lane] = pack2<f16_t>(f[0], f[1]);
    }
}

// Tile with rows = queries qq of the stage at q0, lane = key kj:
// P = SiLU(alpha s) / alpha packed as the A operands w of P^T dO, and
// f = M * SiLU'(alpha s) to the exchange buffer fx as f16 pairs.
template <typename T, bool MASKED, bool A1 = false>
__device__ __forceinline__ void silu_terms_rows_queries(const f32x16_t (&x)[2], op8 (&w)[4], uint32_t* fx, int lane,
                                                        float kexp, float alpha, int q0, int kj, int g, int s_end,
                                                        int r_end, const int64_t* tsq, int64_t tk) {
  // Element (t, j) is query q0 + qq, qq = c + 4 g with c = 32 t + 8 (j / 4)
  // + j % 4 a constant.  The mask's index tests become comparisons of c with
  // per-call values: the query is real-time or later when c >= thr and sits
  // on the key's diagonal when c == dg.  A candidate key takes thr below
  // every c and a timestamp no query is earlier than, which leaves only the
  // diagonal; a static key sees every query.  The empty asm keeps the
  // compiler from rewriting the tests as q0 + c comparisons, which it would
  // otherwise precompute for all 32 elements outside the caller's loop.
  int thr = 0, dg = 0;
  int64_t tke = 0;
  bool kstat = true;
  if (MASKED) {
    const bool kcand = kj >= r_end;
    kstat = kj < s_end;
    thr = kcand ? -1024 : s_end - q0 - 4 * g;
    dg = kj - q0 - 4 * g;
    tke = kcand ? INT64_MAX : tk;
    asm volatile("" : "+v"(thr), "+v"(dg));
  }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float pv[2], f[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = 2 * e + h;
        const float sr = x[t][j];
        const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(sr * kexp));
        pv[h] = sr * sg;
        // SiLU'(y) = sigma + y sigma (1 - sigma), y = alpha s
        // (A1: alpha is 1 and the multiply is skipped, same bits)
        f[h] = __builtin_fmaf(A1 ? pv[h] : alpha * pv[h], 1.0f - sg, sg);
        if (MASKED) {
          const int c = t * 32 + 8 * (j >> 2) + (j & 3);
          // bitwise throughout: a conditional form lets the compiler put the
          // timestamp read under a per-lane branch
          const bool vis = kstat | ((c >= thr) & ((tke < tsq[c + 4 * g]) | (c == dg)));
          pv[h] = vis ? pv[h] : 0.f;
          f[h] = vis ? f[h] : 0.f;
        }
      }
      // element pair (2e, 2e+1) of subtile t is dword e % 4 of k-step 2t + e / 4
      w[2 * t + (e >> 2)].v[e & 3] = pack2<T>(pv[0], pv[1]);
      fx[(t * 8 + e) * 64 + lane] = pack2<f16_t>(f[0], f[1]);
    }
}

// ---------------------------------------------------------------------------
// backward, query-major: dQ = alpha * c * sum_j [M SiLU'(S) (dO v_j)] k_j
// for 128 queries (4 waves x 32), 64 keys per LDS stage.
// ---------------------------------------------------------------------------
// 512 threads in producer/consumer pairs over 128 queries: wave i (i < 4)
// computes S^T for query group i and the factor f = M * SiLU'(alpha s)
// (written to LDS as f16); wave i + 4 computes dA^T = V dO^T for the same
// queries and forms dS = dA * f, which it hands back through LDS; each wave
// of the pair then accumulates half of the dQ = dS K columns, so both do
// the same number of MFMAs.
// One (query tile, head) of the recompute dQ; the whole workgroup calls it
// with the same arguments.
template <typename T, int DH>
__device__ __forceinline__ void dq_mfma_tile(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    int64_t ldqkv, const uint16_t* __restrict__ dO, int64_t lddo, uint16_t* __restrict__ dQ,
    int64_t lddq, const uint16_t* __restrict__ zq, int64_t ldz, const int32_t* __restrict__ seg,
    const int64_t* __restrict__ ts, const int2* __restrict__ tiles, int H, float kexp, float alpha,
    float out_scale, int tile, int h) {
  constexpr int KP = AttnPitch<DH>::B128;
  constexpr int NS = DH / 16, NC = DH / 32;
  struct Smem {
    uint16_t Ks[2][A_BK * KP];
    uint16_t Vs[2][A_BK * KP];
    uint16_t Kt[2][DH * VT_PITCH];
    uint32_t Fx[4][32 * 16 * 2];
    int64_t Tk[2][A_BK];  // key timestamps of the tile
  };
  __shared__ __attribute__((aligned(16))) union {
    Smem m;
    float ep[8 * EP_FLOATS];
  } sm;
  auto& Ks = sm.m.Ks;
  auto& Vs = sm.m.Vs;
  auto& Kt = sm.m.Kt;
  auto& Fx = sm.m.Fx;
  auto& Tk = sm.m.Tk;
  const int2 te = tiles[tile];
  const int b = te.x, q0 = te.y;
  const int lo = seg[b * 5 + 0], s_end = seg[b * 5 + 2], r_end = seg[b * 5 + 3], hi = seg[b * 5 + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), l32 = lane & 31, g = lane >> 5;
  const bool producer = wave < 4;
  const int grp = wave & 3;
  const int ltid = tid & 255;
  const int q_last = min(q0 + A_BQ, hi) - 1;
  const KeyRuns kr = key_runs(lo, q0, q_last, s_end, r_end);
  const int qi = q0 + grp * 32 + l32;
  const bool qv = qi < hi;
  const int qr = qv ? qi : lo;
  const int64_t tq = ts[qr];
  const int hc = h * DH;

  // producer: Q (B operand of S^T = K Q^T); consumer: dO (B of dA^T = V dO^T)
  op8 bop[NS];
  {
    const uint16_t* src = producer ? Q : dO;
    const int64_t lds = producer ? ldqkv : lddo;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4_t a = *(const u32x4_t*)(src + (int64_t)qr * lds + hc + 16 * s + 8 * g);
      bop[s].v = qv ? a : u32x4_t{0, 0, 0, 0};
    }
  }
  // dQ column blocks per role: producers [0, NC / 2), consumers the rest
  // (with one block, DH = 32, the consumers take it)
  constexpr int NCH = (NC + 1) / 2;
  const int ncol = producer ? NC / 2 : NC - NC / 2;
  f32x16_t acc[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[c][j] = 0.f;

  VtLoad<DH> ld;  // producers load K quads (row-major + transposed), consumers V rows
  int64_t rt = 0;
  auto gload = [&](int k0) {
    if (producer) vt_gload<DH>(ld, K, ldqkv, k0, hi, hc, ltid);
    else tile_gload_rows<DH, A_BK>(ld.x, V, ldqkv, k0, hi, hc, ltid);
    if (wave == 0) rt = ts_load(ts, k0, hi, lane);
  };
  auto swrite = [&](int buf) {
    if (producer) {
      quad_swrite_rows<DH>(Ks[buf], ld);
      vt_swrite<DH>(Kt[buf], ld);
    } else {
      tile_swrite_rows<DH, A_BK, KP>(Vs[buf], ld.x, ltid);
    }
    if (wave == 0) Tk[buf][lane] = rt;
  };
  static_assert(A_BK == 64, "key runs count 64-key tiles");
  const int nkt = kr.n;
  const int nfull = min(nkt, max(0, (s_end - lo) / A_BK));
  if (nkt > 0) {
    gload(lo + kr.tile(0) * A_BK);
    swrite(0);
  }
  __syncthreads();
  uint32_t* fx = Fx[grp];
  for (int it = 0; it < nkt; ++it) {
    const int buf = it & 1, k0 = lo + kr.tile(it) * A_BK;
    const bool more = it + 1 < nkt;
    if (more) gload(lo + kr.tile(it + 1) * A_BK);
    // phase 1: S^T (producer) or dA^T (consumer) for 64 keys x 32 queries
    const uint16_t* A = producer ? Ks[buf] : Vs[buf];
    f32x16_t x[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) x[t] = mfma32<T>(row_operand<KP>(A, t * 32, 0, lane), bop[0], f32x16_t{});
#pragma unroll
    for (int s = 1; s < NS; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t) x[t] = mfma32<T>(row_operand<KP>(A, t * 32, s, lane), bop[s], x[t]);
    if (producer) {
      if (it >= nfull)
        silu_grad_rows_keys<true>(x, fx, lane, kexp, alpha, qi, k0, g, s_end, r_end, tq, Tk[buf]);
      else
        silu_grad_rows_keys<false>(x, fx, lane, kexp, alpha, qi, k0, g, s_end, r_end, tq, Tk[buf]);
    }
    __syncthreads();  // f of this tile visible to the consumers
    op8 da[4];
    if (!producer) {
      float d[2][16];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t fv = fx[(t * 8 + e) * 64 + lane];
          d[t][2 * e] = __builtin_fmaf(x[t][2 * e], from_bits16<f16_t>((uint16_t)(fv & 0xffff)), 0.0f);
          d[t][2 * e + 1] = __builtin_fmaf(x[t][2 * e + 1], from_bits16<f16_t>((uint16_t)(fv >> 16)), 0.0f);
        }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        da[u] = pack_kstep<T>(d, u);
        // hand dS to the producer, which accumulates the other half of dQ
        *(u32x4_t*)&fx[(u * 4) * 64 + lane * 4] = da[u].v;
      }
    }
    __syncthreads();  // dS of this tile visible to the producers
    if (producer) {
#pragma unroll
      for (int u = 0; u < 4; ++u) da[u].v = *(const u32x4_t*)&fx[(u * 4) * 64 + lane * 4];
    }
    // dQ += dS K over this role's column blocks
    const int cb = producer ? 0 : NC / 2;
    if (ncol > 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < NCH; ++c)
          acc[c] = mfma32<T>(da[u], vt_operand(Kt[buf], u, (cb + c) * 32, lane), acc[c]);
    }
    if (more) swrite(buf ^ 1);
    __syncthreads();
  }
  if (ncol > 0)
    wave_store_rows<T, NCH>(sm.ep + wave * EP_FLOATS, acc, producer ? 0 : NC / 2, lane, q0 + grp * 32, hi,
                            out_scale, dQ, lddq, hc, zq, ldz);
}

template <typename T, int DH>
__global__ __launch_bounds__(512, 1) void attn_bwd_dq_mfma(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    int64_t ldqkv, const uint16_t* __restrict__ dO, int64_t lddo, uint16_t* __restrict__ dQ,
    int64_t lddq, const uint16_t* __restrict__ zq, int64_t ldz, const int32_t* __restrict__ seg,
    const int64_t* __restrict__ ts, const int2* __restrict__ tiles, const int32_t* __restrict__ ntiles,
    int H, float kexp, float alpha, float out_scale) {
  int tile, h;
  xcd_tile_head(blockIdx.x, H, tile, h);
  if (tile >= *ntiles) return;
  dq_mfma_tile<T, DH>(Q, K, V, ldqkv, dO, lddo, dQ, lddq, zq, ldz, seg, ts, tiles, H, kexp, alpha, out_scale,
                      tile, h);
}

// After the dQ stream: the (query tile, head) items of rows whose stored dS
// did not fit its buffer (rows longer than the declared maximum), which the
// stream skipped.  A small grid walks all items 512 at a time, one check per
// thread, and recomputes only the flagged ones, so that the launch costs a
// few microseconds when no row overflows.
template <typename T, int DH>
__global__ __launch_bounds__(512, 1) void attn_bwd_dq_overflow(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    int64_t ldqkv, const uint16_t* __restrict__ dO, int64_t lddo, uint16_t* __restrict__ dQ,
    int64_t lddq, const uint16_t* __restrict__ zq, int64_t ldz, const int32_t* __restrict__ seg,
    const int64_t* __restrict__ ts, const int2* __restrict__ tiles, const int32_t* __restrict__ ntiles,
    int H, float kexp, float alpha, float out_scale, const int64_t* __restrict__ tprefix, int64_t ds_cap) {
  __shared__ uint8_t flag[512];
  const int total = *ntiles * H;
  for (int base = blockIdx.x * 512; base < total; base += gridDim.x * 512) {
    const int item = base + (int)threadIdx.x;
    uint8_t f = 0;
    if (item < total) {
      const int b = tiles[item / H].x;
      const int nt = (seg[b * 5 + 4] - seg[b * 5 + 0] + 127) >> 7;
      f = tprefix[b] + (int64_t)nt * nt > ds_cap;
    }
    __syncthreads();  // the previous pass's flags have been read
    flag[threadIdx.x] = f;
    if (!__syncthreads_or(f)) continue;  // the usual case: nothing to redo
    for (int i = 0; i < 512 && base + i < total; ++i)
      if (flag[i]) {
        dq_mfma_tile<T, DH>(Q, K, V, ldqkv, dO, lddo, dQ, lddq, zq, ldz, seg, ts, tiles, H, kexp, alpha,
                            out_scale, (base + i) / H, (base + i) % H);
        __syncthreads();  // every wave's epilogue staging read before the LDS is reused
      }
  }
}

// ---------------------------------------------------------------------------
// backward, key-major: dV = c P^T dO, dK = alpha c dS^T Q for 128 keys, 64
// queries per LDS stage.  512 threads in producer/consumer pairs: wave i
// (i < 4) computes S for key group i, the SiLU weights P and the factor
// f = M * SiLU'(alpha s) (written to LDS as f16), then dV; wave i + 4
// computes dA = dO V^T for the same keys, reads f, forms dS = dA * f, then dK.
// Each wave holds only half of the per-key state, so two waves fit per SIMD.
// ---------------------------------------------------------------------------
constexpr int KV_BK = 128;    // keys per workgroup (4 groups of 32)
constexpr int KV_BQ = 64;     // queries per LDS stage
constexpr int F_PITCH = 64;   // f16 exchange tile: [key group][64 queries][32 keys]

template <typename T, int DH, bool STORE, bool A1 = false>
__global__ __launch_bounds__(512, 1) void attn_bwd_dkdv_mfma(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    int64_t ldqkv, const uint16_t* __restrict__ dO, int64_t lddo, uint16_t* __restrict__ dK,
    uint16_t* __restrict__ dV, int64_t lddkv, const uint16_t* __restrict__ zk,
    const uint16_t* __restrict__ zv, int64_t ldz, const int32_t* __restrict__ seg,
    const int64_t* __restrict__ ts, const int2* __restrict__ tiles, const int32_t* __restrict__ ntiles,
    int H, float kexp, float alpha, float scale, uint8_t* __restrict__ dS, int64_t ds_cap,
    const int64_t* __restrict__ tprefix) {
  constexpr int NS = DH / 16, NC = DH / 32;
  // Stage buffers: in iteration it the S side works on stage it, the dA side
  // on stage it - 1 (dA, dS) and on stage it - 2 (its dK product, which
  // reads that stage's Q rows), while stage it + 1 is being written.  So Q
  // rows (and their timestamps) of stage j live in buffer j % 4, dO rows in
  // buffer j % 3.  The dO tiles come first: with DH = 128 the three dO and
  // four Q tiles end at 48 and 112 KB, so the constant part of every operand
  // address (a tile's base plus the 16-row steps of the transposed reads,
  // up to 63 KB) fits the 16-bit offset field of the LDS instructions.
  struct Smem {
    uint16_t Ds[3][QuadRows<DH>::SIZE];
    uint16_t Qs[4][QuadRows<DH>::SIZE];
    uint32_t Fx[2][4][32 * 16 * 2];  // per stage parity and group: 2 x 16 x 32 lanes
    int64_t Tq[4][KV_BQ];            // query timestamps of the stage
  };
  __shared__ __attribute__((aligned(16))) union {
    Smem m;
    float ep[8 * EP_FLOATS];
  } sm;
  auto& Qs = sm.m.Qs;
  auto& Ds = sm.m.Ds;
  auto& Fx = sm.m.Fx;
  auto& Tq = sm.m.Tq;
  int tile, h;
  xcd_tile_head(blockIdx.x, H, tile, h);
  if (tile >= *ntiles) return;
  const int2 te = tiles[tile];
  const int b = te.x, k0 = te.y;
  const int lo = seg[b * 5 + 0], s_end = seg[b * 5 + 2], r_end = seg[b * 5 + 3], hi = seg[b * 5 + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), l32 = lane & 31, g = lane >> 5;
  const bool producer = wave < 4;   // S-side wave; wave + 4 is its dA-side partner
  const int grp = wave & 3;
  const int ltid = tid & 255;
  const int k_last = min(k0 + KV_BK, hi) - 1;
  // Query stages lie on a 64-row grid from the row start, so that every
  // stored dS block has a fixed place; real-time keys start at the stage
  // holding the first real-time query.
  int qlo, qhi;
  if (k0 < s_end) { qlo = lo; qhi = hi; }                              // static keys: every query
  else if (k0 < r_end) { qlo = lo + ((s_end - lo) & ~63); qhi = hi; }  // real-time keys: R and C queries
  else { qlo = k0; qhi = k_last + 1; }                                 // candidate keys: themselves
  const int kj = k0 + grp * 32 + l32;
  const bool kv = kj < hi;
  const int kr = kv ? kj : lo;
  const int64_t tk = ts[kr];
  const int hc = h * DH;
  const bool full = k0 + KV_BK <= s_end;  // every query sees these keys
  // dS store target of this (dA-side) wave: see attn_bwd_dq_stream for the
  // layout.  dsb is the wave's block at query stage 0 (same on every lane).
  const uint8_t* dsb = dS;
  int64_t ds_qt_stride = 0;
  bool ds_on = false;
  if (STORE && !producer) {
    const int nt = (hi - lo + 127) >> 7;
    const int64_t pb = tprefix[b];
    if (pb + (int64_t)nt * nt <= ds_cap) {
      ds_qt_stride = (int64_t)nt * DS_TILE_BYTES;
      dsb = dS + (pb * H + (int64_t)h * nt * nt) * (int64_t)DS_TILE_BYTES +
            (int64_t)((k0 - lo) >> 7) * DS_TILE_BYTES + (grp >> 1) * 16384 + (grp & 1) * 4096;
      ds_on = true;
    }
  }

  // producer: K of its keys (B operand of S = Q K^T); consumer: V (B of dA)
  op8 bop[NS];
  {
    const uint16_t* src = producer ? K : V;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4_t a = *(const u32x4_t*)(src + (int64_t)kr * ldqkv + hc + 16 * s + 8 * g);
      bop[s].v = kv ? a : u32x4_t{0, 0, 0, 0};
    }
  }
  f32x16_t acc[NC];  // producer: dV, consumer: dK
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[c][j] = 0.f;

  // producers load Q rows, consumers dO rows; each wave-wide load covers
  // whole rows (for DH = 128 four rows of 256 bytes), the fewest cache lines
  // per instruction
  constexpr int LCH = DH / 32;
  uint4 ldx[LCH];
  int64_t rt = 0;
  auto gload = [&](int q0) {
    tile_gload_rows<DH, KV_BQ>(ldx, producer ? Q : dO, producer ? ldqkv : lddo, q0, qhi, hc, ltid);
    if (!full && wave == 0) rt = ts_load(ts, q0, qhi, lane);
  };
  auto swrite = [&](int buf) {
    tile_swrite_swz<DH, KV_BQ>(producer ? Qs[buf] : Ds[buf], ldx, ltid);
    if (!full && wave == 0) Tq[buf][lane] = rt;
  };
  const int nqt = (qhi - qlo + KV_BQ - 1) / KV_BQ;
  if (nqt > 0) {
    gload(qlo);
    swrite(0);
  }
  __syncthreads();
  TrAddr<DH> tra;
  tra.init(lane);
  // Iteration it (0..nqt + 1): the S side takes stage it (S, P, f into
  // Fx[it % 2], then dV += P^T dO); the dA side first finishes stage it - 2
  // (dK += dS^T Q with the dS it formed one iteration earlier), then forms
  // dA and dS = dA f for stage it - 1 (with the f written one iteration
  // earlier).  Each SIMD then runs one wave's MFMAs beside the other wave's
  // vector work in every phase: S products beside the dK product, the SiLU
  // terms beside dA, dV beside dS.  One barrier per iteration; both sides
  // write their halves of stage it + 1 (Q rows, dO rows) mid-iteration, the
  // S side before its dV product and the dA side before its dS, rather than
  // just before the barrier (dK/dV 0.81 -> 0.79 ms).  Each side runs a loop
  // of its own, so that neither carries the other's registers; both pass
  // nqt + 2 barriers after the first.
  //
  // A second use of the loaded values, under a condition that never holds
  // (the stage row is never negative) but that the compiler cannot fold,
  // keeps each iteration's loads at its top: their real use is the stage
  // write later on, and code sinking would otherwise move them there, the
  // latency hiding lost.
  auto keep_loads_early = [&](int it, int nbuf) {
    if (qlo + it * KV_BQ < 0) {
      uint32_t any = 0;
#pragma unroll
      for (int r = 0; r < LCH; ++r) any |= ldx[r].x | ldx[r].y | ldx[r].z | ldx[r].w;
      Tq[nbuf][lane] = any;
    }
  };
  // phase 1: S (producer) or dA (consumer) for 64 queries x 32 keys.  The
  // operand reads run three k-steps ahead of the MFMAs in source order too:
  // where register pressure makes the compiler drop the scheduling hint and
  // keep source order, each MFMA would otherwise wait a full LDS round trip.
  // byte offsets of the phase-1 operand reads inside a tile, whole (row and
  // swizzled chunk, scaled to bytes): the compiler would otherwise keep the
  // parts apart, or the element offset, and spend vector instructions on
  // every read joining or scaling them
  int p1off[NS][2];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      p1off[s][t] = 2 * QuadRows<DH>::off(t * 32 + l32, 2 * s + g);
      asm volatile("" : "+v"(p1off[s][t]));
    }
  auto p1read = [&](const uint16_t* A, int s, int t) {
    op8 o;
    o.v = *(const u32x4_t*)((const char*)A + p1off[s][t]);
    return o;
  };
  auto phase1 = [&](const uint16_t* A, f32x16_t (&x)[2]) {
    constexpr int AH = NS < 3 ? NS : 3;
    op8 ring[AH][2];
#pragma unroll
    for (int s = 0; s < AH; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t) ring[s][t] = p1read(A, s, t);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int t = 0; t < 2; ++t) x[t] = mfma32<T>(ring[s % AH][t], bop[s], s == 0 ? f32x16_t{} : x[t]);
      if (s + AH < NS) {
#pragma unroll
        for (int t = 0; t < 2; ++t) ring[s % AH][t] = p1read(A, s + AH, t);
      }
    }
    pipeline_lds_mfma<2 * NS, 2 * AH>();
  };
  // phase 2: dV += P^T dO (producer) or dK += dS^T Q (consumer), the B
  // operand read transposed from the other role's row-major tile
  auto phase2 = [&](const op8 (&w)[4], const uint16_t* Bt) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c] = mfma32<T>(w[u], tra.get(Bt, u, c), acc[c]);
    pipeline_lds2_mfma<4 * NC, 8>();
  };
  // Stage buffer j of a tile array, offset by a scalar byte count the
  // compiler cannot see through: otherwise it strength-reduces the rotating
  // buffer index into per-lane base registers and spends a vector add per
  // register and iteration advancing them.
  auto stage_tile = [&](const uint16_t* t0, int j) {
    int off = j * (int)(QuadRows<DH>::SIZE * sizeof(uint16_t));
    asm volatile("" : "+s"(off));
    return (const uint16_t*)((const char*)t0 + off);
  };
  if (producer) {
    // one loop per mask variant, so that the mask-free loop keeps its
    // registers to itself
    auto run = [&](auto masked) {
      for (int it = 0; it < nqt; ++it) {
        const int qb = it & 3, nqb = (it + 1) & 3, q0 = qlo + it * KV_BQ;
        gload(q0 + KV_BQ);  // past the query range: zeros, never used
        keep_loads_early(it, nqb);
        f32x16_t x[2];
        phase1(Qs[qb], x);
        op8 w[4];
        silu_terms_rows_queries<T, decltype(masked)::value, A1>(x, w, Fx[it & 1][grp], lane, kexp, alpha, q0, kj, g,
                                                             s_end, r_end, Tq[qb], tk);
        swrite(nqb);
        phase2(w, stage_tile(Ds[0], it % 3));
        __syncthreads();
      }
    };
    if (full) run(std::false_type{});
    else run(std::true_type{});
    __syncthreads();  // the dA side's last stage
    __syncthreads();  // its last dK product
  } else {
    // iteration 0: only the dO rows of stage 1
    gload(qlo + KV_BQ);
    swrite(1);
    __syncthreads();
    op8 wp[4];  // dS operands of the previous stage, for its dK product
    for (int it = 1; it <= nqt; ++it) {
      const int st = it - 1, buf = st % 3, nbuf = (it + 1) % 3, q0 = qlo + st * KV_BQ;
      gload(qlo + (it + 1) * KV_BQ);  // past the query range: zeros, never used
      keep_loads_early(it, nbuf);
      if (it >= 2) phase2(wp, stage_tile(Qs[0], (st - 1) & 3));
      f32x16_t x[2];
      phase1(Ds[buf], x);
      swrite(nbuf);
      const uint32_t* fx = Fx[st & 1][grp];
      float d[2][16];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t fv = fx[(t * 8 + e) * 64 + lane];
          d[t][2 * e] = __builtin_fmaf(x[t][2 * e], from_bits16<f16_t>((uint16_t)(fv & 0xffff)), 0.0f);
          d[t][2 * e + 1] = __builtin_fmaf(x[t][2 * e + 1], from_bits16<f16_t>((uint16_t)(fv >> 16)), 0.0f);
        }
      op8 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = pack_kstep<T>(d, u);
      if (STORE) {
        // Non-temporal dS stores through a resource of size zero where
        // nothing is kept (rows beyond the dS buffer), never under a branch:
        // the wait before the stage write then covers only this iteration's
        // loads, not the stores, whose completion takes far longer.
        const int qs = (q0 - lo) >> 6;  // 64-row stage of the user's rows
        const __amdgpu_buffer_rsrc_t drs =
            make_rsrc(ds_on ? dsb + (qs >> 1) * ds_qt_stride + (qs & 1) * 8192 : dS, ds_on ? 4096 : 0);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, w[u].v), drs, lane * 16 + u * 1024, 0,
                                                 2 /* non-temporal */);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) wp[u] = w[u];
      __syncthreads();
    }
    if (nqt >= 1) phase2(wp, Qs[(nqt - 1) & 3]);
    __syncthreads();  // every read of the stage tiles done before the epilogue reuses the LDS
  }
  // producer holds dV, consumer dK; both scale by alpha * c
  wave_store_rows<T, NC>(sm.ep + wave * EP_FLOATS, acc, 0, lane, k0 + grp * 32, hi, alpha * scale,
                         producer ? dV : dK, lddkv, hc, producer ? zv : zk, ldz);
}

// ---------------------------------------------------------------------------
// backward, query-major from stored dS: dQ = alpha c dS K.
// ---------------------------------------------------------------------------
// dS layout.  For user b and head h the buffer holds n_t x n_t tiles of
// 128 queries x 128 keys (n_t = ceil(L / 128)), 32 KB each, at
//   ((P_b H + h n_t^2) + qt n_t + kt) * 32 KB,   P_b = sum_{b' < b} n_t(b')^2.
// Inside a tile, 16 KB per 64-key half; inside a half, 8 KB per 64-query
// stage; inside a stage, 4 KB per 32-key group, written by the dK/dV wave of
// that key group as its dK A operands: [k-step u][lane][16 B], lane = key
// (l32) + 32 g, the 16 bytes holding queries 16u + 8e + 4g + (0..3) for
// e = 0, 1.  Tiles the dK/dV pass does not visit (fully masked) are never
// written and never read.
//
// Each workgroup takes 128 queries (4 waves x 32) and walks 64-key steps:
// the 16 KB dS piece and the K rows go to LDS, dS is read back transposed
// (one query per lane) with the LDS transpose load and K as V^T-style tiles.
// LDS position of byte b of a 16 KB dS piece: address bits 6 <-> 10 and
// 7 <-> 9 exchanged, so that the 32 lanes of each half-wave of a transpose
// read (4 keys x 2 query quads x 2 query eighths x 2 sixteenths) land on 32
// distinct 8-byte bank slots, while the k-step and the second key quad of
// a read move only bits 8, 9 and 12 (plain immediate offsets).
__device__ __forceinline__ int ds_lds_pos(int b) {
  const int b6 = (b >> 6) & 1, b7 = (b >> 7) & 1, b9 = (b >> 9) & 1, b10 = (b >> 10) & 1;
  return (b & ~0x6c0) | (b10 << 6) | (b9 << 7) | (b7 << 9) | (b6 << 10);
}

template <typename T, int DH>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_stream(
    const uint16_t* __restrict__ K, int64_t ldqkv, const uint8_t* __restrict__ dS, int64_t ds_cap,
    const int64_t* __restrict__ tprefix, uint16_t* __restrict__ dQ, int64_t lddq,
    const uint16_t* __restrict__ zq, int64_t ldz, const int32_t* __restrict__ seg,
    const int2* __restrict__ tiles, const int32_t* __restrict__ ntiles, int H, float out_scale) {
  constexpr int NC = DH / 32;
  struct Smem {
    uint8_t Ss[2][16384];
    uint16_t Ks[2][QuadRows<DH>::SIZE];
  };
  __shared__ __attribute__((aligned(16))) union {
    Smem m;
    float ep[4 * EP_FLOATS];
  } sm;
  auto& Ss = sm.m.Ss;
  auto& Ks = sm.m.Ks;
  int tile, h;
  xcd_tile_head(blockIdx.x, H, tile, h);
  if (tile >= *ntiles) return;
  const int2 te = tiles[tile];
  const int b = te.x, q0 = te.y;
  const int lo = seg[b * 5 + 0], s_end = seg[b * 5 + 2], r_end = seg[b * 5 + 3], hi = seg[b * 5 + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), l32 = lane & 31, g = lane >> 5;
  const int hc = h * DH;
  const int nt = (hi - lo + 127) >> 7;
  const int qt = (q0 - lo) >> 7;
  const int64_t pb = tprefix[b];
  // a row whose dS did not fit the buffer (longer than the declared
  // maximum) is left to the recompute kernel launched after this one
  if (pb + (int64_t)nt * nt > ds_cap) return;
  const uint8_t* dsq = dS + (pb * H + (int64_t)h * nt * nt + (int64_t)qt * nt) * (int64_t)DS_TILE_BYTES;
  const int q_last = min(q0 + 128, hi) - 1;
  const int kv_end = key_end_for(q_last, s_end, r_end);
  // key tiles with k0 < r_end (static or real-time) come first; of the
  // candidate tiles only this query tile's own (the diagonal) is visible
  const int n_nc = (r_end - lo + 127) >> 7;
  const int end_a = min(kv_end, lo + 128 * n_nc);
  const int na = end_a > lo ? (end_a - lo + 63) >> 6 : 0;
  const int nb = qt >= n_nc ? (kv_end - q0 + 63) >> 6 : 0;
  const int nsteps = na + nb;
  const int rt_stage0 = (s_end - lo) >> 6;

  // Per-thread pieces of the 16 KB dS step: 16-byte chunk cidx + 256 i
  // (stage i >> 1).  The chunk of each lane is chosen so that the LDS
  // positions ds_lds_pos of the 16 lanes of each write group fall on 16
  // distinct 16-byte bank groups (lane bits 0-3 land on position bits 4-7);
  // lanes 0-1 of every quad still read one full 64-byte global segment.
  const int cidx = (lane & 3) | (((lane >> 4) & 3) << 2) | ((wave & 1) << 4) | (((lane >> 2) & 3) << 5) |
                   ((wave >> 1) << 7);
  // Loads of one 64-key step: the 16 KB dS piece (two 8 KB query stages)
  // and the 64 K rows.  Both go through range-checked buffer resources, so
  // that a stage the dK/dV pass never wrote, or a step past the last, reads
  // nothing and costs no branch: the loads stay straight-line code, and the
  // wait before a step's LDS writes covers only that step's loads.
  constexpr int LCH = DH / 32;
  struct StepRegs {
    u32x4_t s[4];
    uint4 k[LCH];
  };
  auto gload = [&](StepRegs& R, int it) {
    const bool live = it < nsteps;
    const int kpos = it < na ? lo + 64 * it : q0 + 64 * (it - na);
    const int kt = (kpos - lo) >> 7, half = ((kpos - lo) >> 6) & 1;
    const int k0 = lo + 128 * kt;
    const uint8_t* src = dsq + (int64_t)kt * DS_TILE_BYTES + half * 16384;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int st = 2 * qt + p;
      const bool avail = live && lo + 64 * st < hi && (k0 < s_end || k0 >= r_end || st >= rt_stage0);
      const __amdgpu_buffer_rsrc_t r = make_rsrc(avail ? src + 8192 * p : dS, avail ? 8192 : 0);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        R.s[2 * p + i] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, 16 * (cidx + 256 * i), 0, 2 /* non-temporal */));
    }
    tile_gload_rows<DH, 64>(R.k, K, ldqkv, live ? kpos : hi, hi, hc, tid);
  };
  const int wsw = ds_lds_pos(16 * cidx);
  auto swrite = [&](int buf, const StepRegs& R) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4_t*)(Ss[buf] + wsw + 4096 * i) = R.s[i];
    tile_swrite_swz<DH, 64>(Ks[buf], R.k, tid);
  };

  // transposed dS reads: lane 4r + c of quarter G supplies (key 4g + r of
  // the k-step half, queries 4c..4c+3 of the quarter's 16)
  const int G = lane >> 4, qi4 = lane & 15, rr = qi4 >> 2, cc = qi4 & 3;
  const int rd_base = ds_lds_pos((wave >> 1) * 8192 + (2 * (wave & 1) + (G & 1)) * 1024 + (cc & 1) * 512 +
                                 (cc >> 1) * 8 + (4 * g + rr) * 16);
  f32x16_t acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[c][j] = 0.f;
  TrAddr<DH> tra;
  tra.init(lane);

  // Two register sets alternate, so that a step's loads are issued two
  // steps ahead of the step that reads them: step it loads step it + 2 and
  // writes step it + 1 (loaded during step it - 1) to LDS.
  StepRegs R0, R1;
  gload(R0, 0);
  swrite(0, R0);
  gload(R1, 1);
  __syncthreads();
  auto step = [&](int it, StepRegs& Rl, const StepRegs& Rw) {
    gload(Rl, it + 2);
    const uint8_t* sb = Ss[it & 1] + rd_base;
    const uint16_t* kb = Ks[it & 1];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      // key 16 ks + 8 rd + 4 g + r: stored byte bits 12 (ks / 2), 8 (ks % 2)
      // and 7 (rd), the last at LDS bit 9
      const int off = (ks >> 1) * 4096 + (ks & 1) * 256;
      const uint2 lo2 = lds_read_tr16(sb + off);
      const uint2 hi2 = lds_read_tr16(sb + off + 512);
      op8 a;
      a.v[0] = lo2.x; a.v[1] = lo2.y; a.v[2] = hi2.x; a.v[3] = hi2.y;
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c] = mfma32<T>(a, tra.get(kb, ks, c), acc[c]);
    }
    swrite((it + 1) & 1, Rw);
    __syncthreads();
  };
  // Steps in pairs, with no branch between them (a branch there would make
  // the wait counts merged at the loop head wait for loads a step early);
  // for an odd count the last step of the last pair reads nothing (sizes
  // zero) and adds zero.
  for (int it = 0; it < nsteps; it += 2) {
    step(it, R0, R1);
    step(it + 1, R1, R0);
  }
  wave_store_rows<T, NC>(sm.ep + wave * EP_FLOATS, acc, 0, lane, q0 + wave * 32, hi, out_scale, dQ, lddq, hc, zq,
                         ldz);
}

// ---------------------------------------------------------------------------
// f32 kernels: one thread per (token, head), plain loops (parity workloads).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int find_user(const int32_t* __restrict__ seg, int B, int tok) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {  // last user whose start <= tok (skips empty users)
    int mid = (lo + hi + 1) >> 1;
    if (seg[mid * 5] <= tok) lo = mid; else hi = mid - 1;
  }
  while (lo > 0 && seg[lo * 5 + 4] <= tok) --lo;
  return lo;
}

__device__ __forceinline__ float sigmoid_precise(float x) { return 1.0f / (1.0f + expf(-x)); }

template <int DH>
__global__ void attn_fwd_f32(const float* __restrict__ Q, const float* __restrict__ K,
                             const float* __restrict__ V, int64_t ldqkv, float* __restrict__ O,
                             int64_t ldo, const int32_t* __restrict__ seg, int B, int64_t T,
                             const int64_t* __restrict__ ts, float alpha, float scale) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T) return;
  const int h = blockIdx.y, hc = h * DH;
  const int b = find_user(seg, B, (int)i);
  const int lo = seg[b * 5], s_end = seg[b * 5 + 2], r_end = seg[b * 5 + 3], hi = seg[b * 5 + 4];
  const int qi = (int)i;
  const int kend = key_end_for(qi, s_end, r_end);
  const int64_t tq = ts[qi];
  float q[DH], acc[DH];
  for (int e = 0; e < DH; ++e) { q[e] = Q[i * ldqkv + hc + e]; acc[e] = 0.f; }
  for (int kj = lo; kj < kend; ++kj) {
    if (!mask_visible(qi, kj, s_end, r_end, hi, tq, ts)) continue;
    float s = 0.f;
    for (int e = 0; e < DH; ++e) s += q[e] * K[(int64_t)kj * ldqkv + hc + e];
    s *= alpha;
    const float p = s * sigmoid_precise(s);
    for (int e = 0; e < DH; ++e) acc[e] += p * V[(int64_t)kj * ldqkv + hc + e];
  }
  for (int e = 0; e < DH; ++e) O[i * ldo + hc + e] = acc[e] * scale;
}

template <int DH>
__global__ void attn_bwd_dq_f32(const float* __restrict__ Q, const float* __restrict__ K,
                                const float* __restrict__ V, int64_t ldqkv, const float* __restrict__ dO,
                                int64_t lddo, float* __restrict__ dQ, int64_t lddq,
                                const float* __restrict__ zq, int64_t ldz, const int32_t* __restrict__ seg,
                                int B, int64_t T, const int64_t* __restrict__ ts, float alpha, float scale) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T) return;
  const int h = blockIdx.y, hc = h * DH;
  const int b = find_user(seg, B, (int)i);
  const int lo = seg[b * 5], s_end = seg[b * 5 + 2], r_end = seg[b * 5 + 3], hi = seg[b * 5 + 4];
  const int qi = (int)i;
  const int kend = key_end_for(qi, s_end, r_end);
  const int64_t tq = ts[qi];
  float q[DH], d[DH], acc[DH];
  for (int e = 0; e < DH; ++e) { q[e] = Q[i * ldqkv + hc + e]; d[e] = dO[i * lddo + hc + e]; acc[e] = 0.f; }
  for (int kj = lo; kj < kend; ++kj) {
    if (!mask_visible(qi, kj, s_end, r_end, hi, tq, ts)) continue;
    float s = 0.f, da = 0.f;
    for (int e = 0; e < DH; ++e) {
      s += q[e] * K[(int64_t)kj * ldqkv + hc + e];
      da += d[e] * V[(int64_t)kj * ldqkv + hc + e];
    }
    s *= alpha;
    const float w = da * silu_grad_from(s, sigmoid_precise(s));
    for (int e = 0; e < DH; ++e) acc[e] += w * K[(int64_t)kj * ldqkv + hc + e];
  }
  for (int e = 0; e < DH; ++e) {
    float v = acc[e] * alpha * scale;
    if (zq) {
      v *= zq[i * ldz + hc + e];
    }
    dQ[i * lddq + hc + e] = v;
  }
}

template <int DH>
__global__ void attn_bwd_dkdv_f32(const float* __restrict__ Q, const float* __restrict__ K,
                                  const float* __restrict__ V, int64_t ldqkv,
                                  const float* __restrict__ dO, int64_t lddo, float* __restrict__ dK,
                                  float* __restrict__ dV, int64_t lddkv, const float* __restrict__ zk,
                                  const float* __restrict__ zv, int64_t ldz,
                                  const int32_t* __restrict__ seg, int B, int64_t T,
                                  const int64_t* __restrict__ ts, float alpha, float scale) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T) return;
  const int h = blockIdx.y, hc = h * DH;
  const int b = find_user(seg, B, (int)i);
  const int lo = seg[b * 5], s_end = seg[b * 5 + 2], r_end = seg[b * 5 + 3], hi = seg[b * 5 + 4];
  const int kj = (int)i;
  float k[DH], v[DH], ak[DH], av[DH];
  for (int e = 0; e < DH; ++e) {
    k[e] = K[i * ldqkv + hc + e];
    v[e] = V[i * ldqkv + hc + e];
    ak[e] = av[e] = 0.f;
  }
  for (int qi = lo; qi < hi; ++qi) {
    if (!mask_visible(qi, kj, s_end, r_end, hi, ts[qi], ts)) continue;
    float s = 0.f, da = 0.f;
    for (int e = 0; e < DH; ++e) {
      s += Q[(int64_t)qi * ldqkv + hc + e] * k[e];
      da += dO[(int64_t)qi * lddo + hc + e] * v[e];
    }
    s *= alpha;
    const float sg = sigmoid_precise(s);
    const float p = s * sg, w = da * silu_grad_from(s, sg);
    for (int e = 0; e < DH; ++e) {
      av[e] += p * dO[(int64_t)qi * lddo + hc + e];
      ak[e] += w * Q[(int64_t)qi * ldqkv + hc + e];
    }
  }
  for (int e = 0; e < DH; ++e) {
    float a = ak[e] * alpha * scale, bv = av[e] * scale;
    if (zk) {
      a *= zk[i * ldz + hc + e];
      bv *= zv[i * ldz + hc + e];
    }
    dK[i * lddkv + hc + e] = a;
    dV[i * lddkv + hc + e] = bv;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename T, int DH>
static void fwd_mfma(const AttnArgs& a, const PrepView& pv, hipStream_t st) {
  // SiLU(alpha s) = alpha * s * sigmoid(alpha s); sigmoid via exp2 with the
  // factor -alpha*log2(e) folded in; alpha and the normaliser scale O once.
  const float kexp = -a.alpha * 1.4426950408889634f;
  const unsigned base = xcd_grid(pv.q.max_tiles, a.H);
  const int ns = a.part ? a.nsplit : 1;
  {
    ProfScope ps("attn_fwd", st);
    hipLaunchKernelGGL((attn_fwd_mfma<T, DH>), dim3(base * ns), dim3(256), 0, st, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, a.ldqkv, (uint16_t*)a.o, a.ldo, pv.seg, a.ts,
                       pv.q.tiles, pv.q.ntiles, a.H, kexp, a.alpha * a.scale, ns, (int)base, a.part, a.T);
  }
}

int attn_fwd_splits(int dt, int B, int64_t T, int H) {
  if (dt == MTGR_F32 || B <= 0 || T <= 0) return 1;
  // two forward workgroups fit on each of the 256 compute units
  const int64_t wgs = (int64_t)xcd_grid(max_tiles(B, T, ATTN_QTILE), H);
  if (wgs >= 512) return 1;
  const int64_t s = (512 + wgs - 1) / wgs;
  return (int)(s < ATTN_MAX_SPLITS ? s : ATTN_MAX_SPLITS);
}

size_t attn_fwd_part_bytes(int dt, int B, int64_t T, int H, int dh) {
  const int s = attn_fwd_splits(dt, B, T, H);
  return s > 1 ? (size_t)s * (size_t)T * (size_t)H * dh * sizeof(float) : 0;
}

template <typename T, int DH>
static void bwd_mfma(const AttnArgs& a, const PrepView& pv, hipStream_t st) {
  const float kexp = -a.alpha * 1.4426950408889634f;
  {
    ProfScope ps("attn_bwd_dkdv", st);
    // alpha = 1 (the layer's default) saves one multiply per score of the
    // S side's vector work, which bounds the kernel (1-2% of its time)
    if (a.ds && a.alpha == 1.0f)
      hipLaunchKernelGGL((attn_bwd_dkdv_mfma<T, DH, true, true>), dim3(xcd_grid(pv.k.max_tiles, a.H)), dim3(512), 0,
                         st, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.ldqkv,
                         (const uint16_t*)a.d_o, a.lddo, (uint16_t*)a.dk, (uint16_t*)a.dv, a.lddqkv,
                         (const uint16_t*)a.zk, (const uint16_t*)a.zv, a.ldz, pv.seg, a.ts, pv.k.tiles,
                         pv.k.ntiles, a.H, kexp, a.alpha, a.scale, (uint8_t*)a.ds, a.ds_cap,
                         (const int64_t*)pv.tprefix);
    else if (a.ds)
      hipLaunchKernelGGL((attn_bwd_dkdv_mfma<T, DH, true>), dim3(xcd_grid(pv.k.max_tiles, a.H)), dim3(512), 0,
                         st, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.ldqkv,
                         (const uint16_t*)a.d_o, a.lddo, (uint16_t*)a.dk, (uint16_t*)a.dv, a.lddqkv,
                         (const uint16_t*)a.zk, (const uint16_t*)a.zv, a.ldz, pv.seg, a.ts, pv.k.tiles,
                         pv.k.ntiles, a.H, kexp, a.alpha, a.scale, (uint8_t*)a.ds, a.ds_cap,
                         (const int64_t*)pv.tprefix);
    else
      hipLaunchKernelGGL((attn_bwd_dkdv_mfma<T, DH, false>), dim3(xcd_grid(pv.k.max_tiles, a.H)), dim3(512), 0,
                         st, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.ldqkv,
                         (const uint16_t*)a.d_o, a.lddo, (uint16_t*)a.dk, (uint16_t*)a.dv, a.lddqkv,
                         (const uint16_t*)a.zk, (const uint16_t*)a.zv, a.ldz, pv.seg, a.ts, pv.k.tiles,
                         pv.k.ntiles, a.H, kexp, a.alpha, a.scale, nullptr, (int64_t)0, (const int64_t*)nullptr);
  }
  if (a.ds) {
    {
      ProfScope ps("attn_bwd_dq", st);
      hipLaunchKernelGGL((attn_bwd_dq_stream<T, DH>), dim3(xcd_grid(pv.q.max_tiles, a.H)), dim3(256), 0, st,
                         (const uint16_t*)a.k, a.ldqkv, (const uint8_t*)a.ds, a.ds_cap,
                         (const int64_t*)pv.tprefix, (uint16_t*)a.dq, a.lddqkv, (const uint16_t*)a.zq, a.ldz,
                         pv.seg, pv.q.tiles, pv.q.ntiles, a.H, a.alpha * a.scale);
    }
    // rows longer than the declared maximum, whose dS did not fit
    ProfScope ps("attn_bwd_dq_rest", st);
    const int64_t items = (int64_t)pv.q.max_tiles * a.H;
    const int grid = (int)std::min<int64_t>(256, (items + 511) / 512);
    if (grid > 0)
      hipLaunchKernelGGL((attn_bwd_dq_overflow<T, DH>), dim3(grid), dim3(512), 0, st, (const uint16_t*)a.q,
                         (const uint16_t*)a.k, (const uint16_t*)a.v, a.ldqkv, (const uint16_t*)a.d_o, a.lddo,
                         (uint16_t*)a.dq, a.lddqkv, (const uint16_t*)a.zq, a.ldz, pv.seg, a.ts, pv.q.tiles,
                         pv.q.ntiles, a.H, kexp, a.alpha, a.alpha * a.scale, (const int64_t*)pv.tprefix, a.ds_cap);
    return;
  }
  ProfScope ps("attn_bwd_dq", st);
  hipLaunchKernelGGL((attn_bwd_dq_mfma<T, DH>), dim3(xcd_grid(pv.q.max_tiles, a.H)), dim3(512), 0, st,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.ldqkv,
                     (const uint16_t*)a.d_o, a.lddo, (uint16_t*)a.dq, a.lddqkv, (const uint16_t*)a.zq, a.ldz, pv.seg,
                     a.ts, pv.q.tiles, pv.q.ntiles, a.H, kexp, a.alpha, a.alpha * a.scale);
}

template <int DH>
static void fwd_f32(const AttnArgs& a, const PrepView& pv, hipStream_t st) {
  dim3 grid((unsigned)((a.T + 63) / 64), a.H);
  hipLaunchKernelGGL((attn_fwd_f32<DH>), grid, dim3(64), 0, st, (const float*)a.q, (const float*)a.k,
                     (const float*)a.v, a.ldqkv, (float*)a.o, a.ldo, pv.seg, a.B, a.T, a.ts, a.alpha, a.scale);
}

template <int DH>
static void bwd_f32(const AttnArgs& a, const PrepView& pv, hipStream_t st) {
  dim3 grid((unsigned)((a.T + 63) / 64), a.H);
  hipLaunchKernelGGL((attn_bwd_dq_f32<DH>), grid, dim3(64), 0, st, (const float*)a.q, (const float*)a.k,
                     (const float*)a.v, a.ldqkv, (const float*)a.d_o, a.lddo, (float*)a.dq, a.lddqkv,
                     (const float*)a.zq, a.ldz, pv.seg, a.B, a.T, a.ts, a.alpha, a.scale);
  hipLaunchKernelGGL((attn_bwd_dkdv_f32<DH>), grid, dim3(64), 0, st, (const float*)a.q, (const float*)a.k,
                     (const float*)a.v, a.ldqkv, (const float*)a.d_o, a.lddo, (float*)a.dk, (float*)a.dv,
                     a.lddqkv, (const float*)a.zk, (const float*)a.zv, a.ldz, pv.seg, a.B, a.T, a.ts,
                     a.alpha, a.scale);
}

size_t attn_ds_bytes(int B, int64_t T, int max_len, int H) {
  if (B <= 0 || T <= 0 || max_len <= 0 || H <= 0) return 0;
  const int64_t M = max_len < T ? max_len : T;
  const int64_t ntm = (M + 127) / 128;
  const int64_t by_rows = (int64_t)B * ntm * ntm;
  const int64_t by_tokens = (M * T + 254 * T + 16129 * (int64_t)B + 16383) / 16384;
  const int64_t tiles = by_rows < by_tokens ? by_rows : by_tokens;
  return align_up((size_t)tiles * H * DS_TILE_BYTES, 256);
}

int launch_attn_fwd(int dt, const AttnArgs& a, const PrepView& pv, hipStream_t st) {
  if (a.T <= 0 || a.B <= 0) return MTGR_OK;
  if (dt == MTGR_BF16) {
    if (a.dh == 128) fwd_mfma<bf16_t, 128>(a, pv, st);
    else if (a.dh == 64) fwd_mfma<bf16_t, 64>(a, pv, st);
    else if (a.dh == 32) fwd_mfma<bf16_t, 32>(a, pv, st);
    else return MTGR_ERR_UNSUPPORTED;
  } else if (dt == MTGR_F16) {
    if (a.dh == 128) fwd_mfma<f16_t, 128>(a, pv, st);
    else if (a.dh == 64) fwd_mfma<f16_t, 64>(a, pv, st);
    else if (a.dh == 32) fwd_mfma<f16_t, 32>(a, pv, st);
    else return MTGR_ERR_UNSUPPORTED;
  } else if (dt == MTGR_F32) {
    switch (a.dh) {
      case 16: fwd_f32<16>(a, pv, st); break;
      case 32: fwd_f32<32>(a, pv, st); break;
      case 64: fwd_f32<64>(a, pv, st); break;
      case 128: fwd_f32<128>(a, pv, st); break;
      default: return MTGR_ERR_UNSUPPORTED;
    }
  } else {
    return MTGR_ERR_UNSUPPORTED;
  }
  MTGR_LAUNCH_CHECK();
  return MTGR_OK;
}

int launch_attn_bwd(int dt, const AttnArgs& a, const PrepView& pv, hipStream_t st) {
  if (a.T <= 0 || a.B <= 0) return MTGR_OK;
  if (dt == MTGR_BF16) {
    if (a.dh == 128) bwd_mfma<bf16_t, 128>(a, pv, st);
    else if (a.dh == 64) bwd_mfma<bf16_t, 64>(a, pv, st);
    else if (a.dh == 32) bwd_mfma<bf16_t, 32>(a, pv, st);
    else return MTGR_ERR_UNSUPPORTED;
  } else if (dt == MTGR_F16) {
    if (a.dh == 128) bwd_mfma<f16_t, 128>(a, pv, st);
    else if (a.dh == 64) bwd_mfma<f16_t, 64>(a, pv, st);
    else if (a.dh == 32) bwd_mfma<f16_t, 32>(a, pv, st);
    else return MTGR_ERR_UNSUPPORTED;
  } else if (dt == MTGR_F32) {
    switch (a.dh) {
      case 16: bwd_f32<16>(a, pv, st); break;
      case 32: bwd_f32<32>(a, pv, st); break;
      case 64: bwd_f32<64>(a, pv, st); break;
      case 128: bwd_f32<128>(a, pv, st); break;
      default: return MTGR_ERR_UNSUPPORTED;
    }
  } else {
    return MTGR_ERR_UNSUPPORTED;
  }
  MTGR_LAUNCH_CHECK();
  return MTGR_OK;
}

}  // namespace mtgr
