"""Work counts used to report throughput (host-side metadata arithmetic).

Visible pairs of one user row [U | S | R | C] under the dynamic mask
(fun-rec 7.3.4 rules 1-3): every token sees the n_u + n_s static tokens;
a real-time token r is seen by itself and by every real-time or candidate
token stamped strictly later; a candidate is seen only by itself.
"""

from __future__ import annotations

import numpy as np


def visible_pairs(offsets: np.ndarray, group_ids: np.ndarray, timestamps: np.ndarray) -> int:
    offsets = np.asarray(offsets, dtype=np.int64)
    g = np.asarray(group_ids)
    t = np.asarray(timestamps)
    total = 0
    for b in range(offsets.shape[0] - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        gb, tb = g[lo:hi], t[lo:hi]
        N = hi - lo
        n_static = int(np.count_nonzero(gb <= 1))
        rt = np.sort(tb[gb == 2])
        dyn_t = np.sort(tb[(gb == 2) | (gb == 3)])
        n_c = int(np.count_nonzero(gb == 3))
        # for each RT key: 1 (itself) + number of dynamic tokens stamped later
        later = dyn_t.shape[0] - np.searchsorted(dyn_t, rt, side="right")
        total += N * n_static + int(rt.shape[0] + later.sum()) + n_c
    return total


def attention_flops(offsets, group_ids, timestamps, d: int):
    """(forward, backward) algorithmic flops: 4 d P and 8 d P for P visible pairs."""
    P = visible_pairs(offsets, group_ids, timestamps)
    return 4 * d * P, 8 * d * P


def layer_gemm_flops(T: int, d: int, backward: bool) -> int:
    """UQKV (8 T d^2) and output (2 T d^2) projections; backward doubles each."""
    f = 10 * T * d * d
    return 3 * f if backward else f


def ds_stream_bytes(offsets, group_ids, heads: int) -> int:
    """Bytes of stored 16-bit score gradients the dQ pass streams: per
    128-query tile it visits 64-key steps over the keys its queries can see
    (static and real-time key tiles, plus the candidate tile on the
    diagonal), 16 KB per step and head."""
    offsets = np.asarray(offsets, dtype=np.int64)
    g = np.asarray(group_ids)
    steps = 0
    for b in range(offsets.shape[0] - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        if hi <= lo:
            continue
        gb = g[lo:hi]
        s_end = lo + int(np.count_nonzero(gb <= 1))
        r_end = s_end + int(np.count_nonzero(gb == 2))
        n_nc = (r_end - lo + 127) // 128
        for q0 in range(lo, hi, 128):
            qt = (q0 - lo) // 128
            q_last = min(q0 + 128, hi) - 1
            kv_end = s_end if q_last < s_end else (r_end if q_last < r_end else q_last + 1)
            end_a = min(kv_end, lo + 128 * n_nc)
            na = (end_a - lo + 63) // 64 if end_a > lo else 0
            nb = (kv_end - q0 + 63) // 64 if qt >= n_nc else 0
            steps += na + nb
    return steps * 16384 * heads
