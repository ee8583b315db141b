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
