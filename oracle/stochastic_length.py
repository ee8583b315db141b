"""Plain CPU oracle of Stochastic Length sampling and the token-budget cut.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module; only the tests and the benchmark's CPU-baseline leg do.  It
shares no code with the HIP kernels; the per-user random numbers come from
``mtgr_inputs.make_uniform_draws`` and are passed to both sides.

Source: "MTGR：美团外卖生成式推荐Scaling Law落地实践" (paper-daily summary),
section 计算量涨了 65 倍，训练成本怎么压住: in training, a long user sequence is
shortened by drawing a random segment of it, while online scoring keeps the
full sequence; with it the large model trains at about the baseline's cost
instead of 2.1 times.  Token-balanced batches: "MTGR：工业级生成式推荐框架"
(zzxanthony blog) 11.3, batches sized by token count.

Readings taken where the pages are silent (also listed in the design notes):
  * The long sequence is the history S; profile (U), real-time (R) and
    candidate (C) tokens are always kept, in order.
  * "A segment" is a contiguous window of s_keep history tokens, in order;
    histories of at most s_keep tokens are unchanged.
  * The window start is uniform over the n_s - s_keep + 1 possible starts:
    start = min(floor(u * (n_s - s_keep + 1)), n_s - s_keep) for the user's
    draw u in [0, 1), the product taken in float32 (the integer decision is
    made in the kernel's precision).
  * The batch after sampling is the longest prefix of the (shortened) users
    whose tokens fit the budget.
"""

from __future__ import annotations

from typing import Tuple

import numpy as np

from .mtgr_oracle import GROUP_C, GROUP_R, GROUP_S, GROUP_U


def window_start(u: float, n_s: int, s_keep: int) -> int:
    """First kept history position (0-based within S) for draw u."""
    m = int(n_s) - int(s_keep)
    if m <= 0:
        return 0
    prod = np.float32(u) * np.float32(m + 1)  # one IEEE float32 multiply
    return min(int(np.floor(prod)), m)


def stochastic_length(offsets, group_ids, timestamps, x, u, s_keep: int):
    """Shortened batch: (offsets, group_ids, timestamps, x), users in order.

    Each user's tokens are taken group by group: all U rows, then the window
    of S rows, then all R rows, then all C rows."""
    offsets = np.asarray(offsets, dtype=np.int64)
    g = np.asarray(group_ids)
    ts = np.asarray(timestamps)
    x = np.asarray(x)
    B = offsets.shape[0] - 1
    keep_rows = []
    new_off = [0]
    for b in range(B):
        rows = np.arange(offsets[b], offsets[b + 1])
        gb = g[rows]
        U, S, R, C = (rows[gb == k] for k in (GROUP_U, GROUP_S, GROUP_R, GROUP_C))
        if len(S) > s_keep:
            st = window_start(u[b], len(S), s_keep)
            S = S[st:st + s_keep]
        kept = np.concatenate([U, S, R, C])
        keep_rows.append(kept)
        new_off.append(new_off[-1] + len(kept))
    idx = np.concatenate(keep_rows) if keep_rows else np.zeros(0, dtype=np.int64)
    return (np.asarray(new_off, dtype=np.int32), g[idx].copy(), ts[idx].copy(), x[idx].copy())


def budget_fit(offsets, budget: int) -> Tuple[int, int]:
    """(users, tokens) of the longest prefix of users holding at most
    ``budget`` tokens."""
    offsets = np.asarray(offsets, dtype=np.int64)
    b = 0
    while b + 1 < offsets.shape[0] and offsets[b + 1] <= budget:
        b += 1
    return b, int(offsets[b])
