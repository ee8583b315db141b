"""CPU pins of the Stochastic Length oracle (oracle/stochastic_length.py).

Each check is fixed by the definition, not by the oracle's own code: rows are
tagged with their original index so that kept rows can be traced back; the
window bounds come from the extremes of the draw; the start distribution is
checked on an equidistributed grid of draws; the budget cut against a sorted
search."""

import numpy as np
import pytest

from mtgr_inputs import make_batch_from_lengths, make_uniform_draws, make_user_pool
from oracle import stochastic_length as sl

U_, S_, R_, C_ = 0, 1, 2, 3


def tagged(batch, d=4):
    """Features whose column 0 is the original row index."""
    x = np.zeros((batch.T, d), dtype=np.float32)
    x[:, 0] = np.arange(batch.T)
    x[:, 1:] = np.random.default_rng(3).normal(size=(batch.T, d - 1))
    return x


def rows_of(off, g, b, grp):
    lo, hi = int(off[b]), int(off[b + 1])
    return np.arange(lo, hi)[np.asarray(g[lo:hi]) == grp]


def check_structure(batch, x, u, s_keep):
    off, g, ts, xo = sl.stochastic_length(batch.offsets, batch.group_ids, batch.timestamps, x, u, s_keep)
    assert off[0] == 0 and np.all(np.diff(off) >= 0) and off[-1] == len(g) == len(ts) == len(xo)
    src = xo[:, 0].astype(np.int64)
    # every kept row carries its own group id, timestamp and features
    np.testing.assert_array_equal(g, batch.group_ids[src])
    np.testing.assert_array_equal(ts, batch.timestamps[src])
    np.testing.assert_array_equal(xo, x[src])
    starts = []
    for b in range(batch.B):
        got = src[off[b]:off[b + 1]]
        n = {k: len(rows_of(batch.offsets, batch.group_ids, b, k)) for k in (U_, S_, R_, C_)}
        gu = got[:n[U_]]
        np.testing.assert_array_equal(gu, rows_of(batch.offsets, batch.group_ids, b, U_))
        ns_new = min(n[S_], s_keep)
        gs = got[n[U_]:n[U_] + ns_new]
        s_rows = rows_of(batch.offsets, batch.group_ids, b, S_)
        if ns_new:
            # a contiguous run of the original history, in order
            assert np.all(np.diff(gs) == 1)
            assert gs[0] >= s_rows[0] and gs[-1] <= s_rows[-1]
            starts.append(int(gs[0] - s_rows[0]))
        else:
            starts.append(None)
        rest = got[n[U_] + ns_new:]
        np.testing.assert_array_equal(rest, np.concatenate([rows_of(batch.offsets, batch.group_ids, b, R_),
                                                            rows_of(batch.offsets, batch.group_ids, b, C_)]))
        assert len(got) == n[U_] + ns_new + n[R_] + n[C_]
    return off, starts


def small_batch():
    rng = np.random.default_rng(5)
    lengths = [[8, 40, 5, 3], [8, 3, 0, 2], [0, 0, 0, 0], [2, 0, 4, 1], [8, 17, 9, 0], [0, 25, 0, 6]]
    return make_batch_from_lengths(lengths, rng, ts_max=1000)


def test_identity_when_every_history_fits():
    batch = small_batch()
    x = tagged(batch)
    u = make_uniform_draws(batch.B, seed=1)
    off, g, ts, xo = sl.stochastic_length(batch.offsets, batch.group_ids, batch.timestamps, x, u, 40)
    np.testing.assert_array_equal(off, batch.offsets)
    np.testing.assert_array_equal(g, batch.group_ids)
    np.testing.assert_array_equal(ts, batch.timestamps)
    np.testing.assert_array_equal(xo, x)


@pytest.mark.parametrize("s_keep", [0, 1, 3, 16, 24])
def test_structure_small(s_keep):
    batch = small_batch()
    x = tagged(batch)
    u = make_uniform_draws(batch.B, seed=2)
    check_structure(batch, x, u, s_keep)


def test_structure_on_a_pool_of_long_tail_users():
    batch = make_user_pool(4, 20000, seed=0)
    x = tagged(batch)
    u = make_uniform_draws(batch.B, seed=3)
    off, starts = check_structure(batch, x, u, 256)
    assert off[-1] < batch.T  # long histories were cut


def test_window_extremes():
    """u = 0 keeps the first s_keep history tokens; the largest float32 below
    1 keeps the last ones."""
    top = np.nextafter(np.float32(1), np.float32(0))
    for s_keep in (1, 17, 256, 512):
        for n_s in (s_keep + 1, s_keep + 2, 1000, 2999, 3000):
            assert sl.window_start(np.float32(0), n_s, s_keep) == 0
            assert sl.window_start(top, n_s, s_keep) == n_s - s_keep


def test_starts_are_equidistributed():
    """n_s = 10, s_keep = 4: seven possible starts; on 7000 evenly spaced draws
    each start is taken exactly 1000 times."""
    u = ((np.arange(7000) + 0.5) / 7000).astype(np.float32)
    starts = np.array([sl.window_start(v, 10, 4) for v in u])
    np.testing.assert_array_equal(np.bincount(starts, minlength=7), np.full(7, 1000))


def test_budget_fit_against_sorted_search():
    rng = np.random.default_rng(8)
    for _ in range(50):
        sizes = rng.integers(0, 50, size=rng.integers(1, 30))
        off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        for budget in (0, int(off[-1]), int(off[-1]) + 5, int(rng.integers(0, off[-1] + 1))):
            b, t = sl.budget_fit(off, budget)
            want = int(np.searchsorted(off, budget, side="right")) - 1
            assert b == want and t == off[want]
