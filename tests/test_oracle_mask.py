"""Pins of the oracle's dynamic mask and jagged segments against values fixed
by the pages (worked example), hand-written tables and closed-form counts."""

import json
import os

import numpy as np
import pytest

from mtgr_inputs import make_batch, make_batch_from_lengths
from oracle import mtgr_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("fixture", ["mask_worked_example.json", "mask_toy_ties.json"])
def test_mask_matches_hand_written_table(fixture):
    fx = _load(fixture)
    g = np.array([t["group"] for t in fx["tokens"]], dtype=np.uint8)
    ts = np.array([t["ts"] for t in fx["tokens"]], dtype=np.int64)
    want = np.array(fx["mask_rows_query_cols_key"], dtype=bool)
    got = orc.mask_matrix(g, ts)
    assert got.dtype == bool
    np.testing.assert_array_equal(got, want)


def test_worked_example_statement():
    """The sentence of the worked example itself: scoring B (12:30) must not
    see the 13:00 click, and may see the 12:00 one."""
    fx = _load("mask_worked_example.json")
    names = [t["name"] for t in fx["tokens"]]
    g = np.array([t["group"] for t in fx["tokens"]], dtype=np.uint8)
    ts = np.array([t["ts"] for t in fx["tokens"]], dtype=np.int64)
    M = orc.mask_matrix(g, ts)
    b = names.index("cand_B_1230")
    assert not M[b, names.index("RT_click_C_1300")]
    assert M[b, names.index("RT_click_A_1200")]
    # candidates never see each other
    for i in range(5, 8):
        for j in range(5, 8):
            assert M[i, j] == (i == j)


def _closed_form_pairs(lengths, ts_user):
    """P = N (n_u + n_s) + sum over RT keys r of [1 + #{RT q: t_q > t_r}
    + #{cand c: t_c > t_r}] + n_c, counted independently of the matrix."""
    n_u, n_s, n_r, n_c = (int(v) for v in lengths)
    N = n_u + n_s + n_r + n_c
    rt = ts_user[n_u + n_s:n_u + n_s + n_r]
    cand = ts_user[n_u + n_s + n_r:]
    total = N * (n_u + n_s) + n_c
    for t_r in rt:
        total += 1 + int(np.sum(rt > t_r)) + int(np.sum(cand > t_r))
    return total


@pytest.mark.parametrize("cfg", [1, 2])
def test_visible_pair_count_closed_form(cfg):
    batch = make_batch(cfg)
    users = range(batch.B) if cfg == 1 else range(0, batch.B, 5)
    got = orc.visible_pairs(batch.offsets, batch.group_ids, batch.timestamps)
    for b in users:
        lo, hi = batch.offsets[b], batch.offsets[b + 1]
        assert got[b] == _closed_form_pairs(batch.lengths[b], batch.timestamps[lo:hi])


def test_segments_from_lengths():
    rng = np.random.default_rng(5)
    lengths = [[8, 20, 0, 3], [2, 0, 5, 0], [0, 0, 0, 1], [8, 100, 64, 20], [0, 0, 0, 0]]
    batch = make_batch_from_lengths(lengths, rng, ts_max=50)
    seg = orc.segments(batch.offsets, batch.group_ids)
    start = 0
    for b, (n_u, n_s, n_r, n_c) in enumerate(lengths):
        want = [start, start + n_u, start + n_u + n_s, start + n_u + n_s + n_r,
                start + n_u + n_s + n_r + n_c]
        assert seg[b].tolist() == want
        start = want[-1]


def test_static_queries_see_only_static():
    batch = make_batch(1)
    for b in range(batch.B):
        lo, hi = batch.offsets[b], batch.offsets[b + 1]
        g = batch.group_ids[lo:hi]
        M = orc.mask_matrix(g, batch.timestamps[lo:hi])
        static = g <= 1
        assert M[np.ix_(static, static)].all()
        assert not M[np.ix_(static, ~static)].any()
        # every token sees itself
        assert np.diag(M).all()
