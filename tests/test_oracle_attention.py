"""Pins of the oracle's masked SiLU attention: per-element brute force on tiny
inputs, torch's SiLU, closed forms, padded (per-user) computation, the
invariants the dynamic mask promises, and finite differences for the
backward."""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from mtgr_inputs import make_batch, make_batch_from_lengths
from oracle import mtgr_oracle as orc


def _qkv(T, d, seed, scale=0.5):
    rng = np.random.default_rng(seed)
    return [rng.normal(0, scale, size=(T, d)) for _ in range(3)]


def test_silu_and_grad_match_torch():
    z = np.linspace(-30, 30, 2001)
    zt = torch.tensor(z, requires_grad=True)
    s = F.silu(zt)
    s.sum().backward()
    np.testing.assert_allclose(orc.silu(z), s.detach().numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(orc.silu_grad(z), zt.grad.numpy(), rtol=1e-12, atol=1e-14)


def _brute_force(q, k, v, batch, H, alpha, scale):
    """Scalar loops straight from the rules: key group, query group,
    timestamps and token identity decide visibility."""
    T, d = q.shape
    dh = d // H
    o = np.zeros((T, d))
    g = batch.group_ids
    t = batch.timestamps
    for b in range(batch.B):
        lo, hi = int(batch.offsets[b]), int(batch.offsets[b + 1])
        for i in range(lo, hi):
            for j in range(lo, hi):
                if g[j] in (0, 1):
                    vis = True
                elif g[j] == 2:
                    vis = g[i] in (2, 3) and (t[j] < t[i] or i == j)
                else:
                    vis = i == j
                if not vis:
                    continue
                for h in range(H):
                    s = alpha * sum(q[i, h * dh + e] * k[j, h * dh + e] for e in range(dh))
                    w = s / (1.0 + math.exp(-s))
                    for e in range(dh):
                        o[i, h * dh + e] += scale * w * v[j, h * dh + e]
    return o


def test_attention_matches_brute_force():
    rng = np.random.default_rng(11)
    lengths = [[2, 3, 4, 3], [1, 0, 3, 2], [0, 4, 0, 1]]
    batch = make_batch_from_lengths(lengths, rng, ts_max=6)  # small range: ties
    H, d = 2, 8
    q, k, v = _qkv(batch.T, d, 12)
    got = orc.hstu_attention(q, k, v, batch.offsets, batch.group_ids, batch.timestamps,
                             H, 0.7, 0.25)
    want = _brute_force(q, k, v, batch, H, 0.7, 0.25)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_constant_scores_count_visible_keys():
    """With every score equal to s and v = 1, O_i = scale * SiLU(s) * (number
    of keys token i may see): the mask's row sums, through the attention."""
    batch = make_batch(1)
    H, d = 2, 64
    dh = d // H
    q = np.full((batch.T, d), 1.0)
    k = np.full((batch.T, d), 1.0 / dh)  # <q,k> = 1 per head
    v = np.ones((batch.T, d))
    o = orc.hstu_attention(q, k, v, batch.offsets, batch.group_ids, batch.timestamps, H, 1.0, 1.0)
    silu1 = 1.0 / (1.0 + math.exp(-1.0))
    for b in range(batch.B):
        lo, hi = batch.offsets[b], batch.offsets[b + 1]
        n_u, n_s, n_r, n_c = batch.lengths[b]
        ts = batch.timestamps[lo:hi]
        rt = ts[n_u + n_s:n_u + n_s + n_r]
        for i in range(hi - lo):
            if i < n_u + n_s:
                cnt = n_u + n_s
            elif i < n_u + n_s + n_r:
                cnt = n_u + n_s + int(np.sum(rt < ts[i])) + 1
            else:
                cnt = n_u + n_s + int(np.sum(rt < ts[i])) + 1
            np.testing.assert_allclose(o[lo + i], silu1 * cnt, rtol=1e-13)


def test_all_static_user_is_dense_silu_attention():
    """No real-time tokens and no candidates: every pair is visible, so the
    result is scale * SiLU(alpha Q K^T) V with torch's SiLU and matmul."""
    rng = np.random.default_rng(3)
    batch = make_batch_from_lengths([[3, 17, 0, 0]], rng, ts_max=10)
    q, k, v = _qkv(batch.T, 16, 4)
    got = orc.hstu_attention(q, k, v, batch.offsets, batch.group_ids, batch.timestamps, 2, 1.3, 0.1)
    qt, kt, vt = (torch.from_numpy(a).view(-1, 2, 8).transpose(0, 1) for a in (q, k, v))
    ref = 0.1 * torch.matmul(F.silu(1.3 * torch.matmul(qt, kt.transpose(1, 2))), vt)
    np.testing.assert_allclose(got, ref.transpose(0, 1).reshape(-1, 16).numpy(), rtol=1e-12)


def test_jagged_equals_padded():
    """Jagged result equals a padded [B, Nmax] computation with pad keys
    masked out and pad queries dropped."""
    batch = make_batch(1)
    H, d = 2, 64
    q, k, v = _qkv(batch.T, d, 7)
    got = orc.hstu_attention(q, k, v, batch.offsets, batch.group_ids, batch.timestamps, H, 1.0, 0.05)
    Nmax = batch.max_len
    for b in range(batch.B):
        lo, hi = batch.offsets[b], batch.offsets[b + 1]
        n = hi - lo
        pad = lambda a: np.concatenate([a[lo:hi], np.full((Nmax - n,) + a.shape[1:], 7.0)])
        gp = np.concatenate([batch.group_ids[lo:hi], np.zeros(Nmax - n, np.uint8)])
        tp = np.concatenate([batch.timestamps[lo:hi], np.zeros(Nmax - n, np.int64)])
        M = orc.mask_matrix(gp, tp)
        M[:, n:] = False
        for h in range(H):
            c = slice(h * 32, (h + 1) * 32)
            S = pad(q)[:, c] @ pad(k)[:, c].T
            ob = 0.05 * (orc.silu(S) * M) @ pad(v)[:, c]
            np.testing.assert_allclose(got[lo:hi, c], ob[:n], rtol=1e-12, atol=1e-15)


def _single_user(rng, n_u=4, n_s=10, n_r=6, n_c=5, ts_max=40):
    return make_batch_from_lengths([[n_u, n_s, n_r, n_c]], rng, ts_max=ts_max)


def test_candidate_invariants():
    """A candidate's output does not change when other candidates are
    perturbed or permuted, nor when real-time tokens stamped at or after it
    are perturbed (scale held fixed)."""
    rng = np.random.default_rng(21)
    batch = _single_user(rng)
    H, d = 2, 16
    q, k, v = _qkv(batch.T, d, 22)
    args = (batch.offsets, batch.group_ids, batch.timestamps, H, 1.0, 0.1)
    o = orc.hstu_attention(q, k, v, *args)
    c0 = 4 + 10 + 6
    cand = np.arange(c0, batch.T)
    # perturb all candidates except the first
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for a in (q2, k2, v2):
        a[cand[1:]] += np.random.default_rng(1).normal(size=(len(cand) - 1, d))
    o2 = orc.hstu_attention(q2, k2, v2, *args)
    np.testing.assert_allclose(o2[cand[0]], o[cand[0]], rtol=1e-13, atol=1e-15)
    # permute candidates (with their stamps)
    perm = np.concatenate([np.arange(c0), c0 + np.random.default_rng(2).permutation(len(cand))])
    o3 = orc.hstu_attention(q[perm], k[perm], v[perm], batch.offsets, batch.group_ids,
                            batch.timestamps[perm], H, 1.0, 0.1)
    np.testing.assert_allclose(o3, o[perm], rtol=1e-12, atol=1e-15)
    # perturb real-time tokens not earlier than candidate 0
    t_c = batch.timestamps[cand[0]]
    rt = np.arange(14, 20)
    late = rt[batch.timestamps[rt] >= t_c]
    q4, k4, v4 = q.copy(), k.copy(), v.copy()
    for a in (q4, k4, v4):
        a[late] += 3.0
    o4 = orc.hstu_attention(q4, k4, v4, *args)
    np.testing.assert_allclose(o4[cand[0]], o[cand[0]], rtol=1e-13, atol=1e-15)
    # static outputs ignore every real-time and candidate token
    q5, k5, v5 = q.copy(), k.copy(), v.copy()
    for a in (q5, k5, v5):
        a[14:] = np.random.default_rng(3).normal(size=a[14:].shape)
    o5 = orc.hstu_attention(q5, k5, v5, *args)
    np.testing.assert_array_equal(o5[:14], o[:14])


def test_identical_candidates_identical_outputs():
    rng = np.random.default_rng(31)
    batch = _single_user(rng)
    batch.timestamps[-1] = batch.timestamps[-2]
    q, k, v = _qkv(batch.T, 16, 32)
    for a in (q, k, v):
        a[-1] = a[-2]
    o = orc.hstu_attention(q, k, v, batch.offsets, batch.group_ids, batch.timestamps, 2, 1.0, 0.1)
    np.testing.assert_array_equal(o[-1], o[-2])


def test_linear_in_v_and_scale():
    batch = make_batch(1)
    q, k, v = _qkv(batch.T, 64, 8)
    v2 = np.random.default_rng(9).normal(size=v.shape)
    args = (batch.offsets, batch.group_ids, batch.timestamps, 2, 1.0)
    o1 = orc.hstu_attention(q, k, v, *args, 0.3)
    o2 = orc.hstu_attention(q, k, v2, *args, 0.3)
    o12 = orc.hstu_attention(q, k, 2 * v - v2, *args, 0.3)
    np.testing.assert_allclose(o12, 2 * o1 - o2, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(orc.hstu_attention(q, k, v, *args, 0.6), 2 * o1, rtol=1e-13)


def test_users_are_independent_and_permutable():
    batch = make_batch(1)
    q, k, v = _qkv(batch.T, 64, 10)
    o = orc.hstu_attention(q, k, v, batch.offsets, batch.group_ids, batch.timestamps, 2, 1.0, 0.1)
    order = [2, 0, 3, 1]
    off, g, t, _, rows = orc.select_users(batch.offsets, batch.group_ids, batch.timestamps, None, order)
    o2 = orc.hstu_attention(q[rows], k[rows], v[rows], off, g, t, 2, 1.0, 0.1)
    np.testing.assert_allclose(o2, o[rows], rtol=1e-13, atol=1e-16)


def test_bwd_matches_finite_differences():
    rng = np.random.default_rng(41)
    batch = make_batch_from_lengths([[2, 5, 4, 3], [1, 3, 2, 2]], rng, ts_max=8)
    H, d = 2, 8
    q, k, v = _qkv(batch.T, d, 42)
    dO = np.random.default_rng(43).normal(size=q.shape)
    args = (batch.offsets, batch.group_ids, batch.timestamps, H, 0.9, 0.2)
    dq, dk, dv = orc.hstu_attention_bwd(q, k, v, dO, *args)

    def loss(q_, k_, v_):
        return float((orc.hstu_attention(q_, k_, v_, *args) * dO).sum())

    h = 1e-6
    pick = np.random.default_rng(44)
    for grad, which in ((dq, 0), (dk, 1), (dv, 2)):
        for _ in range(40):
            i, j = pick.integers(batch.T), pick.integers(d)
            a = [q.copy(), k.copy(), v.copy()]
            b = [q.copy(), k.copy(), v.copy()]
            a[which][i, j] += h
            b[which][i, j] -= h
            fd = (loss(*a) - loss(*b)) / (2 * h)
            assert abs(fd - grad[i, j]) <= 1e-7 * max(1.0, abs(fd)), (which, i, j, fd, grad[i, j])
