"""CPU pins of the candidate-head oracle (oracle/candidate_head.py).

Independent routes: PyTorch autograd in float64 on the CPU through its own
linear, SiLU and binary-cross-entropy-with-logits routines; central finite
differences; the closed form of the loss at zero logits; the zero gradient
of every non-candidate row."""

import numpy as np
import pytest
import torch

from mtgr_inputs import make_batch_from_lengths, make_head_params, make_labels
from oracle import candidate_head as ch


def setup(d=12, h=10, bias=True, seed=0):
    rng = np.random.default_rng(seed)
    batch = make_batch_from_lengths([[2, 5, 2, 3], [1, 4, 0, 2], [0, 0, 0, 0], [2, 3, 1, 4]], rng, ts_max=100)
    p = make_head_params(d, h, 2, rng, bias)
    x = rng.normal(size=(batch.T, d))
    y = make_labels(int(np.sum(batch.group_ids == 3)), rng, p_click=0.5, p_order=0.5)
    return batch, p, x, y


def torch_reference(p, x, g, y):
    rows = torch.from_numpy(np.nonzero(g == 3)[0])
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    W1 = torch.tensor(p.W1, dtype=torch.float64, requires_grad=True)
    W2 = torch.tensor(p.W2, dtype=torch.float64, requires_grad=True)
    b1 = torch.tensor(p.b1, dtype=torch.float64, requires_grad=True) if p.b1 is not None else None
    b2 = torch.tensor(p.b2, dtype=torch.float64, requires_grad=True) if p.b2 is not None else None
    hdn = torch.nn.functional.silu(torch.nn.functional.linear(xt[rows], W1, b1))
    logits = torch.nn.functional.linear(hdn, W2, b2)
    yt = torch.tensor(y, dtype=torch.float64)
    loss = torch.nn.functional.binary_cross_entropy_with_logits(logits, yt, reduction="sum") / len(rows)
    loss.backward()
    return logits.detach().numpy(), loss.item(), xt.grad.numpy(), W1.grad.numpy(), W2.grad.numpy(), \
        (b1.grad.numpy() if b1 is not None else None), (b2.grad.numpy() if b2 is not None else None)


@pytest.mark.parametrize("bias", [True, False])
def test_head_matches_torch_autograd(bias):
    batch, p, x, y = setup(bias=bias)
    logits, cache = ch.head_fwd(p, x, batch.group_ids)
    loss = ch.bce_loss(logits, y)
    dx, gr = ch.head_loss_bwd(p, cache, logits, y, batch.T)
    t_logits, t_loss, t_dx, t_W1, t_W2, t_b1, t_b2 = torch_reference(p, x, batch.group_ids, y)
    np.testing.assert_allclose(logits, t_logits, rtol=1e-12, atol=1e-12)
    assert abs(loss - t_loss) < 1e-12
    np.testing.assert_allclose(dx, t_dx, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(gr["W1"], t_W1, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(gr["W2"], t_W2, rtol=1e-10, atol=1e-13)
    if bias:
        np.testing.assert_allclose(gr["b1"], t_b1, rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(gr["b2"], t_b2, rtol=1e-10, atol=1e-13)


def test_head_finite_differences():
    batch, p, x, y = setup(d=6, h=5, seed=3)

    def loss_at(xx, W1=None, W2=None):
        q = type(p)(p.W1 if W1 is None else W1, p.b1, p.W2 if W2 is None else W2, p.b2)
        lg, _ = ch.head_fwd(q, xx, batch.group_ids)
        return ch.bce_loss(lg, y)

    logits, cache = ch.head_fwd(p, x, batch.group_ids)
    dx, gr = ch.head_loss_bwd(p, cache, logits, y, batch.T)
    eps = 1e-6
    rows = ch.candidate_rows(batch.group_ids)
    for (r, c) in [(rows[0], 0), (rows[-1], 5), (rows[3], 2)]:
        xp, xm = x.copy(), x.copy()
        xp[r, c] += eps
        xm[r, c] -= eps
        assert abs((loss_at(xp) - loss_at(xm)) / (2 * eps) - dx[r, c]) < 1e-8
    for (i, j) in [(0, 0), (4, 5), (2, 3)]:
        Wp, Wm = p.W1.astype(np.float64), p.W1.astype(np.float64)
        Wp = Wp.copy(); Wm = Wm.copy()
        Wp[i, j] += eps
        Wm[i, j] -= eps
        assert abs((loss_at(x, W1=Wp) - loss_at(x, W1=Wm)) / (2 * eps) - gr["W1"][i, j]) < 1e-8
    for (i, j) in [(0, 0), (1, 4)]:
        Wp, Wm = p.W2.astype(np.float64).copy(), p.W2.astype(np.float64).copy()
        Wp[i, j] += eps
        Wm[i, j] -= eps
        assert abs((loss_at(x, W2=Wp) - loss_at(x, W2=Wm)) / (2 * eps) - gr["W2"][i, j]) < 1e-8


def test_loss_at_zero_logits_is_ln2_per_task():
    """W2 = 0 and b2 = 0 give zero logits: each task's cross-entropy is ln 2
    whatever the labels, and the gradient of each logit is (1/2 - y) / n."""
    batch, p, x, y = setup()
    q = type(p)(p.W1, p.b1, np.zeros_like(p.W2), np.zeros(2, dtype=np.float32))
    logits, cache = ch.head_fwd(q, x, batch.group_ids)
    assert np.all(logits == 0)
    assert abs(ch.bce_loss(logits, y) - 2 * np.log(2)) < 1e-14
    _, gr = ch.head_loss_bwd(q, cache, logits, y, batch.T)
    n = logits.shape[0]
    np.testing.assert_allclose(gr["b2"], np.sum(0.5 - y.astype(np.float64), axis=0) / n, rtol=0, atol=1e-15)


def test_non_candidate_rows_get_no_gradient():
    batch, p, x, y = setup()
    logits, cache = ch.head_fwd(p, x, batch.group_ids)
    dx, _ = ch.head_loss_bwd(p, cache, logits, y, batch.T)
    other = batch.group_ids != 3
    assert np.all(dx[other] == 0)
    assert np.all(np.abs(dx[~other]).sum(axis=1) > 0)
