"""Pins of the oracle's Group LayerNorm against torch's CPU layer_norm (a
library routine) and torch autograd, plus per-token independence."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import mtgr_oracle as orc

EPS = 1e-5


def _inputs(T=37, d=48, G=4, seed=0, scale=3.0):
    rng = np.random.default_rng(seed)
    x = rng.normal(0.5, scale, size=(T, d))
    g = np.sort(rng.integers(0, G, size=T)).astype(np.uint8)
    gamma = 1.0 + rng.normal(0, 0.3, size=(G, d))
    beta = rng.normal(0, 0.3, size=(G, d))
    return x, g, gamma, beta


def test_single_group_equals_layer_norm():
    x, g, gamma, beta = _inputs()
    gamma[:] = gamma[0]
    beta[:] = beta[0]
    y, mean, rstd = orc.group_layernorm(x, gamma, beta, g, EPS)
    ref = F.layer_norm(torch.from_numpy(x), (x.shape[1],), torch.from_numpy(gamma[0]),
                       torch.from_numpy(beta[0]), eps=EPS).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(mean, x.mean(axis=1), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(rstd, 1 / np.sqrt(x.var(axis=1) + EPS), rtol=1e-12)


def test_each_group_uses_its_own_affine():
    x, g, gamma, beta = _inputs(seed=1)
    y, _, _ = orc.group_layernorm(x, gamma, beta, g, EPS)
    for c in range(4):
        sel = g == c
        if not sel.any():
            continue
        ref = F.layer_norm(torch.from_numpy(x[sel]), (x.shape[1],), torch.from_numpy(gamma[c]),
                           torch.from_numpy(beta[c]), eps=EPS).numpy()
        np.testing.assert_allclose(y[sel], ref, rtol=1e-12, atol=1e-12)


def test_tokens_are_independent():
    x, g, gamma, beta = _inputs(seed=2)
    y, _, _ = orc.group_layernorm(x, gamma, beta, g, EPS)
    x2 = x.copy()
    x2[5:] = np.random.default_rng(9).normal(size=x2[5:].shape)
    y2, _, _ = orc.group_layernorm(x2, gamma, beta, g, EPS)
    np.testing.assert_array_equal(y[:5], y2[:5])


def test_bwd_matches_torch_autograd():
    x, g, gamma, beta = _inputs(seed=3)
    dy = np.random.default_rng(4).normal(size=x.shape)
    y, mean, rstd = orc.group_layernorm(x, gamma, beta, g, EPS)
    dx, dgamma, dbeta = orc.group_layernorm_bwd(dy, x, mean, rstd, gamma, g)

    xt = torch.tensor(x, requires_grad=True)
    gt = torch.tensor(gamma, requires_grad=True)
    bt = torch.tensor(beta, requires_grad=True)
    parts = []
    idx = torch.from_numpy(g.astype(np.int64))
    # per-group library layer_norm, gathered back into token order
    out = torch.zeros_like(xt)
    for c in range(4):
        sel = (idx == c).nonzero().flatten()
        if sel.numel() == 0:
            continue
        out = out.index_put((sel,), F.layer_norm(xt[sel], (x.shape[1],), gt[c], bt[c], eps=EPS))
        parts.append(c)
    (out * torch.from_numpy(dy)).sum().backward()
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dgamma, gt.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dbeta, bt.grad.numpy(), rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("shift", [0.0, 1e3])
def test_constant_rows_give_beta(shift):
    """A constant row has zero variance: the normalised value is 0 and the
    output is beta of its group."""
    x, g, gamma, beta = _inputs(seed=6)
    x[:] = shift
    y, _, _ = orc.group_layernorm(x, gamma, beta, g, EPS)
    np.testing.assert_allclose(y, beta[g.astype(np.int64)], atol=1e-12)
