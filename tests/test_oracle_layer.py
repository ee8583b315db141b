"""Pins of the oracle's whole layer: torch library reductions of the
projection/normalisation steps, finite differences of the backward,
layer-level invariants of the mask, and the probe score helper."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from mtgr_inputs import config_inputs, make_batch_from_lengths, make_layer_params
from oracle import mtgr_oracle as orc

EPS = 1e-5


def _tiny(seed=0, bias=True, d=16, H=2, lengths=((2, 5, 3, 3), (1, 4, 2, 2))):
    rng = np.random.default_rng(seed)
    batch = make_batch_from_lengths(list(lengths), rng, ts_max=10)
    p = make_layer_params(d, H, rng, "normal0.02", bias)
    for name in ("W_uqkv", "b_uqkv", "gamma1", "beta1", "gamma2", "beta2", "W_o", "b_o"):
        if getattr(p, name) is not None:
            setattr(p, name, getattr(p, name).astype(np.float64))
    p.W_uqkv *= 20  # larger weights so that every term carries weight
    p.W_o *= 20
    x = rng.normal(0, 1, size=(batch.T, d))
    return batch, p, x


def test_projection_steps_match_torch_functional():
    batch, p, x = _tiny()
    _, saved = orc.layer_fwd(p, x, batch.offsets, batch.group_ids, batch.timestamps, 1.0, 0.1, EPS)
    xt = torch.from_numpy(x)
    g = torch.from_numpy(batch.group_ids.astype(np.int64))
    xhat = torch.stack([F.layer_norm(xt[i], (x.shape[1],), torch.from_numpy(p.gamma1[g[i]]).double(),
                                     torch.from_numpy(p.beta1[g[i]]).double(), eps=EPS)
                        for i in range(batch.T)])
    np.testing.assert_allclose(saved["xhat"], xhat.numpy(), rtol=1e-12, atol=1e-13)
    z = F.linear(xhat, torch.from_numpy(p.W_uqkv).double(), torch.from_numpy(p.b_uqkv).double())
    np.testing.assert_allclose(saved["z"], z.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(saved["uqkv"], F.silu(z).numpy(), rtol=1e-12, atol=1e-13)


def _a5_a6_by_torch(p, x, saved, group_ids, d):
    """The layer's last two steps composed from torch library routines, from
    the oracle's attention output o and gate u: per token a
    ``torch.nn.functional.layer_norm`` with gamma2/beta2 of the token's
    group (paper-daily 模型怎么搭: normalise the aggregated output), times u
    (gated by U), then ``F.linear`` with W_o and b_o plus the input
    (marovi Métodos, the X-update: one linear layer and the residual)."""
    o = torch.from_numpy(np.asarray(saved["o"], np.float64))
    u = torch.from_numpy(np.asarray(saved["uqkv"], np.float64)[:, :d])
    g = torch.from_numpy(np.asarray(group_ids, np.int64))
    g2 = torch.from_numpy(np.asarray(p.gamma2, np.float64))
    b2 = torch.from_numpy(np.asarray(p.beta2, np.float64))
    n2 = torch.stack([F.layer_norm(o[i], (d,), g2[g[i]], b2[g[i]], eps=EPS) for i in range(o.shape[0])])
    y = n2 * u
    bias = None if p.b_o is None else torch.from_numpy(np.asarray(p.b_o, np.float64))
    x_out = F.linear(y, torch.from_numpy(np.asarray(p.W_o, np.float64)), bias) + torch.from_numpy(x)
    return n2.numpy(), y.numpy(), x_out.numpy()


def _a5_a6_agrees(layer_fwd, p, x, batch):
    d = x.shape[1]
    x_out, saved = layer_fwd(p, x, batch.offsets, batch.group_ids, batch.timestamps, 1.0, 0.1, EPS)
    n2, y, want = _a5_a6_by_torch(p, x, saved, batch.group_ids, d)
    return (np.allclose(saved["n2"], n2, rtol=1e-12, atol=1e-13) and np.allclose(saved["y"], y, rtol=1e-12, atol=1e-13)
            and np.allclose(x_out, want, rtol=1e-12, atol=1e-13))


def _slipped(kind):
    """The oracle's layer with one plausible slip in its last two steps (a
    planted mistake, for the test below): the pin must reject each."""
    def fwd(p, x, offsets, group_ids, timestamps, alpha, attn_scale, eps):
        x_out, saved = orc.layer_fwd(p, x, offsets, group_ids, timestamps, alpha, attn_scale, eps)
        d = x.shape[1]
        u = saved["uqkv"][:, :d]
        W = np.asarray(p.W_o, np.float64)
        b = 0.0 if p.b_o is None else np.asarray(p.b_o, np.float64)[None, :]
        if kind == "norm_after_gate":
            n2, _, _ = orc.group_layernorm(saved["o"] * u, p.gamma2, p.beta2, group_ids, eps)
            y = n2
        else:
            n2, y = saved["n2"], saved["y"]
        if kind == "wo_untransposed":
            out = x + y @ W + b
        elif kind == "no_residual":
            out = y @ W.T + b
        elif kind == "no_bias":
            out = x + y @ W.T
        else:
            out = x + y @ W.T + b
        saved = dict(saved, n2=n2, y=y)
        return out, saved
    return fwd


@pytest.mark.parametrize("bias", [True, False])
def test_gate_and_output_projection_match_torch_functional(bias):
    """a5-a6 pinned on their own: GLN2 of the attention output, times U, then
    the output projection and the residual, against torch's layer_norm and
    linear; and each slip (norm after the gate, W_o untransposed, residual
    dropped, bias dropped) fails that pin."""
    batch, p, x = _tiny(seed=6, bias=bias)
    assert _a5_a6_agrees(orc.layer_fwd, p, x, batch)
    for kind in ("norm_after_gate", "wo_untransposed", "no_residual") + (("no_bias",) if bias else ()):
        assert not _a5_a6_agrees(_slipped(kind), p, x, batch), kind


def test_layer_bwd_matches_finite_differences():
    batch, p, x = _tiny(seed=1)
    args = (batch.offsets, batch.group_ids, batch.timestamps, 1.0, 0.1)
    R = np.random.default_rng(2).normal(size=x.shape)
    x_out, saved = orc.layer_fwd(p, x, *args, EPS)
    dx, grads = orc.layer_bwd(p, x, saved, R, *args)

    def loss(pp, xx):
        return float((orc.layer_fwd(pp, xx, *args, EPS)[0] * R).sum())

    h = 1e-6
    pick = np.random.default_rng(3)
    # input coordinates
    for _ in range(40):
        i, j = pick.integers(batch.T), pick.integers(x.shape[1])
        xa, xb = x.copy(), x.copy()
        xa[i, j] += h
        xb[i, j] -= h
        fd = (loss(p, xa) - loss(p, xb)) / (2 * h)
        assert abs(fd - dx[i, j]) <= 1e-6 * max(1.0, abs(fd)), ("x", i, j, fd, dx[i, j])
    # parameter coordinates
    for name in ("W_uqkv", "b_uqkv", "gamma1", "beta1", "gamma2", "beta2", "W_o", "b_o"):
        arr = getattr(p, name)
        for _ in range(20):
            idx = tuple(int(pick.integers(s)) for s in arr.shape)
            orig = arr[idx]
            arr[idx] = orig + h
            lp = loss(p, x)
            arr[idx] = orig - h
            lm = loss(p, x)
            arr[idx] = orig
            fd = (lp - lm) / (2 * h)
            got = grads[name][idx]
            assert abs(fd - got) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, got)


def test_layer_candidate_and_static_invariants():
    batch, p, x = _tiny(seed=4, lengths=((2, 6, 4, 4),))
    args = (batch.offsets, batch.group_ids, batch.timestamps, 1.0, 0.1)
    y, _ = orc.layer_fwd(p, x, *args, EPS)
    c0 = 12
    x2 = x.copy()
    x2[c0 + 1:] += np.random.default_rng(5).normal(size=x2[c0 + 1:].shape)
    y2, _ = orc.layer_fwd(p, x2, *args, EPS)
    np.testing.assert_allclose(y2[c0], y[c0], rtol=1e-13, atol=1e-14)
    x3 = x.copy()
    x3[8:] = 0.3
    y3, _ = orc.layer_fwd(p, x3, *args, EPS)
    np.testing.assert_array_equal(y3[:8], y[:8])


def test_stack_is_repeated_layers_and_scores():
    batch, params, x = config_inputs(1)
    params = params * 2
    ref = x.astype(np.float64)
    for pp in params:
        ref, _ = orc.layer_fwd(pp, ref, batch.offsets, batch.group_ids, batch.timestamps, 1.0,
                               1.0 / batch.max_len)
    got = orc.stack_fwd(params, x, batch.offsets, batch.group_ids, batch.timestamps, 1.0,
                        1.0 / batch.max_len)
    np.testing.assert_array_equal(got, ref)
    w = np.random.default_rng(0).normal(size=x.shape[1])
    s = orc.candidate_scores(got, batch.group_ids, w)
    want = torch.sigmoid(torch.from_numpy(got[batch.group_ids == 3]) @ torch.from_numpy(w)).numpy()
    np.testing.assert_allclose(s, want, rtol=1e-14)


def test_selected_users_match_full_batch():
    batch, params, x = config_inputs(1)
    p = params[0]
    args = (1.0, 1.0 / batch.max_len)
    full, _ = orc.layer_fwd(p, x, batch.offsets, batch.group_ids, batch.timestamps, *args)
    off, g, t, xs, rows = orc.select_users(batch.offsets, batch.group_ids, batch.timestamps, x, [3, 1])
    part, _ = orc.layer_fwd(p, xs, off, g, t, *args)
    np.testing.assert_allclose(part, full[rows], rtol=1e-13, atol=1e-15)
