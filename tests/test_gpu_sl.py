"""GPU parity of Stochastic Length sampling and the token-budget cut
(mtgr_stochastic_length) against the oracle: offsets, the budget cut, and
the group ids, timestamps and feature rows of the fitting users bit for bit, on small edge batches and on a
pool of long-tail users four times the 65,536-token budget; then the
shortened batch through the layer forward and backward against the oracle."""

import numpy as np
import pytest
import torch

from mtgr_inputs import make_batch_from_lengths, make_layer_params, make_uniform_draws, make_user_pool
from oracle import mtgr_oracle as orc
from oracle import stochastic_length as sl
from tests.gpu_util import TOL, f64, params_to, rel_l2, rounded, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def mb():
    import generative_recommendation_ranking_grouplayernorm_amd.binding as b

    b.load_library()
    return b


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw element bits of a device tensor (exact comparison for any dtype)."""
    t = t.detach().cpu()
    view = {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.float16: torch.int16}[t.dtype]
    return t.view(view).numpy()


def run_gpu(mb, batch, x_dev, u, s_keep, budget):
    B, T = batch.B, batch.T
    off = torch.from_numpy(batch.offsets).to(DEV)
    g = torch.from_numpy(batch.group_ids).to(DEV)
    ts = torch.from_numpy(batch.timestamps).to(DEV)
    ud = torch.from_numpy(np.asarray(u, dtype=np.float32)).to(DEV)
    off_o = torch.full((B + 1,), -7, dtype=torch.int32, device=DEV)
    g_o = torch.full((max(T, 1),), 255, dtype=torch.uint8, device=DEV)
    ts_o = torch.full((max(T, 1),), -99, dtype=torch.int64, device=DEV)
    x_o = torch.full((max(T, 1), x_dev.shape[1]), float("nan"), dtype=x_dev.dtype, device=DEV)
    fit = torch.full((2,), -1, dtype=torch.int64, device=DEV)
    ws = torch.empty(max(mb.mtgr_workspace_size(mb.OP_STOCHASTIC_LENGTH, B, T, 0, x_dev.shape[1], 1, x_dev.dtype),
                         256), dtype=torch.uint8, device=DEV)
    mb.mtgr_stochastic_length(off, g, ts, x_dev, ud, s_keep, budget, off_o, g_o, ts_o, x_o, fit, ws)
    torch.cuda.synchronize()
    return off_o.cpu().numpy(), g_o, ts_o, x_o, fit.cpu().numpy()


def check(mb, batch, x_dev, u, s_keep, budgets):
    x_bits = bits(x_dev)
    want = sl.stochastic_length(batch.offsets, batch.group_ids, batch.timestamps, x_bits, u, s_keep)
    for budget in budgets:
        off_o, g_o, ts_o, x_o, fit = run_gpu(mb, batch, x_dev, u, s_keep, budget)
        np.testing.assert_array_equal(off_o, want[0])
        b, t = sl.budget_fit(want[0], budget)
        assert (int(fit[0]), int(fit[1])) == (b, t), (budget, fit, b, t)
        # the rows of the fitting users are written, the rest left alone
        np.testing.assert_array_equal(g_o.cpu().numpy()[:t], want[1][:t])
        np.testing.assert_array_equal(ts_o.cpu().numpy()[:t], want[2][:t])
        np.testing.assert_array_equal(bits(x_o)[:t], want[3][:t])
        assert np.all(g_o.cpu().numpy()[t:] == 255)
    return want


def edge_batch():
    rng = np.random.default_rng(5)
    lengths = [[8, 40, 5, 3], [8, 3, 0, 2], [0, 0, 0, 0], [2, 0, 4, 1], [8, 17, 9, 0], [0, 25, 0, 6],
               [0, 0, 0, 0], [1, 300, 64, 20]]
    return make_batch_from_lengths(lengths, rng, ts_max=1000)


@pytest.mark.parametrize("dtype,d", [(torch.float32, 8), (torch.bfloat16, 64), (torch.float16, 1024)])
@pytest.mark.parametrize("s_keep", [0, 1, 3, 16, 24, 5000])
def test_sl_edge_batch(mb, dtype, d, s_keep):
    batch = edge_batch()
    x = rounded(np.random.default_rng(9).normal(size=(batch.T, d)), dtype).to(DEV)
    u = make_uniform_draws(batch.B, seed=s_keep)
    say("SL edge", dtype, d, s_keep)
    check(mb, batch, x, u, s_keep, budgets=[0, 10, 57, 10 ** 9])


def test_sl_wide_rows(mb):
    """Rows of more than 4 KB (fp32, d = 1536) take the one-row-per-wave copy."""
    batch = edge_batch()
    x = rounded(np.random.default_rng(2).normal(size=(batch.T, 1536)), torch.float32).to(DEV)
    u = make_uniform_draws(batch.B, seed=3)
    check(mb, batch, x, u, 9, budgets=[0, 60, 10 ** 9])


def test_sl_window_extremes(mb):
    """Every user at u = 0 (first window) and at the largest float32 below 1
    (last window)."""
    batch = edge_batch()
    x = rounded(np.random.default_rng(1).normal(size=(batch.T, 64)), torch.bfloat16).to(DEV)
    top = np.nextafter(np.float32(1), np.float32(0))
    for val in (np.float32(0), top):
        u = np.full(batch.B, val, dtype=np.float32)
        check(mb, batch, x, u, 7, budgets=[100])


def test_sl_pool_at_full_size(mb):
    """A pool of long-tail users (about 262k tokens, d 1024 bf16) shortened to
    512 history tokens and cut to a 65,536-token batch."""
    batch = make_user_pool(4, 4 * 65536, seed=0)
    say("SL pool", batch.B, batch.T)
    gen = torch.Generator(device="cpu").manual_seed(4)
    x = torch.randn(batch.T, 1024, generator=gen).to(torch.bfloat16).to(DEV)
    u = make_uniform_draws(batch.B, seed=0)
    want = check(mb, batch, x, u, 512, budgets=[65536])
    b, t = sl.budget_fit(want[0], 65536)
    say(f"  {batch.B} users / {batch.T} tokens -> {len(want[1])} tokens; budget 65,536 holds {b} users "
        f"({t} tokens)")


def test_sl_batch_through_the_layer(mb):
    """The cut batch feeds the layer as it is (its offsets prefix and its
    first rows): forward and backward against the oracle on the oracle's own
    shortened batch."""
    rng = np.random.default_rng(17)
    lengths = [[8, 400, 20, 20], [8, 90, 5, 20], [8, 700, 64, 20], [8, 33, 0, 20], [8, 260, 3, 20]]
    batch = make_batch_from_lengths(lengths, rng, ts_max=86400)
    d, H, dtype = 256, 2, torch.bfloat16
    x = rounded(rng.normal(size=(batch.T, d)), dtype).to(DEV)
    u = make_uniform_draws(batch.B, seed=5)
    s_keep, budget = 128, 700
    off_o, g_o, ts_o, x_o, fit = run_gpu(mb, batch, x, u, s_keep, budget)
    Bf, Tf = int(fit[0]), int(fit[1])
    want = sl.stochastic_length(batch.offsets, batch.group_ids, batch.timestamps, f64(x), u, s_keep)
    b_ref, t_ref = sl.budget_fit(want[0], budget)
    assert (Bf, Tf) == (b_ref, t_ref) and Bf >= 2
    off_b = torch.from_numpy(off_o[:Bf + 1].copy()).to(DEV)
    p = make_layer_params(d, H, rng, "xavier", False)
    dev_p, q = params_to(p, dtype, DEV)
    prm = mb.make_params(dev_p, H)
    xin = x_o[:Tf]
    scale = 1.0 / int(np.max(np.diff(off_o[:Bf + 1])))
    saved = mb.alloc_saved(Tf, d, dtype, DEV)
    y = torch.empty(Tf, d, dtype=dtype, device=DEV)
    mb.mtgr_hstu_layer_fwd(prm, xin, y, mb.make_saved(saved), off_b, g_o[:Tf], ts_o[:Tf], scale,
                           mb.workspace(mb.OP_LAYER_FWD, Bf, Tf, d, H, dtype, DEV))
    R = rounded(rng.normal(size=(Tf, d)), dtype)
    grads = mb.alloc_grads(d, 4, False, DEV)
    dx = torch.empty_like(y)
    ml = int(np.max(np.diff(off_o[:Bf + 1])))
    mb.mtgr_hstu_layer_bwd(prm, xin, mb.make_saved(saved), R.to(DEV), dx, grads, off_b, g_o[:Tf], ts_o[:Tf], scale,
                           mb.workspace(mb.OP_LAYER_BWD, Bf, Tf, d, H, dtype, DEV, max_len=ml), max_len=ml)
    torch.cuda.synchronize()
    o_off, o_g, o_ts, o_x = want[0][:b_ref + 1], want[1][:t_ref], want[2][:t_ref], want[3][:t_ref]
    ref, sv = orc.layer_fwd(q, o_x, o_off, o_g, o_ts, 1.0, scale)
    dref, gref = orc.layer_bwd(q, o_x, sv, f64(R), o_off, o_g, o_ts, 1.0, scale)
    for name, got, r in (("x_out", f64(y), ref), ("dx", f64(dx), dref),
                         ("dW_uqkv", grads["W_uqkv"].cpu().numpy(), gref["W_uqkv"])):
        err = rel_l2(got, r)
        say(f"  {name}: rel-L2 {err:.3e}")
        assert err <= TOL[dtype]
