"""GPU parity of the serving forward: the multi-layer entry point against
chained single-layer calls and the oracle, and its captured HIP graph against
the eager call, replayed several times with other GPU work in between and
with a new request written into the same buffers between replays."""

import numpy as np
import pytest
import torch

from mtgr_inputs import CONFIGS, config_inputs, make_activations, make_batch_from_lengths
from mtgr_inputs import make_head_params, make_layer_params, make_probe_head
from oracle import candidate_head as chd
from oracle import mtgr_oracle as orc
from tests.gpu_util import TOL, f64, meta, params_to, rel_l2, rounded, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
SCORE_BOUND = 6e-3  # per-candidate score difference (paper-daily deep reading, 3: fp16 vs fp32 <= 0.006)


@pytest.fixture(scope="module")
def mb():
    import generative_recommendation_ranking_grouplayernorm_amd.binding as b

    b.load_library()
    return b


def device_layers(mb, params, dtype):
    """(LayerParams list, device tensors kept alive, fp64 oracle params)."""
    lps, keep, qs = [], [], []
    for p in params:
        dev_p, q = params_to(p, dtype, DEV)
        keep.append(dev_p)
        qs.append(q)
        lps.append(mb.make_params(dev_p, p.H))
    return lps, keep, qs


def chained(mb, lps, h0, off, g, ts, scale, dtype):
    """Reference GPU path: one mtgr_hstu_layer_fwd call per layer."""
    T, d = h0.shape
    ws = mb.workspace(mb.OP_LAYER_FWD, off.numel() - 1, T, d, lps[0].H, dtype, DEV)
    h, nxt = h0.clone(), torch.empty_like(h0)
    for lp in lps:
        mb.mtgr_hstu_layer_fwd(lp, h, nxt, None, off, g, ts, scale, ws)
        h, nxt = nxt, h
    return h


def test_stack_fwd_tiny_fp32_matches_oracle_and_chained_layers(mb):
    """Three fp32 layers on the tiny four-user batch (several tiles, ragged
    tails): the stack call equals chained layer calls bit for bit, and the
    oracle within the fp32 bar.  Odd and even L exercise both buffer orders."""
    batch, _, x = config_inputs(1)
    cfg = CONFIGS[1]
    rng = np.random.default_rng([0, 1, 77])
    params = [make_layer_params(cfg["d"], cfg["H"], rng, cfg["w_init"], cfg["bias"]) for _ in range(3)]
    dtype = torch.float32
    scale = 1.0 / batch.max_len
    off, g, ts = meta(batch, DEV)
    lps, keep, qs = device_layers(mb, params, dtype)
    x_in = rounded(x, dtype).to(DEV)
    for L in (1, 2, 3):
        out = torch.empty_like(x_in)
        ws = mb.workspace(mb.OP_STACK_FWD, batch.B, batch.T, cfg["d"], cfg["H"], dtype, DEV)
        x_copy = x_in.clone()
        mb.mtgr_hstu_stack_fwd(lps[:L], x_in, out, off, g, ts, scale, ws)
        ref_gpu = chained(mb, lps[:L], x_in, off, g, ts, scale, dtype)
        torch.cuda.synchronize()
        assert torch.equal(x_in, x_copy), "input modified"
        assert torch.equal(out, ref_gpu), f"L={L}: stack differs from chained layers"
        ref = orc.stack_fwd(qs[:L], f64(x_in), batch.offsets, batch.group_ids, batch.timestamps, 1.0, scale)
        err = rel_l2(f64(out), ref)
        say(f"  L={L}: rel-L2 vs oracle {err:.3e}")
        assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_stack_fwd_short_halfprec_with_biases_matches_oracle(mb, dtype):
    """A short multi-user 16-bit batch with biases: the output projections
    are split over K into fp32 planes that the next layer's input norm (and
    the final sum) add with bias and residual.  L = 1, 2, 3 against the
    oracle, and close to chained layer calls."""
    rng = np.random.default_rng([0, 5, 61])
    lengths = [[8, 300, 20, 20], [8, 57, 0, 9], [2, 130, 64, 33]]
    batch = make_batch_from_lengths(lengths, rng, ts_max=86400)
    d, H = 256, 2
    params = [make_layer_params(d, H, rng, "xavier", True) for _ in range(3)]
    x = rng.normal(0, 1, size=(batch.T, d))
    scale = 1.0 / batch.max_len
    off, g, ts = meta(batch, DEV)
    lps, keep, qs = device_layers(mb, params, dtype)
    x_in = rounded(x, dtype).to(DEV)
    for L in (1, 2, 3):
        out = torch.full_like(x_in, float("nan"))
        ws = mb.workspace(mb.OP_STACK_FWD, batch.B, batch.T, d, H, dtype, DEV)
        x_copy = x_in.clone()
        mb.mtgr_hstu_stack_fwd(lps[:L], x_in, out, off, g, ts, scale, ws)
        ch = chained(mb, lps[:L], x_in, off, g, ts, scale, dtype)
        torch.cuda.synchronize()
        assert torch.equal(x_in, x_copy), "input modified"
        ref = orc.stack_fwd(qs[:L], f64(x_in), batch.offsets, batch.group_ids, batch.timestamps, 1.0, scale)
        err = rel_l2(f64(out), ref)
        err_ch = rel_l2(f64(out), f64(ch))
        say(f"  {dtype} L={L}: rel-L2 vs oracle {err:.3e}, vs chained layer calls {err_ch:.3e}")
        assert err <= TOL[dtype]
        assert err_ch <= TOL[dtype]


def _serving_request(K: int, seed: int, n_s: int, n_r: int):
    """A one-user request with history n_s, n_r real-time actions and K
    candidates, drawn like the serving sweep (candidates after every
    real-time action)."""
    cfg = CONFIGS[5]
    rng = np.random.default_rng([seed, 5, 9])
    batch = make_batch_from_lengths([[cfg["n_u"], n_s, n_r, K]], rng, cfg["ts_max"], cfg["cand_after_rt"])
    x = make_activations(batch.T, cfg["d"], np.random.default_rng([seed, 5, 10]), cfg["x_init"])
    return batch, x


def _scores_diff(out, ref, g, d):
    w = make_probe_head(d)
    return float(np.max(np.abs(orc.candidate_scores(out, g, w) - orc.candidate_scores(ref, g, w))))


def test_serving_graph_replay_matches_eager(mb):
    """22 fp16 layers, one request, one graph per K in {20, 100, 500, 1000}
    sharing one set of buffers sized for the largest K.  Each replay must
    equal the eager stack call bit for bit: three replays with eager work and
    host synchronisations between them, then a different request of the same
    length (another history / real-time split, new timestamps and features)
    written into the captured buffers.  The eager stack call agrees with
    chained layer calls up to fp32 addition order, and at K=20 the replay matches
    the oracle."""
    cfg = CONFIGS[5]
    dtype = torch.float16
    d, H = cfg["d"], cfg["H"]
    _, params, _ = config_inputs(5)
    lps, keep, qs = device_layers(mb, params, dtype)
    Tmax = cfg["n_u"] + 1000 + 32 + max(cfg["K_sweep"])
    buf_x = torch.empty(Tmax, d, dtype=dtype, device=DEV)
    buf_y = torch.empty(Tmax, d, dtype=dtype, device=DEV)
    buf_off = torch.empty(2, dtype=torch.int32, device=DEV)
    buf_g = torch.empty(Tmax, dtype=torch.uint8, device=DEV)
    buf_ts = torch.empty(Tmax, dtype=torch.int64, device=DEV)
    ws = mb.workspace(mb.OP_STACK_FWD, 1, Tmax, d, H, dtype, DEV)
    graphs = {}
    for K in cfg["K_sweep"]:
        batch, _, x = config_inputs(5, K=K)
        T = batch.T
        scale = 1.0 / batch.max_len
        xs, ys = buf_x[:T], buf_y[:T]
        off, g, ts = buf_off, buf_g[:T], buf_ts[:T]

        def load(b, xx):
            off.copy_(torch.from_numpy(b.offsets))
            g.copy_(torch.from_numpy(b.group_ids))
            ts.copy_(torch.from_numpy(b.timestamps))
            xs.copy_(rounded(xx, dtype))

        load(batch, x)
        graphs[K] = mb.mtgr_stack_graph_create(lps, xs, ys, off, g, ts, scale, ws)
        # eager reference on separate buffers
        e_x, e_off, e_g, e_ts = xs.clone(), off.clone(), g.clone(), ts.clone()
        e_y = torch.empty_like(e_x)
        e_ws = mb.workspace(mb.OP_STACK_FWD, 1, T, d, H, dtype, DEV)
        mb.mtgr_hstu_stack_fwd(lps, e_x, e_y, e_off, e_g, e_ts, scale, e_ws)
        ch = chained(mb, lps, e_x, e_off, e_g, e_ts, scale, dtype)
        torch.cuda.synchronize()
        # the stack splits the output projections of short batches over K:
        # same values up to the order of fp32 additions
        err_ch = rel_l2(f64(e_y), f64(ch))
        say(f"  K={K}: stack vs chained layer calls rel-L2 {err_ch:.3e}")
        assert err_ch <= TOL[dtype], f"K={K}: stack call differs from chained layer calls"
        for rep in range(3):
            ys.fill_(float("nan"))
            graphs[K].launch()
            torch.cuda.synchronize()
            assert torch.equal(ys, e_y), f"K={K}: replay {rep} differs from the eager call"
            # unrelated eager work between replays
            junk = torch.randn(T, d, device=DEV, dtype=dtype)
            mb.mtgr_hstu_stack_fwd(lps[:2], junk, torch.empty_like(junk), e_off, e_g, e_ts, scale, e_ws)
            torch.cuda.synchronize()
        if K == 20:
            ref = orc.stack_fwd(qs, f64(xs), batch.offsets, batch.group_ids, batch.timestamps, 1.0, scale)
            out = f64(ys)
            err = rel_l2(out, ref)
            dmax = _scores_diff(out, ref, batch.group_ids, d)
            say(f"  K=20 replay vs oracle: rel-L2 {err:.3e}, max candidate score diff {dmax:.2e}")
            assert err <= 1e-2
            assert dmax <= SCORE_BOUND
        # a new request of the same length in the same buffers
        b2, x2 = _serving_request(K, seed=11, n_s=990, n_r=42)
        assert b2.T == T
        load(b2, x2)
        graphs[K].launch()
        n_x, n_off, n_g, n_ts = xs.clone(), off.clone(), g.clone(), ts.clone()
        n_y = torch.empty_like(n_x)
        torch.cuda.synchronize()
        mb.mtgr_hstu_stack_fwd(lps, n_x, n_y, n_off, n_g, n_ts, scale, e_ws)
        torch.cuda.synchronize()
        assert torch.equal(ys, n_y), f"K={K}: replay on a new request differs from the eager call"
        assert not torch.equal(n_y, e_y)
        say(f"  K={K}: T={T}, graph replays equal the eager call")
    # every graph still replays after the others ran
    batch, _, x = config_inputs(5, K=20)
    T = batch.T
    buf_off.copy_(torch.from_numpy(batch.offsets))
    buf_g[:T].copy_(torch.from_numpy(batch.group_ids))
    buf_ts[:T].copy_(torch.from_numpy(batch.timestamps))
    buf_x[:T].copy_(rounded(x, dtype))
    graphs[20].launch()
    e_y = torch.empty(T, d, dtype=dtype, device=DEV)
    mb.mtgr_hstu_stack_fwd(lps, buf_x[:T].clone(), e_y, buf_off.clone(), buf_g[:T].clone(), buf_ts[:T].clone(),
                           1.0 / batch.max_len, mb.workspace(mb.OP_STACK_FWD, 1, T, d, H, dtype, DEV))
    torch.cuda.synchronize()
    assert torch.equal(buf_y[:T], e_y)
    for gr in graphs.values():
        gr.close()


def test_serving_graph_with_candidate_head(mb):
    """One request = 22 fp16 layers and the candidate head (1024 -> 512 -> 2
    tasks) in one graph.  Replays give the eager logits bit for bit; at K=20
    the scores sigmoid(logit) of both tasks are within the pages' 6e-3 of the
    fp64 oracle run on the same rounded inputs and weights."""
    cfg = CONFIGS[5]
    dtype = torch.float16
    d, H = cfg["d"], cfg["H"]
    _, params, _ = config_inputs(5)
    lps, keep, qs = device_layers(mb, params, dtype)
    hp = make_head_params(d, 512, 2, np.random.default_rng([0, 5, 77]), True)
    hdev = {k: rounded(getattr(hp, k), dtype).to(DEV) for k in ("W1", "b1", "W2", "b2")}
    hprm = mb.make_head_params(hdev)

    class HQ:
        pass

    hq = HQ()
    for k in ("W1", "b1", "W2", "b2"):
        setattr(hq, k, f64(hdev[k]))
    for K in (20, 1000):
        batch, _, x = config_inputs(5, K=K)
        T = batch.T
        scale = 1.0 / batch.max_len
        off, g, ts = meta(batch, DEV)
        xs = rounded(x, dtype).to(DEV)
        ys = torch.empty_like(xs)
        logits = torch.full((K, 2), float("nan"), device=DEV)
        ws = mb.workspace(mb.OP_STACK_FWD, 1, T, d, H, dtype, DEV)
        hws = mb.head_workspace(1, K, d, 512, 2, dtype, DEV)
        gr = mb.mtgr_serving_graph_create(lps, hprm, xs, ys, logits, K, off, g, ts, scale, ws, hws)
        # eager reference on its own buffers
        e_y = torch.empty_like(xs)
        e_logits = torch.empty(K, 2, device=DEV)
        e_ws = mb.workspace(mb.OP_STACK_FWD, 1, T, d, H, dtype, DEV)
        e_hws = mb.head_workspace(1, K, d, 512, 2, dtype, DEV)
        mb.mtgr_hstu_stack_fwd(lps, xs, e_y, off, g, ts, scale, e_ws)
        mb.mtgr_candidate_head_fwd(hprm, e_y, off, g, K, e_logits, e_hws)
        torch.cuda.synchronize()
        for rep in range(3):
            logits.fill_(float("nan"))
            gr.launch()
            torch.cuda.synchronize()
            assert torch.equal(logits, e_logits), f"K={K}: replay {rep} logits differ from the eager call"
            mb.mtgr_hstu_stack_fwd(lps[:1], xs, torch.empty_like(xs), off, g, ts, scale, e_ws)
            torch.cuda.synchronize()
        if K == 20:
            ref = orc.stack_fwd(qs, f64(xs), batch.offsets, batch.group_ids, batch.timestamps, 1.0, scale)
            lg_ref, _ = chd.head_fwd(hq, ref, batch.group_ids)
            s_gpu = 1.0 / (1.0 + np.exp(-logits.cpu().numpy().astype(np.float64)))
            s_ref = 1.0 / (1.0 + np.exp(-lg_ref))
            dmax = float(np.max(np.abs(s_gpu - s_ref)))
            say(f"  K=20 head scores vs oracle: max |diff| {dmax:.2e} over {s_ref.size} scores")
            assert dmax <= SCORE_BOUND
        gr.close()
        say(f"  K={K}: serving graph with head, replays equal the eager call")
