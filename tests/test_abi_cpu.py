"""Host-side checks of the C-ABI library that need no GPU: it loads, exports
every symbol include/mtgr.h declares, reports its version and status texts,
sizes workspaces monotonically, and rejects bad arguments before launching
anything; plus the host-side work counter against the oracle's mask."""

import ctypes
import os
import re

import numpy as np
import pytest

from mtgr_inputs import make_batch
from oracle import mtgr_oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mtgr.h")


@pytest.fixture(scope="module")
def lib():
    from generative_recommendation_ranking_grouplayernorm_amd import binding

    if not os.path.exists(binding.LIB_PATH):
        from generative_recommendation_ranking_grouplayernorm_amd import build

        build.build()
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(mtgr_\w+)\s*\(", text, re.M)))


def test_header_declares_the_abi():
    names = declared_functions()
    for n in ("mtgr_group_layernorm", "mtgr_hstu_attn_fwd", "mtgr_hstu_attn_bwd", "mtgr_hstu_layer_fwd",
              "mtgr_hstu_layer_bwd", "mtgr_group_layernorm_bwd", "mtgr_jagged_prep", "mtgr_workspace_size",
              "mtgr_status_string", "mtgr_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = os.popen(f"nm -D --defined-only {lib._name}").read()
    for n in declared_functions():
        assert re.search(rf"\bT {n}\b", out), n


def test_version_and_status_strings(lib):
    from generative_recommendation_ranking_grouplayernorm_amd import binding as b

    assert "gfx950" in b.mtgr_version()
    texts = {s: b.mtgr_status_string(s) for s in (0, -1, -2, -3, -4, -5, -99)}
    assert texts[0] == "ok"
    assert len(set(texts.values())) == len(texts)


def test_workspace_sizes_grow(lib):
    from generative_recommendation_ranking_grouplayernorm_amd import binding as b
    import torch

    for op in (b.OP_ATTN_FWD, b.OP_ATTN_BWD, b.OP_LAYER_FWD, b.OP_LAYER_BWD, b.OP_GLN_BWD):
        a = b.mtgr_workspace_size(op, 8, 1000, 256, 2, torch.bfloat16)
        c = b.mtgr_workspace_size(op, 80, 65536, 256, 2, torch.bfloat16)
        assert 0 < a <= c
    assert b.mtgr_workspace_size(b.OP_GLN_FWD, 8, 1000, 256, 2, torch.bfloat16) == 0


def _call_attn_fwd(lib, **kw):
    P = ctypes.c_void_p
    args = dict(q=8192, k=8192, v=8192, ldqkv=256, o=8192, ldo=256, offsets=4096, g=4096, ts=4096, B=1, T=10,
                H=2, dh=128, alpha=1.0, scale=0.1, dt=1, ws=8192, ws_bytes=1 << 20)
    args.update(kw)
    return lib.mtgr_hstu_attn_fwd(P(args["q"]), P(args["k"]), P(args["v"]), args["ldqkv"], P(args["o"]),
                                  args["ldo"], P(args["offsets"]), P(args["g"]), P(args["ts"]), args["B"],
                                  args["T"], args["H"], args["dh"], args["alpha"], args["scale"], args["dt"],
                                  P(args["ws"]), args["ws_bytes"], None)


def test_argument_errors_are_reported_before_launch(lib):
    # pointers here are never dereferenced: every call must fail validation
    assert _call_attn_fwd(lib, dt=7) == -2            # unknown dtype
    assert _call_attn_fwd(lib, dh=96) == -2           # unsupported head size
    assert _call_attn_fwd(lib, q=0) == -1             # null input
    assert _call_attn_fwd(lib, ldqkv=128) == -1       # stride shorter than H*dh
    assert _call_attn_fwd(lib, q=8200) == -1          # misaligned base
    assert _call_attn_fwd(lib, ws_bytes=16) == -3     # workspace too small
    assert _call_attn_fwd(lib, H=0) == -1
    assert _call_attn_fwd(lib, B=-1) == -1
    P = ctypes.c_void_p
    # group norm: d not a multiple of 8, too many groups
    assert lib.mtgr_group_layernorm(P(8192), P(8192), P(8192), P(8192), P(4096), 10, 60, 4, 1e-5, 1,
                                    None, None, None) == -1
    assert lib.mtgr_group_layernorm(P(8192), P(8192), P(8192), P(8192), P(4096), 10, 64, 9, 1e-5, 1,
                                    None, None, None) == -1
    # empty inputs are a no-op
    assert lib.mtgr_group_layernorm(None, None, None, None, None, 0, 64, 4, 1e-5, 1, None, None, None) == 0
    assert lib.mtgr_jagged_prep(None, None, 0, 0, None, None, 0, None) == 0


def test_layer_param_errors(lib):
    from generative_recommendation_ranking_grouplayernorm_amd import binding as b

    P = ctypes.c_void_p
    good = dict(W_uqkv=8192, b_uqkv=None, gamma1=8192, beta1=8192, gamma2=8192, beta2=8192, W_o=8192, b_o=None,
                d=256, H=2, dh=128, G=4, eps=1e-5, alpha=1.0)

    def call(**kw):
        p = dict(good, **kw)
        lp = b.LayerParams(*(p[k] for k in ("W_uqkv", "b_uqkv", "gamma1", "beta1", "gamma2", "beta2", "W_o",
                                              "b_o", "d", "H", "dh", "G", "eps", "alpha")))
        return lib.mtgr_hstu_layer_fwd(ctypes.byref(lp), P(8192), P(16384), None, P(4096), P(4096), P(4096), 1,
                                       10, 0.1, 1, P(8192), 1 << 30, None)

    assert call(d=250) == -1        # d != H * dh
    assert call(H=4, dh=64, d=256, G=9) == -1
    assert call(W_o=None) == -1
    assert call(H=2, dh=96, d=192) == -2


@pytest.mark.parametrize("cfg", [1, 2])
def test_flop_counter_matches_oracle_mask(cfg):
    from generative_recommendation_ranking_grouplayernorm_amd import flops

    batch = make_batch(cfg)
    if cfg == 2:
        keep = list(range(0, batch.B, 4))
        off, g, t, _, _ = orc.select_users(batch.offsets, batch.group_ids, batch.timestamps, None, keep)
    else:
        off, g, t = batch.offsets, batch.group_ids, batch.timestamps
    assert flops.visible_pairs(off, g, t) == int(orc.visible_pairs(off, g, t).sum())
