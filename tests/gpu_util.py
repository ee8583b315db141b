"""Helpers shared by the GPU parity tests: device placement of seeded inputs,
rounding to the device dtype, and error measures."""

from __future__ import annotations

import sys

import numpy as np
import torch

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
# rel-L2 bars: 1e-5 for fp32 storage, 1e-2 for bf16/f16 storage
TOL = {torch.float32: 1e-5, torch.bfloat16: 1e-2, torch.float16: 1e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def rounded(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """CPU tensor of ``a`` rounded to ``dtype``."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def meta(batch, dev):
    return (torch.from_numpy(batch.offsets).to(dev), torch.from_numpy(batch.group_ids).to(dev),
            torch.from_numpy(batch.timestamps).to(dev))


class P64:
    """Layer parameters in fp64 as the oracle expects them."""


def params_to(p, dtype: torch.dtype, dev):
    """(device tensors dict, fp64 oracle params) from LayerParams, both from the
    same rounded values."""
    names = ["W_uqkv", "gamma1", "beta1", "gamma2", "beta2", "W_o", "b_uqkv", "b_o"]
    dev_p = {}
    q = P64()
    for k in names:
        v = getattr(p, k)
        if v is None:
            setattr(q, k, None)
            continue
        t = rounded(v, dtype)
        dev_p[k] = t.to(dev)
        setattr(q, k, f64(t))
    q.H = p.H
    return dev_p, q


GROUP_SETS = {"U/S": (0, 1), "R": (2,), "C": (3,)}


def group_errors(got, ref, group_ids):
    """rel-L2 over the rows of each token group (U/S, R, C) and the largest
    absolute error of any row, so that an error confined to a few rows of one
    group is not diluted by the rest."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    g = np.asarray(group_ids)
    out = {}
    for name, grp in GROUP_SETS.items():
        sel = np.isin(g, grp)
        if sel.any():
            out[name] = rel_l2(got[sel], ref[sel])
    out["max_abs"] = float(np.max(np.abs(got - ref))) if got.size else 0.0
    return out
