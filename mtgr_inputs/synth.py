"""Seeded generators for jagged user-aggregated token batches and layer weights.

Token order inside one user row is [U | S | R | C] (profile tokens, long-term
sequence, real-time actions, candidates), following the aggregated sample
layout D = [U, S, R, (C, I)_1..K] of the MTGR pages (blog reading, section 4
"data re-arrangement"; marovi summary, "Métodos"; fun-rec 7.3.1).

Everything here is drawing and layout only: lengths, group ids, timestamps,
activations and weights.  No normalisation, projection, mask or attention
arithmetic lives in this module.

The pages train on Meituan's proprietary logs (marovi summary, "Resultados"),
which are not available; the draws below stand in for them with the shapes the
pages give: long-tail history lengths, S <= 1000 / R <= 100 online, 1k / 3k
maximum lengths, 20 exposures against a 1000-long history.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

GROUP_U = 0  # user profile tokens
GROUP_S = 1  # long-term behaviour sequence
GROUP_R = 2  # real-time behaviour sequence
GROUP_C = 3  # candidate (cross + item) tokens
NUM_GROUPS = 4

DAY_SECONDS = 86400

# One entry per workload.  Sizes follow the pages' model shapes (small d512,
# large d1024 with 8x128 heads, 22 layers, sequence caps 1k / 3k) and the
# serving example (one request, 1000 history tokens, K candidates).
CONFIGS: Dict[int, dict] = {
    1: dict(name="tiny_fp32", dtype="f32", B=4, n_u=8, n_s=("uniform", 16, 48),
            n_r=("fixed", 8), n_c=("fixed", 4), d=64, H=2, dh=32, layers=1,
            ts_max=100, x_init="normal0.02", w_init="normal0.02", bias=True),
    2: dict(name="fwd_bf16_d512", dtype="bf16", B=32, n_u=8,
            n_s=("lognormal", 6.0, 1.0, 32, 3000), n_r=("uniform", 0, 64),
            n_c=("fixed", 20), d=512, H=4, dh=128, layers=1,
            ts_max=DAY_SECONDS, x_init="normal1", w_init="xavier", bias=False),
    3: dict(name="fwd22_fp16_d1024", dtype="f16", B=64, n_u=8,
            n_s=("lognormal", 6.0, 1.0, 32, 1000), n_r=("uniform", 0, 64),
            n_c=("uniform", 20, 200), d=1024, H=8, dh=128, layers=22,
            ts_max=DAY_SECONDS, x_init="normal1", w_init="xavier", bias=False),
    4: dict(name="train_bf16_d1024_65536tok", dtype="bf16", total_tokens=65536, n_u=8,
            n_s=("lognormal", 6.0, 1.0, 32, 3000), n_r=("uniform", 0, 64),
            n_c=("fixed", 20), d=1024, H=8, dh=128, layers=1,
            ts_max=DAY_SECONDS, x_init="normal1", w_init="xavier", bias=False),
    5: dict(name="serve_fp16_d1024_sweep", dtype="f16", B=1, n_u=8, n_s=("fixed", 1000),
            n_r=("fixed", 32), n_c=("fixed", 20), d=1024, H=8, dh=128, layers=22,
            ts_max=DAY_SECONDS, x_init="normal1", w_init="xavier", bias=False,
            cand_after_rt=600, K_sweep=(20, 100, 500, 1000)),
}


@dataclass
class Batch:
    """A jagged batch of user rows.

    offsets   int32 [B+1]   token offset of each user, offsets[0] = 0
    group_ids uint8 [T]     0=U, 1=S, 2=R, 3=C, non-decreasing inside a user
    timestamps int64 [T]    U/S carry negative stamps (ignored by the mask)
    lengths   int64 [B, 4]  (n_u, n_s, n_r, n_c) per user
    max_len   int           longest user row N_b
    """

    offsets: np.ndarray
    group_ids: np.ndarray
    timestamps: np.ndarray
    lengths: np.ndarray
    max_len: int
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.offsets.shape[0] - 1)

    @property
    def T(self) -> int:
        return int(self.offsets[-1])


@dataclass
class LayerParams:
    """Float32 master copies of one HSTU layer's weights.

    W_uqkv [4d, d]  (output feature major, blocks U|Q|K|V), b_uqkv [4d] or None
    gamma1, beta1 [G, d]   group norm on the layer input
    gamma2, beta2 [G, d]   group norm on the attention output
    W_o [d, d] (output feature major), b_o [d] or None
    """

    W_uqkv: np.ndarray
    b_uqkv: Optional[np.ndarray]
    gamma1: np.ndarray
    beta1: np.ndarray
    gamma2: np.ndarray
    beta2: np.ndarray
    W_o: np.ndarray
    b_o: Optional[np.ndarray]
    H: int
    dh: int

    @property
    def d(self) -> int:
        return int(self.W_o.shape[0])


def _draw_len(rng: np.random.Generator, spec) -> int:
    kind = spec[0]
    if kind == "fixed":
        return int(spec[1])
    if kind == "uniform":  # inclusive integer range
        return int(rng.integers(spec[1], spec[2] + 1))
    if kind == "lognormal":
        mu, sigma, lo, hi = spec[1:]
        return int(np.clip(np.round(rng.lognormal(mu, sigma)), lo, hi))
    raise ValueError(spec)


def make_batch_from_lengths(lengths, rng: np.random.Generator, ts_max: int,
                            cand_after_rt: Optional[int] = None) -> Batch:
    """Lay out users with the given (n_u, n_s, n_r, n_c) and draw timestamps.

    Timestamps: S tokens get -n_s .. -1 in order, U tokens -n_s-1; real-time
    tokens are sorted uniform draws in [0, ts_max); candidates are unsorted
    uniform draws in [0, ts_max), or, with ``cand_after_rt``, uniform in
    [max_rt + 1, max_rt + cand_after_rt] so that every candidate comes after
    every real-time action.
    """
    lengths = np.asarray(lengths, dtype=np.int64).reshape(-1, 4)
    sizes = lengths.sum(axis=1)
    B = lengths.shape[0]
    offsets = np.zeros(B + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(sizes)
    T = int(offsets[-1])
    groups = np.empty(T, dtype=np.uint8)
    ts = np.empty(T, dtype=np.int64)
    for b in range(B):
        n_u, n_s, n_r, n_c = (int(v) for v in lengths[b])
        o = int(offsets[b])
        groups[o:o + n_u] = GROUP_U
        groups[o + n_u:o + n_u + n_s] = GROUP_S
        groups[o + n_u + n_s:o + n_u + n_s + n_r] = GROUP_R
        groups[o + n_u + n_s + n_r:o + n_u + n_s + n_r + n_c] = GROUP_C
        ts[o:o + n_u] = -n_s - 1
        ts[o + n_u:o + n_u + n_s] = np.arange(-n_s, 0, dtype=np.int64)
        rt = np.sort(rng.integers(0, ts_max, size=n_r)).astype(np.int64)
        ts[o + n_u + n_s:o + n_u + n_s + n_r] = rt
        if cand_after_rt is None:
            cand = rng.integers(0, ts_max, size=n_c)
        else:
            top = int(rt.max()) if n_r > 0 else 0
            cand = rng.integers(top + 1, top + cand_after_rt + 1, size=n_c)
        ts[o + n_u + n_s + n_r:o + n_u + n_s + n_r + n_c] = cand
    max_len = int(sizes.max()) if B > 0 else 0
    return Batch(offsets=offsets, group_ids=groups, timestamps=ts,
                 lengths=lengths, max_len=max_len)


def _token_balanced_lengths(cfg: dict, rng: np.random.Generator) -> List[List[int]]:
    """Draw users until the next one would overflow the token budget, then
    fill the budget exactly (the pages balance per-GPU batches by token count:
    blog 11.3, paper-daily "训练成本" section)."""
    budget = int(cfg["total_tokens"])
    n_u = int(cfg["n_u"])
    n_c = _draw_len(rng, cfg["n_c"])
    s_lo, s_hi = cfg["n_s"][3], cfg["n_s"][4]
    users: List[List[int]] = []
    total = 0
    while True:
        n_s = _draw_len(rng, cfg["n_s"])
        n_r = _draw_len(rng, cfg["n_r"])
        size = n_u + n_s + n_r + n_c
        if total + size <= budget:
            users.append([n_u, n_s, n_r, n_c])
            total += size
            if total == budget:
                break
            continue
        rem = budget - total
        if rem >= n_u + s_lo + n_r + n_c:
            users.append([n_u, rem - n_u - n_r - n_c, n_r, n_c])
        elif rem >= n_u + s_lo + n_c:
            users.append([n_u, rem - n_u - n_c, 0, n_c])
        else:
            # too short for a user of its own: lengthen earlier histories
            for u in reversed(users):
                take = min(rem, s_hi - u[1])
                u[1] += take
                rem -= take
                if rem == 0:
                    break
            assert rem == 0
        break
    return users


def make_batch(cfg_id: int, seed: int = 0, K: Optional[int] = None) -> Batch:
    """The jagged batch of one workload, drawn from ``default_rng([seed, cfg_id])``.

    ``K`` overrides the candidate count (serving sweep)."""
    cfg = CONFIGS[cfg_id]
    rng = np.random.default_rng([seed, cfg_id])
    if "total_tokens" in cfg:
        users = _token_balanced_lengths(cfg, rng)
    else:
        users = []
        for _ in range(cfg["B"]):
            n_s = _draw_len(rng, cfg["n_s"])
            n_r = _draw_len(rng, cfg["n_r"])
            n_c = _draw_len(rng, cfg["n_c"]) if K is None else int(K)
            users.append([cfg["n_u"], n_s, n_r, n_c])
    batch = make_batch_from_lengths(users, rng, cfg["ts_max"], cfg.get("cand_after_rt"))
    batch.meta = dict(cfg_id=cfg_id, seed=seed, name=cfg["name"])
    return batch


def make_layer_params(d: int, H: int, rng: np.random.Generator, w_init: str = "xavier",
                      bias: bool = False, G: int = NUM_GROUPS) -> LayerParams:
    """Random-init weights of one layer (there are no trained weights to load).

    Group-norm affine parameters are drawn around (1, 0) per group so that a
    wrong group routing changes the result: gamma = 1 + N(0, 0.1),
    beta = N(0, 0.1)."""
    assert d % H == 0
    dh = d // H

    def lin(out_f, in_f):
        if w_init == "xavier":
            bound = np.sqrt(6.0 / (in_f + out_f))
            return rng.uniform(-bound, bound, size=(out_f, in_f)).astype(np.float32)
        if w_init == "normal0.02":
            return rng.normal(0.0, 0.02, size=(out_f, in_f)).astype(np.float32)
        raise ValueError(w_init)

    W_uqkv = lin(4 * d, d)
    b_uqkv = rng.normal(0.0, 0.02, size=4 * d).astype(np.float32) if bias else None
    gamma1 = (1.0 + rng.normal(0.0, 0.1, size=(G, d))).astype(np.float32)
    beta1 = rng.normal(0.0, 0.1, size=(G, d)).astype(np.float32)
    gamma2 = (1.0 + rng.normal(0.0, 0.1, size=(G, d))).astype(np.float32)
    beta2 = rng.normal(0.0, 0.1, size=(G, d)).astype(np.float32)
    W_o = lin(d, d)
    b_o = rng.normal(0.0, 0.02, size=d).astype(np.float32) if bias else None
    return LayerParams(W_uqkv, b_uqkv, gamma1, beta1, gamma2, beta2, W_o, b_o, H, dh)


def make_activations(T: int, d: int, rng: np.random.Generator, init: str = "normal1") -> np.ndarray:
    if init == "normal1":
        return rng.normal(0.0, 1.0, size=(T, d)).astype(np.float32)
    if init == "normal0.02":
        return rng.normal(0.0, 0.02, size=(T, d)).astype(np.float32)
    raise ValueError(init)


def make_probe_head(d: int, seed: int = 1234) -> np.ndarray:
    """Fixed probe vector w ~ N(0, 1/d) used to turn candidate outputs into
    scores for the fp16-vs-fp32 score-difference check."""
    rng = np.random.default_rng(seed)
    return rng.normal(0.0, 1.0 / np.sqrt(d), size=d)


def _truncate_candidates(batch: Batch, x: np.ndarray, K: int):
    """Keep the first K candidates of a single-user batch (serving sweep: the
    history and the first candidates stay identical across K)."""
    assert batch.B == 1
    n_u, n_s, n_r, n_c = (int(v) for v in batch.lengths[0])
    assert K <= n_c
    N = n_u + n_s + n_r + K
    lengths = np.array([[n_u, n_s, n_r, K]], dtype=np.int64)
    out = Batch(offsets=np.array([0, N], dtype=np.int32), group_ids=batch.group_ids[:N].copy(),
                timestamps=batch.timestamps[:N].copy(), lengths=lengths,
                max_len=batch.max_len, meta=dict(batch.meta, K=K))
    return out, x[:N].copy()


def config_inputs(cfg_id: int, seed: int = 0, K: Optional[int] = None):
    """Batch, per-layer params and layer input X of one workload.

    For the serving sweep the row is drawn once with the largest K and cut to
    the first K candidates; ``max_len`` stays that of the largest row, so the
    attention scale is the same for every K."""
    cfg = CONFIGS[cfg_id]
    wrng = np.random.default_rng([seed, cfg_id, 1])
    params = [make_layer_params(cfg["d"], cfg["H"], wrng, cfg["w_init"], cfg["bias"])
              for _ in range(cfg["layers"])]
    xrng = np.random.default_rng([seed, cfg_id, 2])
    if "K_sweep" in cfg:
        kmax = max(cfg["K_sweep"])
        full = make_batch(cfg_id, seed, K=kmax)
        x = make_activations(full.T, cfg["d"], xrng, cfg["x_init"])
        batch, x = _truncate_candidates(full, x, kmax if K is None else int(K))
        return batch, params, x
    batch = make_batch(cfg_id, seed, K=K)
    x = make_activations(batch.T, cfg["d"], xrng, cfg["x_init"])
    return batch, params, x


def make_user_pool(cfg_id: int, min_tokens: int, seed: int = 0) -> Batch:
    """Users drawn one after another with a workload's length distributions
    (no trimming) until they hold at least ``min_tokens`` tokens: the pool a
    training batch is cut from after Stochastic Length sampling shortens its
    histories (paper-daily "计算量涨了 65 倍" section)."""
    cfg = CONFIGS[cfg_id]
    rng = np.random.default_rng([seed, cfg_id, 7])
    users: List[List[int]] = []
    total = 0
    while total < min_tokens:
        n_s = _draw_len(rng, cfg["n_s"])
        n_r = _draw_len(rng, cfg["n_r"])
        n_c = _draw_len(rng, cfg["n_c"])
        users.append([cfg["n_u"], n_s, n_r, n_c])
        total += cfg["n_u"] + n_s + n_r + n_c
    batch = make_batch_from_lengths(users, rng, cfg["ts_max"], cfg.get("cand_after_rt"))
    batch.meta = dict(cfg_id=cfg_id, seed=seed, name=cfg["name"] + "_pool")
    return batch


def make_uniform_draws(n: int, seed: int = 0) -> np.ndarray:
    """``n`` float32 uniforms in [0, 1): the per-user random numbers of
    Stochastic Length sampling, drawn here and passed to both sides."""
    return np.random.default_rng([seed, 11]).random(n, dtype=np.float32)


@dataclass
class HeadParams:
    """Candidate head: Linear(d -> h) + bias, then Linear(h -> n_tasks) + bias."""
    W1: np.ndarray
    b1: Optional[np.ndarray]
    W2: np.ndarray
    b2: Optional[np.ndarray]


def make_head_params(d: int, h: int, n_tasks: int, rng: np.random.Generator, bias: bool = True) -> HeadParams:
    """Xavier-uniform weights, biases N(0, 0.02) (random init: no trained head)."""
    def lin(out_f, in_f):
        bound = np.sqrt(6.0 / (in_f + out_f))
        return rng.uniform(-bound, bound, size=(out_f, in_f)).astype(np.float32)

    W1 = lin(h, d)
    b1 = rng.normal(0.0, 0.02, size=h).astype(np.float32) if bias else None
    W2 = lin(n_tasks, h)
    b2 = rng.normal(0.0, 0.02, size=n_tasks).astype(np.float32) if bias else None
    return HeadParams(W1, b1, W2, b2)


def make_labels(n_cand: int, rng: np.random.Generator, p_click: float = 0.1,
                p_order: float = 0.3) -> np.ndarray:
    """[n_cand, 2] float32 labels: click ~ Bernoulli(p_click), and click-then-
    order (a subset of clicks) ~ click * Bernoulli(p_order)."""
    click = (rng.random(n_cand) < p_click).astype(np.float32)
    order = click * (rng.random(n_cand) < p_order).astype(np.float32)
    return np.stack([click, order], axis=1)
