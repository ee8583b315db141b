"""Plain fp64 CPU oracle of one MTGR HSTU layer over a jagged user batch.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module; only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP kernels: inputs come from the seeded
generators in ``mtgr_inputs``, which hold none of the layer's arithmetic.

Every function is the plain definition, written out in float64 with NumPy,
one user (and one head) at a time, without blocking, fusion or reordering.
Matrix products use ``numpy.matmul`` as a library primitive.

Sources (the pages' titles and sections):
  [blog]  "MTGR：工业级生成式推荐框架" (zzxanthony blog): 4 data re-arrangement,
          7 HSTU encoder, 8 Group-Layer Normalization, 9 Dynamic Masking.
  [wiki]  "MTGR: Industrial-Scale Generative Recommendation Framework in
          Meituan/es" (marovi): Métodos, the V-tilde and X-update equations.
  [pd]    "MTGR：美团外卖生成式推荐Scaling Law落地实践" (paper-daily summary):
          模型怎么搭 (layer order), 训练数据怎么组织，掩码怎么设 (timestamps).
  [fr]    "MTGR：混合范式建模" (fun-rec 7.3): 7.3.3 GLN formula, 7.3.4 rules 1-3.
  [dr]    paper-daily deep reading of the Meituan blog: 2 方法详解.

Readings taken where the pages are silent or disagree (each is also listed in
the design notes):
  * GLN: statistics per token over the d features (biased variance, eps under
    the root), affine gamma/beta chosen by the token's group.
  * The attention output is group-normalised (own gamma2/beta2) and then gated
    by U ([pd] 模型怎么搭 order), then one linear layer and the residual.
  * SiLU on all four projections U, Q, K, V ([pd] 模型怎么搭).
  * Attention normaliser: an explicit scalar ``attn_scale`` (1/max_len of the
    batch), temperature ``alpha`` inside the SiLU (1 by default).
  * Mask: static (U, S) keys visible to every query; a real-time key j is
    visible to real-time or candidate query i iff t_j < t_i (strict) or
    i == j; a candidate key is visible only to itself.

Parity pins: see the tests (golden masks from the pages' worked example,
torch library reductions, closed forms, finite differences, invariants).
``group_layernorm`` with pooled statistics is not offered: parity unpinned
for that reading, which is not the contract.
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

GROUP_U, GROUP_S, GROUP_R, GROUP_C = 0, 1, 2, 3


# --------------------------------------------------------------------------
# a1: jagged layout
# --------------------------------------------------------------------------
def segments(offsets: np.ndarray, group_ids: np.ndarray) -> np.ndarray:
    """Per user b: [start of U, start of S, start of R, start of C, end].

    A user row is [U | S | R | C] ([blog] 4; [fr] 7.3.1), so each start is the
    previous start plus that group's token count."""
    offsets = np.asarray(offsets, dtype=np.int64)
    g = np.asarray(group_ids)
    B = offsets.shape[0] - 1
    seg = np.zeros((B, 5), dtype=np.int64)
    for b in range(B):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        gb = g[lo:hi]
        start = lo
        for grp in range(4):
            seg[b, grp] = start
            start += int(np.count_nonzero(gb == grp))
        seg[b, 4] = hi
    return seg


# --------------------------------------------------------------------------
# a2 / a5: Group LayerNorm  ([fr] 7.3.3 formula; [pd] 模型怎么搭; [dr] 2)
# --------------------------------------------------------------------------
def group_layernorm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray,
                    group_ids: np.ndarray, eps: float):
    """y_i = (x_i - mean_i) / sqrt(var_i + eps) * gamma[g(i)] + beta[g(i)].

    Returns (y, mean [T], rstd [T])."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(group_ids, dtype=np.int64)
    mean = x.mean(axis=1)
    var = ((x - mean[:, None]) ** 2).mean(axis=1)
    rstd = 1.0 / np.sqrt(var + eps)
    xn = (x - mean[:, None]) * rstd[:, None]
    y = xn * np.asarray(gamma, np.float64)[g] + np.asarray(beta, np.float64)[g]
    return y, mean, rstd


def group_layernorm_bwd(dy: np.ndarray, x: np.ndarray, mean: np.ndarray, rstd: np.ndarray,
                        gamma: np.ndarray, group_ids: np.ndarray, G: int = 4):
    """Gradients of ``group_layernorm`` w.r.t. x, gamma and beta.

    With n = (x - mean) * rstd and e = dy * gamma[g]:
      dx = rstd * (e - mean_j(e) - n * mean_j(e * n))
      dgamma[c] = sum over tokens of group c of dy * n,  dbeta[c] = sum of dy."""
    dy = np.asarray(dy, np.float64)
    x = np.asarray(x, np.float64)
    g = np.asarray(group_ids, dtype=np.int64)
    n = (x - mean[:, None]) * rstd[:, None]
    e = dy * np.asarray(gamma, np.float64)[g]
    dx = rstd[:, None] * (e - e.mean(axis=1, keepdims=True)
                          - n * (e * n).mean(axis=1, keepdims=True))
    d = x.shape[1]
    dgamma = np.zeros((G, d))
    dbeta = np.zeros((G, d))
    for c in range(G):
        sel = g == c
        dgamma[c] = (dy[sel] * n[sel]).sum(axis=0)
        dbeta[c] = dy[sel].sum(axis=0)
    return dx, dgamma, dbeta


# --------------------------------------------------------------------------
# a3: fused UQKV projection with SiLU  ([pd] 模型怎么搭; [wiki] Métodos)
# --------------------------------------------------------------------------
def sigmoid(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z)."""
    return z * sigmoid(z)


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d/dz [z * sigmoid(z)] = sigmoid(z) * (1 + z * (1 - sigmoid(z)))."""
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def uqkv_projection(xhat: np.ndarray, W_uqkv: np.ndarray, b_uqkv: Optional[np.ndarray]):
    """z = xhat W^T + b (W is [4d, d]); returns (z, SiLU(z)).  Columns of z are
    the blocks U | Q | K | V, each d wide and split into heads of dh."""
    z = np.asarray(xhat, np.float64) @ np.asarray(W_uqkv, np.float64).T
    if b_uqkv is not None:
        z = z + np.asarray(b_uqkv, np.float64)[None, :]
    return z, silu(z)


# --------------------------------------------------------------------------
# Dynamic mask  ([fr] 7.3.4 rules 1-3; [blog] 9.1-9.3; [wiki] Métodos;
#                [pd] 训练数据怎么组织，掩码怎么设)
# --------------------------------------------------------------------------
def mask_matrix(group_ids: np.ndarray, timestamps: np.ndarray) -> np.ndarray:
    """M[i, j] = 1 when query token i may attend to key token j (one user).

    rule 1: U and S keys are visible to every token;
    rule 2: a real-time key j is visible to a real-time or candidate query i
            when t_j < t_i, and always to itself;
    rule 3: a candidate key is visible only to itself."""
    g = np.asarray(group_ids, dtype=np.int64)
    t = np.asarray(timestamps, dtype=np.int64)
    N = g.shape[0]
    same = np.eye(N, dtype=bool)
    key_static = (g == GROUP_U) | (g == GROUP_S)
    key_rt = g == GROUP_R
    key_cand = g == GROUP_C
    query_dynamic = (g == GROUP_R) | (g == GROUP_C)
    earlier = t[None, :] < t[:, None]  # [i, j]: t_j < t_i
    M = np.broadcast_to(key_static[None, :], (N, N)).copy()
    M |= key_rt[None, :] & query_dynamic[:, None] & (earlier | same)
    M |= key_cand[None, :] & same
    return M


def visible_pairs(offsets: np.ndarray, group_ids: np.ndarray, timestamps: np.ndarray) -> np.ndarray:
    """Number of visible (query, key) pairs per user: the sum of its mask."""
    offsets = np.asarray(offsets, dtype=np.int64)
    out = np.zeros(offsets.shape[0] - 1, dtype=np.int64)
    for b in range(out.shape[0]):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        out[b] = int(mask_matrix(group_ids[lo:hi], timestamps[lo:hi]).sum())
    return out


# --------------------------------------------------------------------------
# a4 / a7: pointwise SiLU attention under the dynamic mask
#   ([wiki] Métodos: silu(K^T Q) / normaliser, masked, times V, no softmax;
#    [pd] 模型怎么搭: weights SiLU(QK^T) without softmax)
# --------------------------------------------------------------------------
def hstu_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, offsets: np.ndarray,
                   group_ids: np.ndarray, timestamps: np.ndarray, H: int,
                   alpha: float, attn_scale: float) -> np.ndarray:
    """O_i,h = attn_scale * sum_j M_ij * SiLU(alpha * <q_i,h, k_j,h>) * v_j,h.

    q, k, v: [T, H*dh], head h occupies columns h*dh .. (h+1)*dh."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, d = q.shape
    dh = d // H
    o = np.zeros((T, d))
    offsets = np.asarray(offsets, dtype=np.int64)
    for b in range(offsets.shape[0] - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        if hi == lo:
            continue
        M = mask_matrix(group_ids[lo:hi], timestamps[lo:hi])
        for h in range(H):
            c = slice(h * dh, (h + 1) * dh)
            S = alpha * (q[lo:hi, c] @ k[lo:hi, c].T)
            A = silu(S) * M
            o[lo:hi, c] = attn_scale * (A @ v[lo:hi, c])
    return o


def hstu_attention_bwd(q, k, v, do, offsets, group_ids, timestamps, H: int,
                       alpha: float, attn_scale: float):
    """Gradients of ``hstu_attention`` for an upstream gradient dO.

    With S = alpha q k^T, A = SiLU(S) * M, O = c A v:
      dv = c A^T dO,  dA = c dO v^T,  dS = dA * M * SiLU'(S),
      dq = alpha dS k,  dk = alpha dS^T q."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    T, d = q.shape
    dh = d // H
    dq = np.zeros((T, d))
    dk = np.zeros((T, d))
    dv = np.zeros((T, d))
    offsets = np.asarray(offsets, dtype=np.int64)
    for b in range(offsets.shape[0] - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        if hi == lo:
            continue
        M = mask_matrix(group_ids[lo:hi], timestamps[lo:hi])
        for h in range(H):
            c = slice(h * dh, (h + 1) * dh)
            S = alpha * (q[lo:hi, c] @ k[lo:hi, c].T)
            A = silu(S) * M
            dv[lo:hi, c] = attn_scale * (A.T @ do[lo:hi, c])
            dA = attn_scale * (do[lo:hi, c] @ v[lo:hi, c].T)
            dS = dA * M * silu_grad(S)
            dq[lo:hi, c] = alpha * (dS @ k[lo:hi, c])
            dk[lo:hi, c] = alpha * (dS.T @ q[lo:hi, c])
    return dq, dk, dv


# --------------------------------------------------------------------------
# One layer: GLN -> UQKV+SiLU -> attention -> GLN(AV) * U -> linear + residual
#   ([pd] 模型怎么搭; [wiki] Métodos X-update; [dr] 2 per-layer input norm)
# --------------------------------------------------------------------------
def layer_fwd(p, x: np.ndarray, offsets, group_ids, timestamps, alpha: float,
              attn_scale: float, eps: float = 1e-5):
    """Forward of one HSTU layer.  ``p`` has W_uqkv [4d,d], b_uqkv, gamma1,
    beta1, gamma2, beta2 [G,d], W_o [d,d], b_o, H.  Returns (x_out, saved)."""
    x = np.asarray(x, np.float64)
    d = x.shape[1]
    xhat, mean1, rstd1 = group_layernorm(x, p.gamma1, p.beta1, group_ids, eps)
    z, a = uqkv_projection(xhat, p.W_uqkv, p.b_uqkv)
    u, q, k, v = a[:, :d], a[:, d:2 * d], a[:, 2 * d:3 * d], a[:, 3 * d:]
    o = hstu_attention(q, k, v, offsets, group_ids, timestamps, p.H, alpha, attn_scale)
    n2, mean2, rstd2 = group_layernorm(o, p.gamma2, p.beta2, group_ids, eps)
    y = n2 * u
    x_out = x + y @ np.asarray(p.W_o, np.float64).T
    if p.b_o is not None:
        x_out = x_out + np.asarray(p.b_o, np.float64)[None, :]
    saved = dict(xhat=xhat, mean1=mean1, rstd1=rstd1, z=z, uqkv=a, o=o, n2=n2,
                 mean2=mean2, rstd2=rstd2, y=y)
    return x_out, saved


def layer_bwd(p, x: np.ndarray, saved: Dict[str, np.ndarray], dx_out: np.ndarray,
              offsets, group_ids, timestamps, alpha: float, attn_scale: float):
    """Backward of ``layer_fwd`` for an upstream gradient dx_out.

    Returns (dx, grads) with grads keys W_uqkv, b_uqkv, gamma1, beta1, gamma2,
    beta2, W_o, b_o, and the intermediates dy, dU, dO, dQ, dK, dV, dz, dxhat."""
    x = np.asarray(x, np.float64)
    dx_out = np.asarray(dx_out, np.float64)
    d = x.shape[1]
    W_o = np.asarray(p.W_o, np.float64)
    W_uqkv = np.asarray(p.W_uqkv, np.float64)
    a = saved["uqkv"]
    u, q, k, v = a[:, :d], a[:, d:2 * d], a[:, 2 * d:3 * d], a[:, 3 * d:]
    # output projection
    dy = dx_out @ W_o
    dW_o = dx_out.T @ saved["y"]
    db_o = dx_out.sum(axis=0)
    # gate and second group norm
    du = dy * saved["n2"]
    dn2 = dy * u
    do, dgamma2, dbeta2 = group_layernorm_bwd(dn2, saved["o"], saved["mean2"], saved["rstd2"],
                                              p.gamma2, group_ids)
    # attention
    dq, dk, dv = hstu_attention_bwd(q, k, v, do, offsets, group_ids, timestamps, p.H,
                                    alpha, attn_scale)
    # UQKV projection and its SiLU
    da = np.concatenate([du, dq, dk, dv], axis=1)
    dz = da * silu_grad(saved["z"])
    dxhat = dz @ W_uqkv
    dW_uqkv = dz.T @ saved["xhat"]
    db_uqkv = dz.sum(axis=0)
    # input group norm and residual
    dx1, dgamma1, dbeta1 = group_layernorm_bwd(dxhat, x, saved["mean1"], saved["rstd1"],
                                               p.gamma1, group_ids)
    dx = dx1 + dx_out
    grads = dict(W_uqkv=dW_uqkv, b_uqkv=db_uqkv, gamma1=dgamma1, beta1=dbeta1,
                 gamma2=dgamma2, beta2=dbeta2, W_o=dW_o, b_o=db_o,
                 dy=dy, dU=du, dO=do, dQ=dq, dK=dk, dV=dv, dz=dz, dxhat=dxhat)
    return dx, grads


def stack_fwd(params: Sequence, x: np.ndarray, offsets, group_ids, timestamps,
              alpha: float, attn_scale: float, eps: float = 1e-5) -> np.ndarray:
    """L stacked layers ([blog] 7; [wiki] Métodos: L stacked HSTU blocks)."""
    h = np.asarray(x, np.float64)
    for p in params:
        h, _ = layer_fwd(p, h, offsets, group_ids, timestamps, alpha, attn_scale, eps)
    return h


def candidate_scores(x_out: np.ndarray, group_ids: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Probe score sigmoid(w . x) of every candidate token (fp64)."""
    sel = np.asarray(group_ids) == GROUP_C
    return sigmoid(np.asarray(x_out, np.float64)[sel] @ np.asarray(w, np.float64))


def select_users(offsets, group_ids, timestamps, x, users: List[int]):
    """Sub-batch made of the given users (layers act on users independently
    once the attention scale is fixed)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    rows = np.concatenate([np.arange(offsets[b], offsets[b + 1]) for b in users])
    sizes = [int(offsets[b + 1] - offsets[b]) for b in users]
    new_off = np.zeros(len(users) + 1, dtype=np.int64)
    new_off[1:] = np.cumsum(sizes)
    return new_off, np.asarray(group_ids)[rows], np.asarray(timestamps)[rows], \
        (None if x is None else np.asarray(x)[rows]), rows
