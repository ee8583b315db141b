"""Plain fp64 CPU oracle of the candidate head and the discriminative loss.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module; only the tests and the benchmark's CPU-baseline leg do.  It
shares no code with the HIP kernels; weights and labels come from the seeded
generators in ``mtgr_inputs``.

Sources (the pages' titles and sections):
  "MTGR：工业级生成式推荐框架" (zzxanthony blog), 5.4 and 7 (the candidate
  tokens' outputs pass through an MLP to one logit per candidate) and 6 (the
  training objective is a discriminative ranking loss, not next-token);
  "MTGR：混合范式建模" (fun-rec 7.3), 7.3.1: the loss is taken at candidate
  positions only;
  "MTGR：美团外卖生成式推荐Scaling Law落地实践" (paper-daily), 它解决什么问题:
  the model outputs a click-through rate and a conversion rate for every
  exposed candidate.

Readings taken where the pages are silent (also listed in the design notes):
  * The MLP is Linear(d -> h) + bias, SiLU, Linear(h -> n_tasks) + bias.
  * The tasks are click (CTR) and click-then-order (CTCVR), one logit each.
  * The loss is the binary cross-entropy of each task's logit, averaged over
    the batch's candidate tokens and summed over tasks.
  * The head reads the last layer's output rows of the candidate tokens as
    they are (no extra norm).
"""

from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

from .mtgr_oracle import GROUP_C


def candidate_rows(group_ids) -> np.ndarray:
    """Row indices of the candidate tokens, in batch order."""
    return np.nonzero(np.asarray(group_ids) == GROUP_C)[0]


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _silu_grad(z):
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def head_fwd(p, x, group_ids) -> Tuple[np.ndarray, Dict[str, np.ndarray]]:
    """Logits [n_cand, n_tasks] of the candidate rows of x [T, d]."""
    rows = candidate_rows(group_ids)
    xc = np.asarray(x, np.float64)[rows]
    z1 = xc @ np.asarray(p.W1, np.float64).T
    if p.b1 is not None:
        z1 = z1 + np.asarray(p.b1, np.float64)
    h = _silu(z1)
    logits = h @ np.asarray(p.W2, np.float64).T
    if p.b2 is not None:
        logits = logits + np.asarray(p.b2, np.float64)
    return logits, {"rows": rows, "xc": xc, "z1": z1, "h": h}


def bce_loss(logits, labels) -> float:
    """Mean over candidates of the summed per-task binary cross-entropy:
    -y log sigmoid(z) - (1 - y) log(1 - sigmoid(z)) = softplus(z) - y z."""
    z = np.asarray(logits, np.float64)
    y = np.asarray(labels, np.float64)
    n = z.shape[0]
    if n == 0:
        return 0.0
    return float(np.sum(np.logaddexp(0.0, z) - y * z) / n)


def head_loss_bwd(p, cache, logits, labels, T: int):
    """Gradients of bce_loss(head_fwd(x)) with respect to x (zero on every
    non-candidate row) and the head weights."""
    z = np.asarray(logits, np.float64)
    y = np.asarray(labels, np.float64)
    n = z.shape[0]
    dz = (1.0 / (1.0 + np.exp(-z)) - y) / max(n, 1)
    W1 = np.asarray(p.W1, np.float64)
    W2 = np.asarray(p.W2, np.float64)
    grads = {"W2": dz.T @ cache["h"], "b2": dz.sum(axis=0)}
    dh = dz @ W2
    dz1 = dh * _silu_grad(cache["z1"])
    grads["W1"] = dz1.T @ cache["xc"]
    grads["b1"] = dz1.sum(axis=0)
    dx = np.zeros((T, W1.shape[1]))
    dx[cache["rows"]] = dz1 @ W1
    grads["dz1"] = dz1
    return dx, grads
