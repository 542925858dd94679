"""fp64 reference of the gradients of the sparse MoE layer.

TEST INFRASTRUCTURE ONLY (see the package header).

Why gradients: the expanded layers are bases for fine-tuning, and activating
more experts per token gives each token's gradient more parameters to reach
("gpt-oss-40b-64a8-init" page, section 1, Train Wide, Deploy Narrow).
Section 5.2 of the same page asks for selective gradient control: the
original experts may be frozen while the copies train, and the router stays
trainable throughout.  So the gradients computed are those of the router
(W_r, b_r), of every trainable expert's three matrices, and of the layer
input h.

The layer (section 2, Proof; field guide cutaway 03 for the SwiGLU expert):

    s = W_r h + b_r,   S = top-k(s),   p_i = exp(s_i) / sum_{j in S} exp(s_j)
    g_i = W_g[i] h,   u_i = W_u[i] h,   a_i = silu(g_i) * u_i,   y_i = W_d[i] a_i
    out = sum_{i in S} p_i y_i

Given an upstream gradient ``dout`` (the derivative of a scalar loss with
respect to ``out``), the chain rule gives, per token and selected expert i:

    dp_i  = dout . y_i
    da_i  = p_i W_d[i]^T dout
    dg_i  = da_i * u_i * silu'(g_i),   du_i = da_i * silu(g_i)
    dW_d[i] += (p_i dout) a_i^T,  dW_g[i] += dg_i h^T,  dW_u[i] += du_i h^T
    dh    += W_g[i]^T dg_i + W_u[i]^T du_i
    ds_i  = p_i (dp_i - sum_{j in S} p_j dp_j)      (softmax over S)
    dW_r[i] += ds_i h,  db_r[i] += ds_i,  dh += ds_i W_r[i]

The selection S is piecewise constant in s, so it passes no gradient: logits
outside S get ds = 0.  ``silu'(z) = sigma(z) (1 + z (1 - sigma(z)))``.

Parity status: pinned.  Central finite differences of the (separately
pinned) forward oracle in fp64 on small layers, for every output of this
module; the silent expansion carried to the gradients (the copies of an
expert share its gradient equally); k = E, where the layer is the dense
softmax mixture; the frozen experts' gradients left out without changing the
others.
"""
from __future__ import annotations

import numpy as np

from .moe import LayerWeights, router_logits, select_topk, selected_softmax, silu


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d silu / dz = sigma(z) (1 + z (1 - sigma(z)))."""
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-z))
    return sig * (1.0 + z * (1.0 - sig))


def moe_backward(h: np.ndarray, weights: LayerWeights, k: int, dout: np.ndarray, idx: np.ndarray | None = None,
                 trainable: np.ndarray | None = None) -> dict:
    """Gradients of ``sum(dout * out)`` for the layer on float64 ``h [T, H]``.

    ``idx`` replaces the selection (a valid top-k set per token, as in
    ``moe_forward``); ``trainable[e]`` false leaves expert e's matrices out
    (their entries are None).  Evaluated expert by expert, rows of an expert
    together.

    Returns ``dh [T, H]``, ``dw_router [E, H]``, ``db_router [E]``, lists
    ``dw_gate`` / ``dw_up`` ``[I, H]`` and ``dw_down`` ``[H, I]`` per expert,
    and ``idx``, ``p``, ``dp [T, k]``, ``ds [T, k]``."""
    h = np.asarray(h, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    T, H = h.shape
    s = router_logits(h, weights.w_router, weights.b_router)
    E = s.shape[1]
    if idx is None:
        idx = select_topk(s, k)
    p = selected_softmax(s, idx)
    if trainable is None:
        trainable = np.ones(E, dtype=bool)
    dh = np.zeros((T, H))
    dp = np.zeros((T, k))
    dw_gate, dw_up, dw_down = [None] * E, [None] * E, [None] * E
    for e in range(E):
        rows, slots = np.nonzero(idx == e)
        wg, wu, wd = weights.expert(e)
        if trainable[e]:
            dw_gate[e] = np.zeros_like(wg)
            dw_up[e] = np.zeros_like(wu)
            dw_down[e] = np.zeros_like(wd)
        if rows.size == 0:
            continue
        x = h[rows]
        pe = p[rows, slots][:, None]
        g = x @ wg.T
        u = x @ wu.T
        a = silu(g) * u
        y = a @ wd.T
        dy = dout[rows]
        dp[rows, slots] = np.sum(dy * y, axis=1)
        da = pe * (dy @ wd)
        dg = da * u * silu_grad(g)
        du = da * silu(g)
        np.add.at(dh, rows, dg @ wg + du @ wu)
        if trainable[e]:
            dw_down[e] = (pe * dy).T @ a
            dw_gate[e] = dg.T @ x
            dw_up[e] = du.T @ x
    ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    dsd = np.zeros((T, E))
    np.put_along_axis(dsd, idx, ds, axis=1)
    dh += dsd @ weights.w_router
    return {"dh": dh, "dw_router": dsd.T @ h, "db_router": dsd.sum(axis=0), "dw_gate": dw_gate,
            "dw_up": dw_up, "dw_down": dw_down, "idx": idx, "p": p, "dp": dp, "ds": ds}
