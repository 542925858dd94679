"""fp64 reference of the pre-normalised MoE sublayer with its residual add.

TEST INFRASTRUCTURE ONLY (see the package header).

What it computes, per token ``t`` with residual-stream row ``x_t``:

1. ``n_t = g * x_t / sqrt(mean_j(x_t[j]^2) + eps)`` — Root Mean Square Layer
   Normalization, applied before the MoE sublayer ("gpt-oss 20B" field
   guide, cutaway 04 "One decoder block": RMSNorm before attention and before
   MoE).  The normaliser has one learned gain per hidden feature and no bias
   ("openai/gpt-oss-20b" fixture comparison page, "Where the parameters are":
   the final norm holds 2.9K parameters at hidden size 2880, 64 at 64), stored
   like the router in the activation format ("gpt-oss-40b-64a8-init" page,
   section 4 "Architecture": norms in BF16).  The pages give neither the
   formula nor epsilon; this is the standard definition of RMSNorm, with
   epsilon inside the square root, and epsilon is an argument;
2. ``out_t = x_t + MoE(n)_t`` — the sublayer's output added back to the
   residual stream (same cutaway), ``MoE`` being ``moe.moe_forward``.

Parity status: pinned.  ``rms_norm`` by closed forms and invariants that do
not restate its formula (unit mean square of the output, a constant row, the
joint scaling of input and epsilon, the gain acting per feature, a
hand-computed two-element example); ``block_forward`` by a zero-expert special
case (output equals the input exactly) and by an independent per-token
evaluation built on ``moe.moe_forward_per_token``.
"""
from __future__ import annotations

import numpy as np

from .moe import LayerWeights, moe_forward, moe_forward_per_token


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """``g * x / sqrt(mean(x^2) + eps)`` over the last axis, in float64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(g, dtype=np.float64) * (x / np.sqrt(ms + eps))


def block_forward(x: np.ndarray, g: np.ndarray, eps: float, weights: LayerWeights, k: int,
                  idx: np.ndarray | None = None, tokens: np.ndarray | None = None, workers: int = 1) -> dict:
    """``x + MoE(rms_norm(x))``.  Returns the ``moe_forward`` dictionary with
    ``out`` replaced by the block output (for ``tokens``, default all) and the
    normalised input added as ``n``."""
    n = rms_norm(x, g, eps)
    r = moe_forward(n, weights, k, idx=idx, tokens=tokens, workers=workers)
    rows = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    r["out"] = np.asarray(x, dtype=np.float64)[rows] + r["out"]
    r["n"] = n
    return r


def block_forward_per_token(x: np.ndarray, g: np.ndarray, eps: float, weights: LayerWeights, k: int) -> np.ndarray:
    """The same sublayer token by token: the mean square by an explicit loop,
    then the per-token MoE evaluation."""
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    n = np.empty_like(x)
    for t in range(T):
        acc = 0.0
        for j in range(H):
            acc += x[t, j] * x[t, j]
        scale = 1.0 / np.sqrt(acc / H + eps)
        for j in range(H):
            n[t, j] = g[j] * x[t, j] * scale
    return x + moe_forward_per_token(n, weights, k)["out"]
