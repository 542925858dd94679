"""fp64 reference of decode attention with learned sinks.

TEST INFRASTRUCTURE ONLY (see the package header).

What it computes, for every sequence ``b`` and query head ``h`` (the newest
token of the sequence, at position ``len_b - 1``):

1. scores ``s_j = scale * q[b, h] . k[b, g(h), j]`` for the visible keys
   ``j``; ``g(h) = h // (Hq / Hkv)``: query heads share key/value heads in
   groups ("gpt-oss 20B" field guide: 64 query heads, every group of eight
   sharing one key head and one value head; fixture comparison page:
   head_dim 64);
2. visible keys: all ``j < len_b`` for full attention, the last ``window``
   of them (``len_b - window <= j < len_b``) for local attention (field
   guide: local attention over the previous 128 tokens alternates with full
   causal attention);
3. ``w_j = exp(s_j) / (exp(sink_h) + sum_i exp(s_i))`` — the head's learned
   sink takes part in the normalisation but carries no value, so the weights
   of the real tokens may sum to less than one ("gpt-oss-20b and
   gpt-oss-120b" explainer, "Two attention savings, and a sink"; field guide
   cutaway 05);
4. ``out[b, h] = sum_j w_j v[b, g(h), j]``.

The pages give neither the score scale nor whether the local window counts
the query's own position: ``scale`` is an argument (the tests use 1/sqrt(D),
the usual one) and the window includes the query's position.

Parity status: pinned.  The explainer's worked example (three equal scores,
values 2, 6, 10: 6 without a sink, 4.5 with a sink of the same score), the
reduction to plain softmax attention as the sink goes to -inf (against
``scipy.special.softmax``), the sink's own weight filling the gap to one, the
output vanishing as the sink goes to +inf, a one-key window in closed form,
and the head grouping by a relabelling check.
"""
from __future__ import annotations

import numpy as np


def sink_softmax(s: np.ndarray, sink: float) -> np.ndarray:
    """Weights of scores ``s`` (last axis) with a sink logit in the
    normalisation: ``exp(s_j) / (exp(sink) + sum exp(s))``.  ``sink = -inf``
    gives the plain softmax."""
    s = np.asarray(s, dtype=np.float64)
    m = np.maximum(np.max(s, axis=-1, keepdims=True), sink)
    e = np.exp(s - m)
    return e / (np.exp(sink - m) + np.sum(e, axis=-1, keepdims=True))


def attn_sink_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, sinks: np.ndarray, lens: np.ndarray,
                     window: int, scale: float) -> np.ndarray:
    """Decode attention with sinks, float64.

    ``q`` ``[B, Hq, D]``; ``k``, ``v`` ``[B, Hkv, Tk, D]``; ``sinks`` ``[Hq]``;
    ``lens`` ``[B]`` (1 <= len <= Tk); ``window`` 0 for full attention.
    Returns ``[B, Hq, D]``."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must split evenly over key/value heads")
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        n = int(lens[b])
        lo = max(0, n - window) if window > 0 else 0
        for h in range(Hq):
            kv = h // G
            s = scale * (k[b, kv, lo:n] @ q[b, h])
            w = sink_softmax(s, float(sinks[h]))
            out[b, h] = w @ v[b, kv, lo:n]
    return out
