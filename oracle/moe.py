"""fp64 reference of the sparse MoE feed-forward layer (forward pass).

TEST INFRASTRUCTURE ONLY (see the package header).

What it computes, per token ``t`` with input row ``h_t``:

1. router logits ``s_i = W_r[i].h_t + b_r[i]`` for every expert ``i``
   ("gpt-oss-40b-64a8-init" page, section 2, Proof);
2. the selected set ``S_t``: the ``k`` largest logits ("top-k(s)", same
   Proof; "selects the top four", "gpt-oss 20B" field guide, cutaway 03).
   The pages do not say how ties are broken: the lower expert index wins, and
   ``S_t`` is reported in ascending expert id;
3. ``p_i = exp(s_i) / sum_{j in S_t} exp(s_j)`` for ``i in S_t`` — softmax over
   the selected set only (Proof; the field guide's "normalizes those selected
   scores").  The maximum over ``S_t`` is subtracted first, which changes
   nothing mathematically;
4. each selected expert is a SwiGLU network
   ``E_i(x) = W_down[i] (silu(W_gate[i] x) * (W_up[i] x))`` with
   ``silu(z) = z / (1 + exp(-z))`` (field guide, cutaway 03 "SwiGLU experts";
   fixture comparison page, ``hidden_act = silu``).  No expert biases, clamps
   or extra scale factors: the pages name none;
5. ``out_t = sum_{i in S_t} p_i E_i(h_t)`` (Proof, first formula).

Plus the routing metadata that the GPU path exposes (per-expert counts,
their exclusive prefix sums, and the expert-major permutation whose rows are
ordered by token within each expert), and the silent expansion ``X'[j] =
X[j mod E]`` of the Proof / section 5.2.

Two independent evaluations of the layer are given: ``moe_forward`` groups the
work per expert (gather the expert's rows, three matrix products), and
``moe_forward_per_token`` walks each token's selected set with matrix-vector
products and an iterative arg-max selection.  Tests require them to agree.

Parity status: pinned.  Selection by brute force over all C(E, k) subsets;
weights by closed forms (sum to one, k = 1, equal logits); the whole layer by
the two evaluations agreeing, the k = E dense-mixture reduction, the k = 1
single-expert reduction, identical-expert and zero-down special cases,
relabelling invariance, a hand-computed one-unit example, and the silent-init
identity for M = 2, 3.  Absolute outputs at full size have no printed worked
example on the pages; they rest on those pins.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable

import numpy as np

from .mxfp4 import mxfp4_dequant


# ---------------------------------------------------------------- inputs --

def widen(x, fmt: str) -> np.ndarray:
    """Exact float64 view of a stored tensor: ``fmt`` is "f32" (float32 array)
    or "bf16" (raw uint16 bits: the high half of an IEEE float32)."""
    if fmt == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if fmt == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown format {fmt!r}")


@dataclass
class LayerWeights:
    """fp64 parameters of one layer.  ``expert(e)`` returns the float64
    ``(W_gate [I,H], W_up [I,H], W_down [H,I])`` of expert ``e``; it is called
    once per needed expert so that large layers stream through memory."""
    w_router: np.ndarray            # [E, H]
    b_router: np.ndarray            # [E]
    expert: Callable[[int], tuple]

    @property
    def E(self) -> int:
        return self.w_router.shape[0]

    @staticmethod
    def from_storage(act_fmt: str, expert_fmt: str, w_router, b_router, expert_source):
        """``expert_source(e)`` returns the stored tensors of expert ``e``:
        ``gate``, ``up``, ``down`` (and ``s_gate``, ``s_up``, ``s_down`` for MXFP4)."""
        def expert(e):
            w = expert_source(e)
            if expert_fmt == "mxfp4":
                return tuple(mxfp4_dequant(w[n], w["s_" + n]) for n in ("gate", "up", "down"))
            return tuple(widen(w[n], expert_fmt) for n in ("gate", "up", "down"))
        return LayerWeights(widen(w_router, act_fmt), widen(b_router, act_fmt), expert)


# ------------------------------------------------------------ the router --

def router_logits(h: np.ndarray, w_router: np.ndarray, b_router: np.ndarray) -> np.ndarray:
    """``s[t, i] = W_r[i] . h[t] + b_r[i]`` (Proof: router logits)."""
    return h @ w_router.T + b_router[None, :]


def select_topk(s: np.ndarray, k: int) -> np.ndarray:
    """Indices of the ``k`` largest logits per row, ascending expert id.
    Order by (-logit, index): equal logits go to the lower index."""
    order = np.argsort(-s, axis=1, kind="stable")
    return np.sort(order[:, :k], axis=1)


def topk_gap(s: np.ndarray, k: int) -> np.ndarray:
    """``s_(k) - s_(k+1)`` per row (the margin of the selection boundary);
    +inf when every expert is selected."""
    E = s.shape[1]
    if k >= E:
        return np.full(s.shape[0], np.inf)
    srt = -np.sort(-s, axis=1)
    return srt[:, k - 1] - srt[:, k]


def selected_softmax(s: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """``p_i = exp(s_i) / sum_{j in S} exp(s_j)`` over the selected set (Proof)."""
    sel = np.take_along_axis(s, idx, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


# ------------------------------------------------------------ the experts --

def silu(z: np.ndarray) -> np.ndarray:
    """``silu(z) = z * sigmoid(z) = z / (1 + exp(-z))``."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """One SwiGLU expert on rows ``x [n, H]``: ``(silu(x W_g^T) * (x W_u^T)) W_d^T``."""
    g = x @ w_gate.T
    u = x @ w_up.T
    return (silu(g) * u) @ w_down.T


# ------------------------------------------------------------- the layer --

def moe_forward(h: np.ndarray, weights: LayerWeights, k: int, idx: np.ndarray | None = None,
                tokens: np.ndarray | None = None, workers: int = 1) -> dict:
    """The layer, evaluated expert by expert.

    ``h`` is float64 ``[T, H]``.  Routing (logits, selection, weights) is done
    for every token; outputs are formed for ``tokens`` (default: all).
    ``idx`` replaces the selection (it must be a valid top-k set per token; the
    parity check passes one only to settle near-ties).  ``workers > 1``
    evaluates experts on that many threads; their contributions are still
    added in ascending expert order.

    Returns ``out`` (``[len(tokens), H]``), ``s``, ``idx``, ``p``, ``gap``.
    """
    s = router_logits(h, weights.w_router, weights.b_router)
    E = s.shape[1]
    if not 1 <= k <= E:
        raise ValueError(f"k={k} outside 1..{E}")
    if idx is None:
        idx = select_topk(s, k)
    p = selected_softmax(s, idx)
    gap = topk_gap(s, k)
    if tokens is None:
        tokens = np.arange(h.shape[0])
    tokens = np.asarray(tokens)
    sub_idx = idx[tokens]
    sub_p = p[tokens]
    out = np.zeros((len(tokens), h.shape[1]))

    def contribution(e):
        rows, slots = np.nonzero(sub_idx == e)
        if rows.size == 0:
            return rows, None
        wg, wu, wd = weights.expert(e)
        y = swiglu_expert(h[tokens[rows]], wg, wu, wd)
        return rows, sub_p[rows, slots][:, None] * y

    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            parts = ex.map(contribution, range(E))
            for rows, c in parts:
                if c is not None:
                    np.add.at(out, rows, c)
    else:
        for e in range(E):
            rows, c = contribution(e)
            if c is not None:
                np.add.at(out, rows, c)
    return {"out": out, "s": s, "idx": idx, "p": p, "gap": gap}


def moe_forward_per_token(h: np.ndarray, weights: LayerWeights, k: int) -> dict:
    """The same layer, token by token: logits by one dot product per expert,
    the selected set by taking the arg-max ``k`` times (``np.argmax`` keeps the
    first, i.e. lowest-index, maximum), then a matrix-vector pass through each
    selected expert.  Independent of ``moe_forward``; meant for small inputs."""
    T, H = h.shape
    E = weights.E
    cache = {}

    def expert(e):
        if e not in cache:
            cache[e] = weights.expert(e)
        return cache[e]

    out = np.zeros((T, H))
    idx = np.zeros((T, k), dtype=np.int64)
    p = np.zeros((T, k))
    for t in range(T):
        logits = np.array([np.dot(weights.w_router[e], h[t]) + weights.b_router[e] for e in range(E)])
        remaining = logits.copy()
        chosen = []
        for _ in range(k):
            j = int(np.argmax(remaining))
            chosen.append(j)
            remaining[j] = -np.inf
        chosen.sort()
        top = max(logits[j] for j in chosen)
        num = [np.exp(logits[j] - top) for j in chosen]
        den = sum(num)
        acc = np.zeros(H)
        for slot, j in enumerate(chosen):
            wg, wu, wd = expert(j)
            g = wg @ h[t]
            u = wu @ h[t]
            a = (g / (1.0 + np.exp(-g))) * u
            acc += (num[slot] / den) * (wd @ a)
            idx[t, slot] = j
            p[t, slot] = num[slot] / den
        out[t] = acc
    return {"out": out, "idx": idx, "p": p}


# -------------------------------------------------- routing metadata ------

def routing_metadata(idx: np.ndarray, E: int) -> dict:
    """Expert-major view of the assignments.

    Assignment ``a = t*k + slot`` sends token ``t`` to expert ``idx[t, slot]``.
    ``counts[e]`` = number of assignments to ``e``; ``offsets`` = exclusive
    prefix sum (``offsets[E] = T*k``); ``perm_src[r]`` = the assignment at row
    ``r`` of the expert-major order, rows of one expert ordered by token;
    ``inv`` its inverse (assignment -> row)."""
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    perm_src = np.argsort(flat, kind="stable")
    inv = np.empty_like(perm_src)
    inv[perm_src] = np.arange(flat.size)
    return {"counts": counts, "offsets": offsets, "perm_src": perm_src, "inv": inv}


# ------------------------------------------------------ silent expansion --

def expand_rows(x: np.ndarray, copy_of) -> np.ndarray:
    """Expanded per-expert tensor (expert axis first) in which expanded expert
    ``j`` is a copy of original expert ``copy_of[j]``: the silent-init
    construction ("gpt-oss-40b-64a8-init" page, section 2: every new expert is
    initialised from an existing one, router row included) with any number of
    copies per original, e.g. the 248 expert rows of "gpt-oss-220a20b" (Model
    Details: 128 base rows plus 120 added rows)."""
    x = np.asarray(x)
    copy_of = np.asarray(copy_of)
    if copy_of.ndim != 1 or copy_of.size == 0:
        raise ValueError("copy_of must be a non-empty list of original expert ids")
    if copy_of.min() < 0 or copy_of.max() >= x.shape[0]:
        raise ValueError("copy_of names an expert that does not exist")
    return x[copy_of]


def expand_silent(x: np.ndarray, M: int, copy_of: np.ndarray | None = None) -> np.ndarray:
    """Expand a per-expert tensor (expert axis first) to ``M*E`` experts.

    Default mapping: expanded expert ``j`` copies original ``j mod E``, i.e.
    originals keep indices ``0..E-1`` and the copies follow
    ("gpt-oss-40b-64a8-init" page, section 2 Principle; section 5.2 on the
    original indices 0-31 and the expanded 32-63).  ``copy_of`` gives any other
    mapping (each original must appear exactly ``M`` times for the identity)."""
    x = np.asarray(x)
    E = x.shape[0]
    if M < 1:
        raise ValueError("M must be >= 1")
    if copy_of is None:
        copy_of = np.arange(M * E) % E
    copy_of = np.asarray(copy_of)
    if copy_of.shape != (M * E,):
        raise ValueError("copy_of must map every expanded expert")
    return x[copy_of]
