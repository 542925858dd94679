"""Helpers shared by the GPU tests: put a seeded layer on the device, run the
library through its C interface, compute the fp64 reference, settle near-ties
and compare."""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle
import sparse_mixture_experts_token_amd as smoe
import synth

NEAR_TIE = 1e-5
DT = {"f32": smoe.MOE_F32, "bf16": smoe.MOE_BF16, "mxfp4": smoe.MOE_MXFP4}


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def to_dev(a: np.ndarray, fmt: str) -> torch.Tensor:
    if fmt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    if fmt == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def problem(cfg: synth.Config, T: int, E: int | None = None, k: int | None = None) -> smoe.Problem:
    return smoe.Problem(T, cfg.H, cfg.I, cfg.E if E is None else E, cfg.k if k is None else k,
                        DT[cfg.act], DT[cfg.expert])


def device_weights(layer: synth.Layer, stacked: dict) -> dict:
    c = layer.cfg
    w = {"w_router": to_dev(layer.w_router, c.act), "b_router": to_dev(layer.b_router, c.act)}
    for n in ("gate", "up", "down"):
        w["w_" + n] = to_dev(stacked[n], c.expert)
        if c.expert == "mxfp4":
            w["s_" + n] = to_dev(stacked["s_" + n], "u8")
    return w


def oracle_weights(layer: synth.Layer, stacked: dict) -> oracle.LayerWeights:
    c = layer.cfg
    return oracle.LayerWeights.from_storage(c.act, c.expert, layer.w_router, layer.b_router,
                                            lambda e: {n: a[e] for n, a in stacked.items()})


GUARD = 4096     # canary bytes before and after every buffer the library writes
CANARY = 0xA5
_guarded: list = []


def poisoned(shape, dtype, byte: int = 0xFF, device="cuda") -> torch.Tensor:
    """A tensor whose every byte is ``byte``: 0xFF reads as NaN in fp32 and
    bf16 and as -1 in int32, so a result the library fails to write, or a
    workspace region it reads before writing, shows up in the comparison.
    The tensor sits between two GUARD-byte runs of CANARY (its start stays
    16-byte aligned); ``check_canaries`` then shows any write just outside it."""
    n = int(np.prod(shape, dtype=np.int64)) * torch.empty((), dtype=dtype).element_size()
    raw = torch.empty(n + 2 * GUARD, dtype=torch.uint8, device=device)
    raw.fill_(CANARY)
    raw[GUARD:GUARD + n].fill_(byte)
    _guarded.append((raw, n))
    return raw[GUARD:GUARD + n].view(dtype).view(shape)


def check_canaries() -> None:
    """Every buffer made by ``poisoned`` since the last check still has its
    canary runs intact (call after the stream has been synchronized)."""
    try:
        for raw, n in _guarded:
            assert bool((raw[:GUARD] == CANARY).all()), "write before the start of a buffer"
            assert bool((raw[GUARD + n:] == CANARY).all()), "write past the end of a buffer"
    finally:
        _guarded.clear()


def routing_outputs(T: int, E: int, k: int, dev, byte: int = 0xFF) -> dict:
    return {"logits": poisoned((T, E), torch.float32, byte, dev),
            "topk_idx": poisoned((T, k), torch.int32, byte, dev),
            "topk_w": poisoned((T, k), torch.float32, byte, dev),
            "expert_offsets": poisoned((E + 1,), torch.int32, byte, dev),
            "perm_src": poisoned((T * k,), torch.int32, byte, dev)}


def run(prob: smoe.Problem, w: dict, h: torch.Tensor, act_fmt: str, byte: int = 0xFF) -> dict:
    """One forward pass with every routing output requested; results as numpy.
    The workspace, the output and the routing outputs are filled with
    ``byte`` first (0xFF: NaN), so stale or unwritten data cannot pass, and
    each is fenced by canary bytes that must survive the call."""
    T, E, k, H = prob.T, prob.E, prob.k, prob.H
    dev = h.device
    out = poisoned((T, H), h.dtype, byte, dev)
    r = routing_outputs(T, E, k, dev, byte)
    nb = smoe.moe_workspace_bytes(prob)
    ws = poisoned((max(nb, 1),), torch.uint8, byte, dev)
    smoe.moe_forward(prob, w, h, out, routing=r, workspace=ws, workspace_bytes=nb)
    torch.cuda.synchronize()
    check_canaries()
    res = {n: t.cpu().numpy() for n, t in r.items()}
    res["out"] = out.float().cpu().numpy().astype(np.float64)
    res["out_raw"] = out.cpu()
    return res


def reconcile(ref_idx: np.ndarray, s: np.ndarray, gap: np.ndarray, gpu_idx: np.ndarray, k: int):
    """Settle near-ties: tokens whose k-th and (k+1)-th reference logits differ
    by less than 1e-5 may pick either side.  Every other token must match
    exactly; a near-tie token's GPU set may differ only by experts within the
    band around the k-th logit.  Returns (selection to recompute with, count of
    near-tie tokens, count of near-tie tokens that differ)."""
    near = gap < NEAR_TIE
    differ = np.any(ref_idx != gpu_idx, axis=1)
    bad = np.nonzero(differ & ~near)[0]
    assert bad.size == 0, f"{bad.size} tokens select different experts (first: {bad[:5]})"
    eff = ref_idx.copy()
    kth = -np.sort(-s, axis=1)[:, k - 1]
    for t in np.nonzero(differ & near)[0]:
        g = gpu_idx[t]
        assert len(set(g.tolist())) == k and np.all(np.diff(g) > 0), f"token {t}: invalid GPU set {g}"
        for e in set(g.tolist()) ^ set(ref_idx[t].tolist()):
            assert abs(s[t, e] - kth[t]) < NEAR_TIE, f"token {t}: expert {e} is outside the tie band"
        eff[t] = g
    return eff, int(near.sum()), int((differ & near).sum())


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_out(got: np.ndarray, ref: np.ndarray, fmt: str) -> dict:
    r = rel_l2(got, ref)
    mx = float(np.abs(got - ref).max())
    lim = float(np.abs(ref).max())
    if fmt == "f32":
        assert r <= 1e-5, f"relative L2 {r:.3e} > 1e-5"
    else:
        assert r <= 5e-3, f"relative L2 {r:.3e} > 5e-3"
        assert mx <= 1e-2 * lim, f"max abs {mx:.3e} > 1e-2 * {lim:.3e}"
    return {"rel_l2": r, "max_abs": mx, "max_ref": lim}


_ref_cache: dict = {}


def reference_out(layer: synth.Layer, stacked: dict, T: int, idx: np.ndarray, tokens=None) -> np.ndarray:
    """fp64 outputs of the first ``T`` tokens of a workload with selection
    ``idx`` (cached: the full-size layers take tens of seconds)."""
    c = layer.cfg
    # keyed by the weights object too (each entry keeps it alive, so its id is not reused)
    key = (c, T, id(stacked), hash(idx.tobytes()), None if tokens is None else hash(np.asarray(tokens).tobytes()))
    if key not in _ref_cache:
        if len(_ref_cache) > 4:
            _ref_cache.clear()
        ow = oracle_weights(layer, stacked)
        h64 = oracle.widen(layer.h[:T], c.act)
        _ref_cache[key] = (stacked, oracle.moe_forward(h64, ow, c.k, idx=idx, tokens=tokens, workers=workers())["out"])
    return _ref_cache[key][1]


def check_layer(layer: synth.Layer, stacked: dict, w_dev: dict | None = None, tokens=None, T: int | None = None):
    """Full parity check of one layer: routing bit-exact (after near-ties),
    outputs within tolerance on ``tokens`` (default all)."""
    c = layer.cfg
    T = layer.T if T is None else T
    prob = problem(c, T)
    w_dev = device_weights(layer, stacked) if w_dev is None else w_dev
    h_dev = to_dev(layer.h[:T], c.act)
    g = run(prob, w_dev, h_dev, c.act)
    ow = oracle_weights(layer, stacked)
    h64 = oracle.widen(layer.h[:T], c.act)
    s = oracle.router_logits(h64, ow.w_router, ow.b_router)
    ref_idx = oracle.select_topk(s, c.k)
    gap = oracle.topk_gap(s, c.k)
    eff, n_near, n_swapped = reconcile(ref_idx, s, gap, g["topk_idx"].astype(np.int64), c.k)
    np.testing.assert_array_equal(g["topk_idx"], eff)
    md = oracle.routing_metadata(eff, c.E)
    np.testing.assert_array_equal(g["expert_offsets"], md["offsets"])
    np.testing.assert_array_equal(g["perm_src"], md["perm_src"])
    # fp32 logits and weights against fp64
    np.testing.assert_allclose(g["logits"], s, rtol=0, atol=1e-5 * max(1.0, np.abs(s).max()))
    p_ref = oracle.selected_softmax(s, eff)
    np.testing.assert_allclose(g["topk_w"], p_ref, rtol=0, atol=2e-6)
    ref_out = reference_out(layer, stacked, T, eff, tokens)
    got = g["out"] if tokens is None else g["out"][tokens]
    m = check_out(got, ref_out, c.act)
    m.update(n_near=n_near, n_swapped=n_swapped)
    return m, g
