"""Parity of the layer's gradients (``moe_backward``) with the fp64
reference ``oracle.moe_backward``: d_h, the router's and every trainable
expert's gradients within relative L2 5e-3 and max abs 1e-2*max|ref| (bf16
products), on seeded layers with ragged expert row counts, empty experts,
k = E, and the gpt-oss-20b expert shape; frozen experts' slices untouched;
run-to-run bitwise equal."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_token_amd as smoe
import synth
from gpu_util import check_out, device_weights, oracle_weights, reconcile, to_dev

# The first GPU run of these tests ended in a GPU memory fault whose cause has
# not been found (the kernels' index arithmetic checks out on the CPU); the
# entry point is switched off (MOE_ERR_DISABLED) until it is.
pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="moe_backward switched off: unexplained GPU memory fault "
                                                       "on its first run; cause not yet found")]

GRADS = ("d_w_router", "d_b_router", "d_w_gate", "d_w_up", "d_w_down")


def forward_routing(prob, w, h):
    T, E, k = prob.T, prob.E, prob.k
    r = {"logits": torch.empty((T, E), dtype=torch.float32, device="cuda"),
         "topk_idx": torch.empty((T, k), dtype=torch.int32, device="cuda"),
         "topk_w": torch.empty((T, k), dtype=torch.float32, device="cuda"),
         "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device="cuda"),
         "perm_src": torch.empty(T * k, dtype=torch.int32, device="cuda")}
    out = torch.empty((T, prob.H), dtype=torch.bfloat16, device="cuda")
    smoe.moe_forward(prob, w, h, out, routing=r)
    return r


def alloc_grads(prob, fill=0.0):
    E, H, I = prob.E, prob.H, prob.I
    shapes = {"d_w_router": (E, H), "d_b_router": (E,), "d_w_gate": (E, I, H), "d_w_up": (E, I, H),
              "d_w_down": (E, H, I)}
    return {n: torch.full(s, fill, dtype=torch.float32, device="cuda") for n, s in shapes.items()}


def run_backward(L, st, seed, trainable=None, fill=0.0):
    c = L.cfg
    prob = smoe.Problem(L.T, c.H, c.I, c.E, c.k, smoe.MOE_BF16, smoe.MOE_BF16)
    w = device_weights(L, st)
    h = to_dev(L.h, "bf16")
    dout_bits = synth.grad_output(seed, L.T, c.H)
    r = forward_routing(prob, w, h)
    dh = torch.empty((L.T, c.H), dtype=torch.bfloat16, device="cuda")
    g = alloc_grads(prob, fill)
    tr = None if trainable is None else torch.from_numpy(trainable.astype(np.uint8)).cuda()
    smoe.moe_backward(prob, w, h, to_dev(dout_bits, "bf16"), {n: r[n] for n in
                      ("topk_idx", "topk_w", "expert_offsets", "perm_src")}, d_h=dh, grads=g, trainable=tr)
    torch.cuda.synchronize()
    return prob, w, h, dout_bits, r, dh, g


def reference(L, st, dout_bits, r, trainable=None):
    c = L.cfg
    ow = oracle_weights(L, st)
    h64 = oracle.widen(L.h, "bf16")
    s = oracle.router_logits(h64, ow.w_router, ow.b_router)
    eff, _, _ = reconcile(oracle.select_topk(s, c.k), s, oracle.topk_gap(s, c.k),
                          r["topk_idx"].cpu().numpy().astype(np.int64), c.k)
    return oracle.moe_backward(h64, ow, c.k, oracle.widen(dout_bits, "bf16"), idx=eff, trainable=trainable)


def compare(dh, g, ref, experts):
    m = {"dh": check_out(dh.float().cpu().numpy().astype(np.float64), ref["dh"], "bf16")}
    m["dw_router"] = check_out(g["d_w_router"].cpu().numpy().astype(np.float64), ref["dw_router"], "bf16")
    m["db_router"] = check_out(g["d_b_router"].cpu().numpy().astype(np.float64), ref["db_router"], "bf16")
    for e in experts:
        for n, rn in (("d_w_gate", "dw_gate"), ("d_w_up", "dw_up"), ("d_w_down", "dw_down")):
            got = g[n][e].cpu().numpy().astype(np.float64)
            if not np.any(ref[rn][e]):
                assert not np.any(got), f"{n}[{e}] should be zero (expert not selected)"
            else:
                m[f"{rn}[{e}]"] = check_out(got, ref[rn][e], "bf16")
    return m


CASES = [
    synth.Config(201, "ragged-7e-top3", T=333, H=128, I=192, E=7, k=3, act="bf16", expert="bf16"),
    synth.Config(202, "many-tiles-per-expert", T=1500, H=64, I=128, E=3, k=2, act="bf16", expert="bf16"),
    synth.Config(203, "k-equals-E", T=50, H=64, I=128, E=6, k=6, act="bf16", expert="bf16"),
    synth.Config(204, "mostly-empty-experts", T=3, H=128, I=128, E=64, k=2, act="bf16", expert="bf16"),
    synth.Config(205, "wide-I-narrow-H", T=200, H=64, I=640, E=5, k=2, act="bf16", expert="bf16"),
]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_backward_parity_small(cfg):
    L = synth.make_layer(cfg)
    st = L.stacked()
    prob, w, h, dout_bits, r, dh, g = run_backward(L, st, cfg.cid)
    ref = reference(L, st, dout_bits, r)
    m = compare(dh, g, ref, range(cfg.E))
    print({k: round(v["rel_l2"], 6) for k, v in m.items()})


def test_backward_gpt_oss_20b_shape_sampled_experts():
    """H = I = 2880, 32 experts, top-4, 256 tokens (about 32 rows per
    expert): every d_h and router entry, the expert gradients of 4 sampled
    experts (the oracle computes only those)."""
    cfg = synth.Config(206, "gpt-oss-20b-256", T=256, H=2880, I=2880, E=32, k=4, act="bf16", expert="bf16")
    L = synth.make_layer(cfg)
    st = L.stacked()
    prob, w, h, dout_bits, r, dh, g = run_backward(L, st, cfg.cid)
    sample = np.zeros(32, dtype=bool)
    sample[[0, 9, 17, 31]] = True
    ref = reference(L, st, dout_bits, r, trainable=sample)
    m = compare(dh, g, ref, np.nonzero(sample)[0])
    print({k: round(v["rel_l2"], 6) for k, v in m.items()})


def test_frozen_experts_untouched_and_rest_bitwise_equal():
    """Section 5.2's split (originals frozen, copies trained): frozen slices
    keep what the caller put there; everything else is bit-identical to the
    all-trainable run, which itself repeats bit for bit."""
    cfg = CASES[0]
    L = synth.make_layer(cfg)
    st = L.stacked()
    mask = np.arange(cfg.E) >= 3
    _, _, _, _, _, dh_a, g_a = run_backward(L, st, cfg.cid)
    _, _, _, _, _, dh_b, g_b = run_backward(L, st, cfg.cid)
    _, _, _, _, _, dh_f, g_f = run_backward(L, st, cfg.cid, trainable=mask, fill=7.0)
    assert torch.equal(dh_a, dh_b) and torch.equal(dh_a, dh_f)
    for n in GRADS:
        assert torch.equal(g_a[n], g_b[n]), n
    for n in ("d_w_router", "d_b_router"):
        assert torch.equal(g_a[n], g_f[n]), n
    for n in ("d_w_gate", "d_w_up", "d_w_down"):
        for e in range(cfg.E):
            if mask[e]:
                assert torch.equal(g_f[n][e], g_a[n][e]), (n, e)
            else:
                assert torch.all(g_f[n][e] == 7.0), (n, e)


def test_silent_expansion_splits_gradients_on_the_gpu():
    """The 2-fold silent expansion at k' = 2k: d_h matches the base layer's
    and each copy's gradients are half the base expert's (same bf16 products,
    so within the bf16 tolerance of each other)."""
    cfg = synth.Config(207, "expand-base", T=300, H=128, I=192, E=6, k=2, act="bf16", expert="bf16")
    L = synth.make_layer(cfg)
    st = L.stacked()
    prob, w, h, dout_bits, r, dh, g = run_backward(L, st, cfg.cid)
    M, E = 2, cfg.E
    pb = smoe.Problem(L.T, cfg.H, cfg.I, M * E, M * cfg.k, smoe.MOE_BF16, smoe.MOE_BF16)
    wx = {n: torch.cat([t] * M, dim=0).contiguous() for n, t in w.items()}
    rx = forward_routing(pb, wx, h)
    dhx = torch.empty_like(dh)
    gx = alloc_grads(pb)
    smoe.moe_backward(pb, wx, h, to_dev(dout_bits, "bf16"), {n: rx[n] for n in
                      ("topk_idx", "topk_w", "expert_offsets", "perm_src")}, d_h=dhx, grads=gx)
    torch.cuda.synchronize()
    check_out(dhx.float().cpu().numpy().astype(np.float64), dh.float().cpu().numpy().astype(np.float64), "bf16")
    for n in GRADS:
        base = g[n].cpu().numpy().astype(np.float64)
        for c in range(M):
            got = gx[n][c * E:(c + 1) * E].cpu().numpy().astype(np.float64) * M
            check_out(got, base, "bf16")
