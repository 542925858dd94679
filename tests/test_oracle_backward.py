"""Pins of the fp64 gradient reference (``oracle.moe_backward``): central
finite differences of the forward oracle, the silent expansion carried to the
gradients ("gpt-oss-40b-64a8-init" page, section 2, Proof), and the frozen
experts of section 5.2.  CPU only."""
import numpy as np
import pytest

import oracle


def rand_layer(rng, T, H, I, E, scale=0.3):
    h = rng.standard_normal((T, H))
    wr = rng.standard_normal((E, H)) * 0.5
    br = rng.standard_normal(E) * 0.2
    ex = [[rng.standard_normal((I, H)) * scale, rng.standard_normal((I, H)) * scale,
           rng.standard_normal((H, I)) * scale] for _ in range(E)]
    return h, wr, br, ex


def loss(h, wr, br, ex, k, dout):
    w = oracle.LayerWeights(wr, br, lambda e: tuple(ex[e]))
    return float(np.sum(dout * oracle.moe_forward(h, w, k)["out"]))


def central(f, x, i, eps=1e-6):
    old = x[i]
    x[i] = old + eps
    fp = f()
    x[i] = old - eps
    fm = f()
    x[i] = old
    return (fp - fm) / (2 * eps)


@pytest.mark.parametrize("T,H,I,E,k,seed", [(6, 5, 7, 5, 2, 1), (4, 4, 6, 4, 4, 2), (5, 6, 4, 6, 1, 3)],
                         ids=["top2-of-5", "k-equals-E", "top1"])
def test_gradients_match_finite_differences(T, H, I, E, k, seed):
    """Every gradient entry against a central difference of sum(dout * out)
    taken on the forward oracle (selection margins kept far above the step)."""
    rng = np.random.default_rng(seed)
    h, wr, br, ex = rand_layer(rng, T, H, I, E)
    dout = rng.standard_normal((T, H))
    w = oracle.LayerWeights(wr, br, lambda e: tuple(ex[e]))
    assert np.all(oracle.topk_gap(oracle.router_logits(h, wr, br), k) > 1e-3)
    g = oracle.moe_backward(h, w, k, dout)
    f = lambda: loss(h, wr, br, ex, k, dout)
    tol = dict(rtol=1e-6, atol=1e-8)
    fd = np.array([central(f, h, i) for i in np.ndindex(h.shape)]).reshape(h.shape)
    np.testing.assert_allclose(g["dh"], fd, **tol)
    fd = np.array([central(f, wr, i) for i in np.ndindex(wr.shape)]).reshape(wr.shape)
    np.testing.assert_allclose(g["dw_router"], fd, **tol)
    fd = np.array([central(f, br, i) for i in np.ndindex(br.shape)])
    np.testing.assert_allclose(g["db_router"], fd, **tol)
    for e in range(E):
        for m, name in enumerate(("dw_gate", "dw_up", "dw_down")):
            x = ex[e][m]
            fd = np.array([central(f, x, i) for i in np.ndindex(x.shape)]).reshape(x.shape)
            np.testing.assert_allclose(g[name][e], fd, **tol, err_msg=f"{name}[{e}]")


def test_router_gradient_vanishes_for_k1_and_sums_to_zero():
    """With one expert selected p = 1 whatever the logit, so the router gets
    no gradient; for any k the logit gradients of a token sum to zero (the
    softmax is invariant to a shift of the selected logits)."""
    rng = np.random.default_rng(4)
    h, wr, br, ex = rand_layer(rng, 9, 6, 5, 6)
    dout = rng.standard_normal((9, 6))
    w = oracle.LayerWeights(wr, br, lambda e: tuple(ex[e]))
    g1 = oracle.moe_backward(h, w, 1, dout)
    assert np.all(g1["ds"] == 0) and np.all(g1["dw_router"] == 0) and np.all(g1["db_router"] == 0)
    g3 = oracle.moe_backward(h, w, 3, dout)
    np.testing.assert_allclose(g3["ds"].sum(axis=1), 0, atol=1e-14)
    assert np.abs(g3["ds"]).max() > 1e-3


@pytest.mark.parametrize("M", [2, 3])
def test_silent_expansion_splits_gradients_evenly(M):
    """After the M-fold expansion with k' = M k each copy carries p_i / M, so
    dh is unchanged and every copy of an expert (and of its router row) gets
    1/M of the original's gradient."""
    rng = np.random.default_rng(30 + M)
    T, H, I, E, k = 12, 6, 8, 5, 2
    h, wr, br, ex = rand_layer(rng, T, H, I, E)
    dout = rng.standard_normal((T, H))
    base = oracle.moe_backward(h, oracle.LayerWeights(wr, br, lambda e: tuple(ex[e])), k, dout)
    cmap = np.arange(M * E) % E
    wx = oracle.LayerWeights(oracle.expand_silent(wr, M), oracle.expand_silent(br, M), lambda j: tuple(ex[cmap[j]]))
    big = oracle.moe_backward(h, wx, M * k, dout)
    np.testing.assert_allclose(big["dh"], base["dh"], rtol=1e-12, atol=1e-13)
    for j in range(M * E):
        e = cmap[j]
        np.testing.assert_allclose(big["dw_router"][j], base["dw_router"][e] / M, rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(big["db_router"][j], base["db_router"][e] / M, rtol=1e-11, atol=1e-13)
        for name in ("dw_gate", "dw_up", "dw_down"):
            np.testing.assert_allclose(big[name][j], base[name][e] / M, rtol=1e-11, atol=1e-13)


def test_frozen_experts_are_left_out_and_change_nothing_else():
    """Section 5.2: the originals frozen, the copies trained; the router and
    dh are the same as with every expert trainable."""
    rng = np.random.default_rng(5)
    h, wr, br, ex = rand_layer(rng, 10, 6, 7, 8)
    dout = rng.standard_normal((10, 6))
    w = oracle.LayerWeights(wr, br, lambda e: tuple(ex[e]))
    full = oracle.moe_backward(h, w, 3, dout)
    mask = np.arange(8) >= 4
    part = oracle.moe_backward(h, w, 3, dout, trainable=mask)
    for name in ("dh", "dw_router", "db_router"):
        np.testing.assert_array_equal(part[name], full[name])
    for e in range(8):
        for name in ("dw_gate", "dw_up", "dw_down"):
            if mask[e]:
                np.testing.assert_array_equal(part[name][e], full[name][e])
            else:
                assert part[name][e] is None


def test_unselected_expert_gets_zero_gradient():
    rng = np.random.default_rng(6)
    h, wr, br, ex = rand_layer(rng, 3, 5, 6, 8)
    br[7] = -50.0  # never selected
    w = oracle.LayerWeights(wr, br, lambda e: tuple(ex[e]))
    g = oracle.moe_backward(h, w, 2, rng.standard_normal((3, 5)))
    assert not np.any(g["idx"] == 7)
    for name in ("dw_gate", "dw_up", "dw_down"):
        assert np.all(g[name][7] == 0)
    assert np.all(g["dw_router"][7] == 0) and g["db_router"][7] == 0
