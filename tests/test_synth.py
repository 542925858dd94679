"""The seeded input generator: determinism, formats and the workloads'
distributions and structure.  CPU only."""
import numpy as np
import pytest
import torch

import oracle
import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10 ** rng.uniform(-30, 30, 100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, 1.0 + 2 ** -8, -1.0 - 3 * 2 ** -9, 0.0, -0.0], np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_determinism_and_stream_independence():
    a = synth.make_layer(2, T=8)
    b = synth.make_layer(2, T=8)
    for n in ("h", "w_router", "b_router"):
        np.testing.assert_array_equal(getattr(a, n), getattr(b, n))
    e0, e0b, e1 = a.expert(0), b.expert(0), a.expert(1)
    np.testing.assert_array_equal(e0["gate"], e0b["gate"])
    assert not np.array_equal(e0["gate"], e1["gate"])
    assert not np.array_equal(e0["gate"], e0["up"])
    # a shorter T is a prefix of the full draw (decode = first rows of prefill)
    full = synth.make_layer(1)
    np.testing.assert_array_equal(synth.make_layer(1, T=16).h, full.h[:16])
    with pytest.raises(ValueError):
        synth.make_layer(1, T=65)


def test_stacked_equals_per_expert():
    L = synth.make_layer(1)
    st = L.stacked(threads=3)
    for e in range(L.E):
        for n, a in L.expert(e).items():
            np.testing.assert_array_equal(st[n][e], a)


@pytest.mark.parametrize("key", [2, 5])
def test_distributions(key):
    c = synth.CONFIGS[key]
    L = synth.make_layer(key, T=256)
    h = oracle.widen(L.h, c.act)
    assert h.shape == (256, c.H)
    assert abs(h.std() - 1.0) < 0.01 and abs(h.mean()) < 0.01
    wr = oracle.widen(L.w_router, c.act)
    assert wr.shape == (c.E, c.H) and abs(wr.std() / 0.02 - 1) < 0.02
    br = oracle.widen(L.b_router, c.act)
    assert br.shape == (c.E,) and abs(br.std() / 0.01 - 1) < 0.25
    w = L.expert(c.E - 1)
    if c.expert == "mxfp4":
        for n in ("gate", "up", "down"):
            d = oracle.mxfp4_dequant(w[n], w["s_" + n])
            assert d.shape == (2880, 2880)
            assert abs(d.std() / 0.02 - 1) < 0.05 and abs(d.mean()) < 1e-4
    else:
        g = oracle.widen(w["gate"], c.expert)
        assert g.shape == (c.I, c.H) and abs(g.std() / 0.02 - 1) < 0.01
        assert oracle.widen(w["down"], c.expert).shape == (c.H, c.I)


def test_fixture_shapes_and_zero_bias():
    c = synth.CONFIGS[1]
    assert (c.T, c.H, c.I, c.E, c.k, c.act, c.expert) == (64, 64, 128, 4, 2, "f32", "f32")
    L = synth.make_layer(1)
    assert L.h.dtype == np.float32 and not L.b_router.any()


def test_mxfp4_encoder_picks_the_spec_scale_and_nearest_codes():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    packed, scales = synth.mxfp4_encode(x)
    codes = np.empty((64, 512), np.uint8)
    codes[:, 0::2] = packed & 15
    codes[:, 1::2] = packed >> 4
    g = x.reshape(64, 16, 32)
    amax = np.abs(g).max(-1)
    # shared exponent floor(log2 amax) - 2: the group maximum lands in [4, 8)
    e = scales.astype(np.int64) - 127
    r = amax / 2.0 ** e
    assert ((r >= 4) & (r < 8)).all()
    # every element decodes to the nearest point of the scaled E2M1 grid
    d = oracle.mxfp4_dequant(packed, scales).reshape(64, 16, 32)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6])
    cand = grid[None, None, None, :] * (2.0 ** e)[..., None, None]
    dist = np.abs(cand - g[..., None].astype(np.float64)).min(-1)
    assert np.all(np.abs(d - g) <= dist + 1e-12)


def test_skewed_workload_hot_share():
    """Eight hot experts take about half of the T*k assignments."""
    L = synth.make_layer(4)
    assert len(L.hot_set) == 8
    h = oracle.widen(L.h, "bf16")
    s = oracle.router_logits(h, oracle.widen(L.w_router, "bf16"), oracle.widen(L.b_router, "bf16"))
    idx = oracle.select_topk(s, L.k)
    share = np.isin(idx, L.hot_set).mean()
    assert 0.49 <= share <= 0.51
    counts = np.bincount(idx.ravel(), minlength=L.E)
    assert counts.min() > 0                     # no empty expert
