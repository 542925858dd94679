"""Pins of the fp64 reference (``oracle/``) against what the pages and the
mathematics fix: brute force, closed forms, special cases, the silent-init
identity, a hand-computed example and the numbers the pages print.  CPU only."""
import itertools
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLD, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]


def rand_layer(rng, T, H, I, E, scale=0.15):
    h = rng.standard_normal((T, H))
    wr = rng.standard_normal((E, H)) * 0.3
    br = rng.standard_normal(E) * 0.1
    ex = [(rng.standard_normal((I, H)) * scale, rng.standard_normal((I, H)) * scale,
           rng.standard_normal((H, I)) * scale) for _ in range(E)]
    return h, oracle.LayerWeights(wr, br, lambda e: ex[e]), ex


def all_expert_outputs(h, ex):
    """Every expert applied to every token, by explicit per-token matrix-vector products."""
    T = h.shape[0]
    out = np.zeros((len(ex), T, h.shape[1]))
    for e, (wg, wu, wd) in enumerate(ex):
        for t in range(T):
            g = wg @ h[t]
            u = wu @ h[t]
            out[e, t] = wd @ (g * u / (1.0 + np.exp(-g)))
    return out


# ------------------------------------------------------------ selection --

@pytest.mark.parametrize("E", [4, 5, 6, 8, 10, 12])
def test_topk_matches_bruteforce_over_all_subsets(E):
    rng = np.random.default_rng(E)
    s = rng.standard_normal((16, E))
    for k in range(1, E + 1):
        combos = np.array(list(itertools.combinations(range(E), k)))
        assert len(combos) == math.comb(E, k)
        sums = s[:, combos].sum(-1)                     # [T, C(E,k)]
        best = combos[np.argmax(sums, axis=1)]          # the unique top-k set
        np.testing.assert_array_equal(oracle.select_topk(s, k), best)
        if k < E:
            # the margin of the boundary: weakest selected minus strongest unselected
            sel = np.zeros_like(s, dtype=bool)
            np.put_along_axis(sel, best, True, axis=1)
            margin = np.where(sel, s, np.inf).min(1) - np.where(sel, -np.inf, s).max(1)
            np.testing.assert_allclose(oracle.topk_gap(s, k), margin, rtol=0, atol=0)


@pytest.mark.parametrize("E", [4, 6, 9])
def test_topk_ties_go_to_lower_index(E):
    # integer logits: many exact ties.  Among the subsets of maximal sum, the
    # lowest-index choice is the lexicographically first one.
    rng = np.random.default_rng(100 + E)
    s = rng.integers(0, 3, size=(40, E)).astype(np.float64)
    for k in range(1, E + 1):
        combos = np.array(list(itertools.combinations(range(E), k)))  # lexicographic
        sums = s[:, combos].sum(-1)
        best = combos[np.argmax(sums, axis=1)]          # first maximum
        np.testing.assert_array_equal(oracle.select_topk(s, k), best)
    # silent copies tie exactly: both copies of the best expert are chosen
    s2 = np.array([[0.3, 1.2, -0.5, 0.3, 1.2, -0.5]])
    np.testing.assert_array_equal(oracle.select_topk(s2, 2), [[1, 4]])
    np.testing.assert_array_equal(oracle.select_topk(s2, 1), [[1]])


# -------------------------------------------------------------- weights --

def test_selected_softmax_closed_forms():
    rng = np.random.default_rng(1)
    s = rng.standard_normal((50, 12)) * 3
    for k in (1, 2, 5, 12):
        idx = oracle.select_topk(s, k)
        p = oracle.selected_softmax(s, idx)
        np.testing.assert_allclose(p.sum(1), 1.0, rtol=0, atol=1e-14)
        assert (p > 0).all()
        sel = np.take_along_axis(s, idx, 1)
        # defining ratio: p_i / p_j = exp(s_i - s_j)
        np.testing.assert_allclose(p[:, :, None] / p[:, None, :],
                                   np.exp(sel[:, :, None] - sel[:, None, :]), rtol=1e-12)
        if k == 1:
            np.testing.assert_array_equal(p, 1.0)
        # adding a constant to every logit changes nothing
        np.testing.assert_allclose(oracle.selected_softmax(s + 7.5, idx), p, rtol=1e-12)
    eq = np.full((3, 8), 0.7)
    for k in (1, 3, 8):
        np.testing.assert_allclose(oracle.selected_softmax(eq, oracle.select_topk(eq, k)), 1.0 / k, rtol=1e-15)


def test_softmax_is_over_selected_set_only():
    # full-softmax weights of the selected experts do NOT sum to one; the
    # layer's weights are those renormalised over the selected set
    s = np.array([[2.0, 1.0, 0.0, -1.0]])
    idx = oracle.select_topk(s, 2)
    full = np.exp(s) / np.exp(s).sum()
    p = oracle.selected_softmax(s, idx)
    np.testing.assert_allclose(p[0], full[0, :2] / full[0, :2].sum(), rtol=1e-15)
    assert abs(full[0, :2].sum() - 1.0) > 0.1


# ----------------------------------------------------------- activation --

def test_silu_special_values():
    L = math.log(3.0)
    np.testing.assert_allclose(oracle.silu(np.array([0.0, L, -L])), [0.0, 0.75 * L, -0.25 * L], rtol=1e-15, atol=0)
    x = np.linspace(-20, 20, 401)
    np.testing.assert_allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=1e-13, atol=1e-13)
    assert abs(oracle.silu(np.array([60.0]))[0] - 60.0) < 1e-20
    assert abs(oracle.silu(np.array([-800.0]))[0]) == 0.0


# ---------------------------------------------------------- whole layer --

def _hand_layer():
    wr = np.array([[1.0, 0.0], [0.0, 1.0]])
    br = np.zeros(2)
    ex = [
        (np.array([[1.0, 0], [0, 1], [2, 0]]), np.array([[1.0, 0], [1, 0], [0, 1]]), np.array([[1.0, 5, 7], [2, 0, 1]])),
        (np.array([[0.0, 0], [1, 0], [0, 0]]), np.array([[0.0, 0], [2, 0], [0, 0]]), np.array([[0.0, 1, 0], [0, -1, 3]])),
    ]
    return oracle.LayerWeights(wr, br, lambda e: ex[e])


def test_hand_computed_unit_example():
    L = math.log(3.0)
    h = np.array([[L, 0.0]])
    w = _hand_layer()
    for k, o0, o1 in _rows("swiglu_unit.txt"):
        k = int(k)
        want = np.array([float(o0), float(o1)]) * L * L
        got = oracle.moe_forward(h, w, k)["out"][0]
        np.testing.assert_allclose(got, want, rtol=1e-14)
        got2 = oracle.moe_forward_per_token(h, w, k)["out"][0]
        np.testing.assert_allclose(got2, want, rtol=1e-14)


def test_two_evaluations_agree_random_layer():
    rng = np.random.default_rng(7)
    h, w, _ = rand_layer(rng, T=40, H=48, I=80, E=12, scale=0.2)
    for k in (1, 3, 7, 12):
        a = oracle.moe_forward(h, w, k)
        b = oracle.moe_forward_per_token(h, w, k)
        np.testing.assert_array_equal(a["idx"], b["idx"])
        np.testing.assert_allclose(a["p"], b["p"], rtol=1e-13)
        np.testing.assert_allclose(a["out"], b["out"], rtol=1e-12, atol=1e-14)


def test_two_evaluations_agree_fixture():
    L = synth.make_layer(1)
    w = oracle.LayerWeights.from_storage("f32", "f32", L.w_router, L.b_router, L.expert)
    h = oracle.widen(L.h, "f32")
    a = oracle.moe_forward(h, w, L.k)
    b = oracle.moe_forward_per_token(h, w, L.k)
    np.testing.assert_array_equal(a["idx"], b["idx"])
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-12, atol=1e-15)
    # sampled tokens give the same rows as the full evaluation
    tok = np.array([63, 0, 17, 17])
    np.testing.assert_allclose(oracle.moe_forward(h, w, L.k, tokens=tok)["out"], a["out"][tok], rtol=1e-12, atol=1e-16)


def test_k_equals_E_is_the_dense_softmax_mixture():
    rng = np.random.default_rng(8)
    h, w, ex = rand_layer(rng, T=10, H=16, I=24, E=6)
    s = h @ w.w_router.T + w.b_router
    full = np.exp(s) / np.exp(s).sum(1, keepdims=True)
    dense = np.einsum("te,eth->th", full, all_expert_outputs(h, ex))
    np.testing.assert_allclose(oracle.moe_forward(h, w, 6)["out"], dense, rtol=1e-12, atol=1e-15)


def test_k1_is_the_argmax_expert():
    rng = np.random.default_rng(9)
    h, w, ex = rand_layer(rng, T=20, H=16, I=24, E=5)
    s = h @ w.w_router.T + w.b_router
    y = all_expert_outputs(h, ex)
    want = y[np.argmax(s, 1), np.arange(20)]
    np.testing.assert_allclose(oracle.moe_forward(h, w, 1)["out"], want, rtol=1e-12, atol=1e-15)


def test_identical_experts_give_that_expert_for_any_routing():
    rng = np.random.default_rng(10)
    h, w, ex = rand_layer(rng, T=12, H=16, I=24, E=7)
    same = oracle.LayerWeights(w.w_router, w.b_router, lambda e: ex[0])
    y0 = all_expert_outputs(h, ex[:1])[0]
    for k in (1, 3, 7):
        np.testing.assert_allclose(oracle.moe_forward(h, same, k)["out"], y0, rtol=1e-12, atol=1e-15)


def test_zero_down_projection_gives_zero():
    rng = np.random.default_rng(11)
    h, w, ex = rand_layer(rng, T=6, H=8, I=12, E=4)
    zero = oracle.LayerWeights(w.w_router, w.b_router, lambda e: (ex[e][0], ex[e][1], np.zeros_like(ex[e][2])))
    assert not oracle.moe_forward(h, zero, 2)["out"].any()


def test_relabelling_experts_changes_only_the_labels():
    rng = np.random.default_rng(12)
    h, w, ex = rand_layer(rng, T=30, H=16, I=24, E=9)
    perm = rng.permutation(9)                 # new expert j is old expert perm[j]
    w2 = oracle.LayerWeights(w.w_router[perm], w.b_router[perm], lambda j: ex[perm[j]])
    inv = np.argsort(perm)
    for k in (2, 4):
        a = oracle.moe_forward(h, w, k)
        b = oracle.moe_forward(h, w2, k)
        np.testing.assert_allclose(b["out"], a["out"], rtol=1e-12, atol=1e-15)
        np.testing.assert_array_equal(np.sort(inv[a["idx"]], 1), b["idx"])


# ----------------------------------------------------- silent expansion --

def _expanded(w, ex, M, copy_of=None):
    E = len(ex)
    cmap = np.arange(M * E) % E if copy_of is None else np.asarray(copy_of)
    wr = oracle.expand_silent(w.w_router, M, cmap)
    br = oracle.expand_silent(w.b_router, M, cmap)
    return oracle.LayerWeights(wr, br, lambda j: ex[cmap[j]])


@pytest.mark.parametrize("M", [2, 3])
def test_silent_init_identity(M):
    """Expanding every expert and router row M times with k' = M*k reproduces
    the layer ("gpt-oss-40b-64a8-init" page, section 2, Proof)."""
    rng = np.random.default_rng(20 + M)
    h, w, ex = rand_layer(rng, T=60, H=24, I=40, E=8)
    rand_map = np.concatenate([rng.permutation(8) for _ in range(M)])
    rng.shuffle(rand_map)
    for k in (1, 2, 4):
        base = oracle.moe_forward(h, w, k)
        for cmap in (None, rand_map):
            wx = _expanded(w, ex, M, cmap)
            big = oracle.moe_forward(h, wx, M * k)
            np.testing.assert_allclose(big["out"], base["out"], rtol=1e-12, atol=1e-14)
            # the selected set is the M copies of each original choice
            m = np.arange(M * 8) % 8 if cmap is None else cmap
            np.testing.assert_array_equal(np.sort(m[big["idx"]], 1), np.repeat(base["idx"], M, axis=1))
        # the same proof with k' = M*j for j < k: equals the base layer at top-j
        if k > 1:
            j = k - 1
            np.testing.assert_allclose(oracle.moe_forward(h, _expanded(w, ex, M), M * j)["out"],
                                       oracle.moe_forward(h, w, j)["out"], rtol=1e-12, atol=1e-14)


def test_expansion_with_k_not_a_multiple_of_M():
    """Three copies of every expert, k' = 4: the selection is the three copies
    of the best expert and the lowest copy of the second (exact ties go to the
    lower index), so the layer is the closed form
    (3 e1 y1 + e2 y2) / (3 e1 + e2), e_i = exp(s_i - s_1), y_i = expert i's output."""
    rng = np.random.default_rng(41)
    E, M = 8, 3
    h, w, ex = rand_layer(rng, T=40, H=24, I=40, E=E)
    big = oracle.moe_forward(h, _expanded(w, ex, M), 4)
    s = h @ w.w_router.T + w.b_router
    order = np.argsort(-s, axis=1, kind="stable")
    for t in range(len(h)):
        b1, b2 = order[t, 0], order[t, 1]
        np.testing.assert_array_equal(big["idx"][t], sorted([b1, b1 + E, b1 + 2 * E, b2]))
        ys = []
        for b in (b1, b2):
            wg, wu, wd = ex[b]
            g, u = wg @ h[t], wu @ h[t]
            ys.append(wd @ (g / (1 + np.exp(-g)) * u))
        e2 = np.exp(s[t, b2] - s[t, b1])
        want = (3 * ys[0] + e2 * ys[1]) / (3 + e2)
        np.testing.assert_allclose(big["out"][t], want, rtol=1e-12, atol=1e-15)


def test_silent_identity_fixture_weights():
    L = synth.make_layer(1)
    w = oracle.LayerWeights.from_storage("f32", "f32", L.w_router, L.b_router, L.expert)
    ex = [w.expert(e) for e in range(L.E)]
    h = oracle.widen(L.h, "f32")
    base = oracle.moe_forward(h, w, L.k)
    for M in (2, 3):
        big = oracle.moe_forward(h, _expanded(w, ex, M), M * L.k)
        np.testing.assert_allclose(big["out"], base["out"], rtol=1e-12, atol=1e-16)


def _greedy_copy_counts(s_row, copies, kp):
    """How many copies of each original a top-kp pick over the expanded logits
    takes: originals in descending logit order (lower id first on equal
    logits), each contributing all its copies until kp are taken.  Copies of
    one original have equal logits, and every copy of a better original beats
    every copy of a worse one, so the pick is exactly this fill."""
    n = np.zeros(len(s_row), dtype=np.int64)
    left = kp
    for i in sorted(range(len(s_row)), key=lambda e: (-s_row[e], e)):
        n[i] = min(copies[i], left)
        left -= n[i]
        if left == 0:
            break
    return n


@pytest.mark.parametrize("kp", [1, 3, 4, 6, 10])
def test_nonuniform_expansion_closed_form(kp):
    """A non-uniform silent expansion ("gpt-oss-220a20b" Model Details: base
    rows plus added rows; here 8 originals and 5 added rows copying originals
    5, 2, 7, 2, 0, so originals have one to three copies): if original i
    contributes n_i selected copies, the layer is
    sum_i n_i e^(s_i) y_i / sum_i n_i e^(s_i), evaluated per token from the
    base logits and base experts only."""
    rng = np.random.default_rng(52 + kp)
    E = 8
    h, w, ex = rand_layer(rng, T=50, H=24, I=40, E=E)
    cmap = np.concatenate([np.arange(E), [5, 2, 7, 2, 0]])
    copies = np.bincount(cmap, minlength=E)
    wx = oracle.LayerWeights(oracle.expand_rows(w.w_router, cmap), oracle.expand_rows(w.b_router, cmap),
                             lambda j: ex[cmap[j]])
    big = oracle.moe_forward(h, wx, kp)
    s = h @ w.w_router.T + w.b_router
    for t in range(len(h)):
        n = _greedy_copy_counts(s[t], copies, kp)
        # the selected expanded ids: for each original its n_i lowest copies
        want_idx = sorted(j for i in range(E) for j in np.nonzero(cmap == i)[0][:n[i]])
        np.testing.assert_array_equal(big["idx"][t], want_idx)
        num = np.zeros(w.w_router.shape[1])
        den = 0.0
        for i in np.nonzero(n)[0]:
            wg, wu, wd = ex[i]
            g, u = wg @ h[t], wu @ h[t]
            e = n[i] * np.exp(s[t, i] - s[t].max())
            num += e * (wd @ (g / (1 + np.exp(-g)) * u))
            den += e
        np.testing.assert_allclose(big["out"][t], num / den, rtol=1e-12, atol=1e-15)


def test_expand_rows_copies_and_checks():
    x = np.arange(4 * 3).reshape(4, 3)
    cmap = np.array([0, 1, 2, 3, 3, 0, 1])
    y = oracle.expand_rows(x, cmap)
    assert y.shape == (7, 3)
    for j, i in enumerate(cmap):
        np.testing.assert_array_equal(y[j], x[i])
    for bad in ([], [4], [-1], [[0, 1]]):
        with pytest.raises(ValueError):
            oracle.expand_rows(x, np.array(bad, dtype=np.int64))


def test_expansion_mapping_keeps_originals_first():
    x = np.arange(4 * 3).reshape(4, 3)
    y = oracle.expand_silent(x, 3)
    assert y.shape == (12, 3)
    for j in range(12):
        np.testing.assert_array_equal(y[j], x[j % 4])
    np.testing.assert_array_equal(oracle.expand_silent(x, 1), x)
    with pytest.raises(ValueError):
        oracle.expand_silent(x, 0)


# ----------------------------------------------------- routing metadata --

def test_routing_metadata_by_explicit_walk():
    rng = np.random.default_rng(30)
    E, k, T = 7, 3, 50
    idx = np.sort(np.array([rng.choice(E, k, replace=False) for _ in range(T)]), 1)
    md = oracle.routing_metadata(idx, E)
    rows = []
    for e in range(E):                      # expert-major, tokens ascending
        for t in range(T):
            for slot in range(k):
                if idx[t, slot] == e:
                    rows.append(t * k + slot)
    np.testing.assert_array_equal(md["perm_src"], rows)
    counts = [sum(int(e in idx[t]) for t in range(T)) for e in range(E)]
    np.testing.assert_array_equal(md["counts"], counts)
    np.testing.assert_array_equal(md["offsets"], [sum(counts[:e]) for e in range(E + 1)])
    assert md["offsets"][-1] == T * k
    np.testing.assert_array_equal(md["perm_src"][md["inv"]], np.arange(T * k))


# ---------------------------------------------------------------- MXFP4 --

def test_widen_bf16_bit_patterns():
    """bf16 is the high half of an IEEE binary32: 1 sign bit, 8 exponent bits
    (bias 127), 7 fraction bits.  Each stored pattern below has a value that
    the format fixes by itself (normal, subnormal, signed zero, infinities,
    NaN, the largest finite value), so a shift, a sign extension or a byte
    swap in the widening fails one of them."""
    cases = {
        0x0000: 0.0, 0x3F80: 1.0, 0xC000: -2.0, 0xBE80: -0.25, 0x3F81: 1.0 + 2.0 ** -7,
        0x4049: 3.140625, 0x0080: 2.0 ** -126, 0x0001: 2.0 ** -133, 0x007F: 127 * 2.0 ** -133,
        0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127, 0xFF7F: -(2.0 - 2.0 ** -7) * 2.0 ** 127,
        0x7F80: np.inf, 0xFF80: -np.inf,
    }
    bits = np.array(list(cases), dtype=np.uint16).reshape(-1, 1)
    got = oracle.widen(bits, "bf16")
    assert got.shape == bits.shape and got.dtype == np.float64
    np.testing.assert_array_equal(got.ravel(), np.array(list(cases.values())))
    neg0 = oracle.widen(np.array([0x8000], dtype=np.uint16), "bf16")[0]
    assert neg0 == 0.0 and np.signbit(neg0)
    assert np.isnan(oracle.widen(np.array([0x7FC0, 0xFFC1], dtype=np.uint16), "bf16")).all()
    # fp32 storage widens without change
    f = np.array([1.5, -2.0 ** -149, 3.4028234663852886e38], dtype=np.float32)
    np.testing.assert_array_equal(oracle.widen(f, "f32"), [1.5, -2.0 ** -149, 3.4028234663852886e38])


def test_e2m1_decode_matches_spec_table():
    for code, val in _rows("e2m1_table.txt"):
        got = oracle.e2m1_value(int(code))
        assert float(got) == float(val) and math.copysign(1, float(got)) == math.copysign(1, float(val)), code


def test_e8m0_special_values():
    v = oracle.e8m0_value(np.array([0, 1, 126, 127, 128, 254, 255]))
    assert v[0] == 2.0 ** -127 and v[1] == 2.0 ** -126
    assert v[2] == 0.5 and v[3] == 1.0 and v[4] == 2.0 and v[5] == 2.0 ** 127
    assert np.isnan(v[6])


def test_mxfp4_dequant_layout_and_scale():
    # one row of 64 elements = two groups; element 2j in the low nibble of byte j
    codes = np.arange(64) % 16
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)[None, :]
    scales = np.array([[127 - 3, 127 + 2]], dtype=np.uint8)
    got = oracle.mxfp4_dequant(packed, scales)[0]
    table = {int(c): float(v) for c, v in _rows("e2m1_table.txt")}
    want = np.array([table[c] for c in codes]) * np.repeat([2.0 ** -3, 2.0 ** 2], 32)
    np.testing.assert_array_equal(got, want)


def test_mxfp4_bits_per_parameter_is_4_25():
    """4.25 bits per expert parameter counting the shared scales
    ("gpt-oss-20b and gpt-oss-120b" explainer, "Four-bit expert weights")."""
    L = synth.make_layer(4, T=1)
    w = L.expert(3)
    for n in ("gate", "up", "down"):
        assert oracle.mxfp4_bits_per_param(w[n], w["s_" + n]) == 4.25
        assert w[n].nbytes + w["s_" + n].nbytes == 2880 * 2880 * 17 // 32


def test_mxfp4_round_trip_of_representable_values():
    # random codes and scales; every group holds a magnitude >= 4 so that its
    # shared exponent is the one the encoder picks back
    rng = np.random.default_rng(40)
    N, K = 16, 256
    codes = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    codes[codes == 8] = 0                               # -0 re-encodes as +0
    codes[:, ::32] = rng.choice([6, 7, 14, 15], size=(N, K // 32))
    scales = rng.integers(100, 150, size=(N, K // 32)).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    x = oracle.mxfp4_dequant(packed, scales)
    p2, s2 = synth.mxfp4_encode(x.astype(np.float32))
    np.testing.assert_array_equal(s2, scales)
    np.testing.assert_array_equal(p2, packed)


# ------------------------------------------------- numbers on the pages --

def test_routing_capacity_table():
    """C(E, k) per layer as tabulated on the "gpt-oss-40b-64a8-init" page,
    section 3.  Exact counts come from the definition (enumerated where small);
    two printed figures are wrong and are checked as such."""
    rows = {r[0]: r[1:] for r in _rows("combinatorics.txt")}
    base = math.comb(32, 4)
    for name, (E, k, printed, ratio, L, mag) in rows.items():
        E, k, L, mag = int(E), int(k), int(L), int(mag)
        exact = math.comb(E, k)
        if exact <= 700_000:
            assert sum(1 for _ in itertools.combinations(range(E), k)) == exact
        # C(E,k)^L printed as ~10^mag: all six rows agree with the exact count
        assert round(L * math.log10(exact)) == mag, name
        if name == "96a12":
            # printed 2.35e13; exact 624,668,654,531,480 ~ 6.25e14, which the
            # page's own "Over L Layers" table uses; the ratio column follows the
            # wrong figure (6.54e8 instead of ~1.74e10)
            assert exact == 624_668_654_531_480
            assert float(printed) == 2.35e13 and abs(float(printed) / base - float(ratio)) / float(ratio) < 0.01
            assert abs(exact / base - 1.737e10) / 1.737e10 < 1e-3
            continue
        assert int(printed) == exact, name
        r = exact / base
        if name == "64a8":
            # printed 123,091x; exact ratio is 123,085.8x
            assert abs(r - 123085.8) < 0.05 and int(ratio) == 123091
        else:
            assert abs(r - float(ratio)) / float(ratio) < 0.01, name


def test_parameter_counts_match_three_HxI_matrices_per_expert():
    """Shape check against the printed sizes: with hidden = intermediate = 2880,
    32 experts of three [2880 x 2880] matrices, top-4, 24 layers, GQA attention
    (64 q / 8 kv heads of 64) and the 201,088-token vocabulary, the counts come
    out at the printed 20.91B total and 3.61B active (embedding lookup not
    counted as active), 19.8B in the layers, 579.1M per embedding matrix."""
    g = {r[0]: float(r[1]) for r in _rows("page_numbers.txt")}
    H, I, E, k, Lyr = int(g["hidden"]), int(g["intermediate"]), int(g["n_experts"]), int(g["top_k"]), int(g["n_layers"])
    q, kv, hd, V = int(g["q_heads"]), int(g["kv_heads"]), int(g["head_dim"]), int(g["vocab"])
    attn = H * q * hd + 2 * H * kv * hd + q * hd * H
    expert = 3 * H * I
    router = E * H + E
    norms = 2 * H
    layer = attn + E * expert + router + norms
    emb = V * H
    total = Lyr * layer + 2 * emb + H
    active = Lyr * (attn + k * expert + router + norms) + emb + H
    assert round(total / 1e9, 2) == g["total_B"]
    assert round(active / 1e9, 2) == g["active_B"]
    # 19,749,658,368 in the layers prints as 19.7B; the page's 19.8B is reached
    # only if biases the pages never describe are counted (per expert 2*I + H,
    # per layer 8,000 attention biases and 64 sinks: 19,756,487,424).  The
    # layer here follows the pages' bias-free SwiGLU; the gap is 0.03%.
    assert abs(Lyr * layer / 1e9 - g["layers_B"]) <= 0.051
    with_bias = Lyr * (layer + E * (2 * I + H) + (q * hd + 2 * kv * hd + H) + q)
    assert round(with_bias / 1e9, 1) == g["layers_B"]
    assert round(emb / 1e6, 1) == g["embed_M"] == g["lm_head_M"]
    assert round(H / 1e3, 1) == g["norm_K"]


# ------------------------------------------- pre-norm and residual add --

def test_rms_norm_unit_mean_square():
    """Unit gain, epsilon 0: every output row has mean square exactly 1."""
    x = np.random.default_rng(50).standard_normal((7, 33)) * 3.0
    n = oracle.rms_norm(x, np.ones(33), 0.0)
    np.testing.assert_allclose(np.mean(n * n, axis=1), 1.0, rtol=1e-14)


def test_rms_norm_constant_row_closed_form():
    """A row of c's: the mean square is c^2, so each element is g c / sqrt(c^2 + eps)."""
    g = np.linspace(0.5, 2.0, 16)
    for c, eps in ((2.0, 0.0), (-0.3, 1e-5), (1e-3, 1e-5), (5.0, 0.25)):
        n = oracle.rms_norm(np.full((1, 16), c), g, eps)
        np.testing.assert_allclose(n[0], g * c / np.sqrt(c * c + eps), rtol=1e-15)


def test_rms_norm_joint_scaling_of_input_and_eps():
    """rms_norm(a x; a^2 eps) = rms_norm(x; eps) for a > 0 (epsilon sits inside
    the square root, in units of the mean square)."""
    rng = np.random.default_rng(51)
    x, g = rng.standard_normal((5, 24)), rng.standard_normal(24)
    for a in (1e-3, 0.5, 7.0):
        np.testing.assert_allclose(oracle.rms_norm(a * x, g, a * a * 1e-4), oracle.rms_norm(x, g, 1e-4),
                                   rtol=1e-13, atol=1e-15)


def test_rms_norm_gain_acts_per_feature():
    """The gain scales features (columns), not tokens: T != H so a transposed
    gain could not broadcast silently."""
    rng = np.random.default_rng(52)
    x, g = rng.standard_normal((3, 8)), rng.standard_normal(8)
    base = oracle.rms_norm(x, np.ones(8), 1e-6)
    np.testing.assert_allclose(oracle.rms_norm(x, g, 1e-6), base * g[None, :], rtol=1e-15)
    with pytest.raises(ValueError):
        oracle.rms_norm(x, np.ones(3), 1e-6)


def test_rms_norm_hand_example():
    """x = (3, 4), unit gain, eps = 0: mean square 12.5, so (3, 4) / sqrt(12.5)."""
    n = oracle.rms_norm(np.array([[3.0, 4.0]]), np.ones(2), 0.0)
    np.testing.assert_allclose(n[0], [0.8485281374238570, 1.1313708498984760], rtol=1e-15)


def test_block_zero_experts_is_identity():
    """Zero down projections: every expert outputs 0, so the block returns its input."""
    rng = np.random.default_rng(53)
    h, w, ex = rand_layer(rng, T=20, H=24, I=40, E=6)
    zex = [(wg, wu, np.zeros_like(wd)) for wg, wu, wd in ex]
    wz = oracle.LayerWeights(w.w_router, w.b_router, lambda e: zex[e])
    out = oracle.block_forward(h, rng.standard_normal(24), 1e-5, wz, 2)["out"]
    np.testing.assert_array_equal(out, h)


def test_block_two_evaluations_agree():
    """Expert-grouped evaluation vs token-by-token loops (mean square summed
    element by element, experts by matrix-vector products)."""
    rng = np.random.default_rng(54)
    h, w, ex = rand_layer(rng, T=24, H=16, I=20, E=5)
    g = rng.uniform(0.5, 1.5, 16)
    for k in (1, 2, 5):
        a = oracle.block_forward(h, g, 1e-5, w, k)["out"]
        b = oracle.block_forward_per_token(h, g, 1e-5, w, k)
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


# --------------------------------------------------- attention with sinks --

def _golden_sink():
    rows = [l.split() for l in open(os.path.join(GOLD, "attention_sink_example.txt")) if l.strip() and l[0] != "#"]
    d = {r[0]: [float(x) for x in r[1:]] for r in rows}
    return np.array(d["values"]), d["no_sink"][0], d["sink_equal_score"][0]


def test_sink_worked_example_from_the_page():
    vals, no_sink, with_sink = _golden_sink()
    s = np.full(3, 0.7)
    assert oracle.sink_softmax(s, -np.inf) @ vals == pytest.approx(no_sink, rel=1e-15)
    assert oracle.sink_softmax(s, 0.7) @ vals == pytest.approx(with_sink, rel=1e-15)
    # the same example through the decode attention: one head, D = 1, q = 1, k = 0 (equal scores)
    q = np.ones((1, 1, 1))
    k = np.zeros((1, 1, 3, 1))
    v = vals.reshape(1, 1, 3, 1)
    out = oracle.attn_sink_decode(q, k, v, np.array([0.0]), np.array([3]), 0, 1.0)
    assert out[0, 0, 0] == pytest.approx(with_sink, rel=1e-15)


def test_sink_to_minus_infinity_is_plain_softmax():
    from scipy.special import softmax
    s = np.random.default_rng(60).standard_normal((4, 9)) * 3
    np.testing.assert_allclose(oracle.sink_softmax(s, -np.inf), softmax(s, axis=-1), rtol=1e-14)


def test_sink_weight_fills_the_gap_to_one():
    """Real-token weights sum to 1 - exp(sink) / (exp(sink) + sum exp(s))."""
    rng = np.random.default_rng(61)
    s, sink = rng.standard_normal(7), 0.3
    w = oracle.sink_softmax(s, sink)
    assert w.sum() == pytest.approx(1 - np.exp(sink) / (np.exp(sink) + np.exp(s).sum()), rel=1e-14)
    assert np.all(w > 0) and w.sum() < 1
    # a dominant sink silences the head
    assert np.abs(oracle.sink_softmax(s, 800.0)).max() < 1e-300


def test_attention_one_key_window_closed_form():
    """Window 1: only the newest key, out = v_last * e^s / (e^s + e^sink)."""
    rng = np.random.default_rng(62)
    B, Hq, Hkv, Tk, D = 2, 4, 2, 5, 8
    q, k, v = rng.standard_normal((B, Hq, D)), rng.standard_normal((B, Hkv, Tk, D)), rng.standard_normal((B, Hkv, Tk, D))
    sinks, lens = rng.standard_normal(Hq), np.array([5, 3])
    out = oracle.attn_sink_decode(q, k, v, sinks, lens, 1, 0.25)
    for b in range(B):
        for h in range(Hq):
            g = h // 2
            s = 0.25 * q[b, h] @ k[b, g, lens[b] - 1]
            w = np.exp(s) / (np.exp(s) + np.exp(sinks[h]))
            np.testing.assert_allclose(out[b, h], w * v[b, g, lens[b] - 1], rtol=1e-13)


def test_attention_head_groups_and_window_by_brute_force():
    """Against an explicit double loop over heads and keys (window and lengths
    applied by position tests), and a permutation of the query heads inside a
    group permutes the output the same way."""
    rng = np.random.default_rng(63)
    B, Hq, Hkv, Tk, D = 3, 8, 2, 40, 4
    q, k, v = rng.standard_normal((B, Hq, D)), rng.standard_normal((B, Hkv, Tk, D)), rng.standard_normal((B, Hkv, Tk, D))
    sinks, lens = rng.standard_normal(Hq), np.array([40, 17, 1])
    for window in (0, 6):
        out = oracle.attn_sink_decode(q, k, v, sinks, lens, window, 0.5)
        for b in range(B):
            for h in range(Hq):
                num, den = np.zeros(D), np.exp(sinks[h])
                for j in range(Tk):
                    if j >= lens[b] or (window and j < lens[b] - window):
                        continue
                    e = np.exp(0.5 * sum(q[b, h, d] * k[b, h // 4, j, d] for d in range(D)))
                    num += e * v[b, h // 4, j]
                    den += e
                np.testing.assert_allclose(out[b, h], num / den, rtol=1e-12)
    perm = np.array([1, 0, 3, 2, 4, 5, 7, 6])
    a = oracle.attn_sink_decode(q[:, perm], k, v, sinks[perm], lens, 0, 0.5)
    np.testing.assert_allclose(a, oracle.attn_sink_decode(q, k, v, sinks, lens, 0, 0.5)[:, perm], rtol=1e-14)
