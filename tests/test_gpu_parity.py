"""Parity of the HIP path (through the C interface) with the fp64 reference.

Routing (top-k indices in ascending expert id, offsets, permutation) must be
bit-exact once near-ties (k-th and (k+1)-th reference logits within 1e-5) are
settled; outputs must be within relative L2 5e-3 and max abs 1e-2*max|ref| for
bf16/MXFP4 and relative L2 1e-5 for fp32.  Every token is compared, at the
full sizes too (the fp64 reference of each full-size layer is computed once
and shared by the tests that need it).  Before every call the workspace, the
output and the routing outputs are filled with 0xFF bytes (NaN, or -1 for
integers), so nothing the library leaves unwritten or reads stale can pass."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_token_amd as smoe
import synth
from gpu_util import (check_layer, check_out, device_weights, oracle_weights, problem, reconcile, reference_out,
                      rel_l2, run, to_dev, workers)

pytestmark = pytest.mark.gpu

_cache = {}


def layer_full(key):
    """Seeded inputs of a workload at its full T, weights stacked (cached)."""
    if key not in _cache:
        L = synth.make_layer(key)
        _cache[key] = (L, L.stacked())
    return _cache[key]


def with_T(L: synth.Layer, T: int) -> synth.Layer:
    return dataclasses.replace(L, T=T, h=L.h[:T])


# ------------------------------------------------------------ small sizes --

def test_fixture_fp32_all_tokens():
    L, st = layer_full(1)
    m, _ = check_layer(L, st)
    assert m["rel_l2"] < 1e-5


@pytest.mark.parametrize("T", [1, 7, 17, 33])
def test_fixture_fp32_ragged_T(T):
    L, st = layer_full(1)
    check_layer(with_T(L, T), st)


EDGE = [
    synth.Config(101, "ragged-7e-top3", T=333, H=128, I=192, E=7, k=3, act="bf16", expert="bf16"),
    synth.Config(102, "top1", T=100, H=64, I=64, E=5, k=1, act="bf16", expert="bf16"),
    synth.Config(103, "k-equals-E", T=50, H=64, I=128, E=6, k=6, act="bf16", expert="bf16"),
    synth.Config(104, "single-expert", T=40, H=64, I=64, E=1, k=1, act="bf16", expert="bf16"),
    synth.Config(105, "mostly-empty-experts", T=3, H=128, I=128, E=64, k=2, act="bf16", expert="bf16"),
    synth.Config(106, "mxfp4-small", T=200, H=128, I=256, E=9, k=2, act="bf16", expert="mxfp4"),
    synth.Config(107, "f32-tails", T=77, H=192, I=320, E=5, k=2, act="f32", expert="f32", bias_std=0.01),
    synth.Config(108, "many-tiles-per-expert", T=1500, H=64, I=128, E=3, k=2, act="bf16", expert="bf16"),
    synth.Config(109, "1024-experts", T=40, H=64, I=64, E=1024, k=9, act="bf16", expert="bf16"),
    # decode-sized (at most 16 rows per expert on average): the weight-streaming kernels
    synth.Config(110, "decode-K-tails", T=24, H=192, I=320, E=8, k=2, act="bf16", expert="bf16"),
    synth.Config(111, "decode-mxfp4-K-tails", T=20, H=192, I=320, E=6, k=3, act="bf16", expert="mxfp4"),
    synth.Config(112, "decode-several-tiles-per-expert", T=64, H=128, I=128, E=8, k=2, act="bf16", expert="bf16"),
    synth.Config(113, "decode-one-token", T=1, H=256, I=192, E=16, k=4, act="bf16", expert="mxfp4"),
    # routing computed inside the gate/up kernel (T <= 64, E <= 64): its largest shape and one expert
    synth.Config(114, "decode-fused-64-tokens-64-experts", T=64, H=256, I=128, E=64, k=16, act="bf16", expert="bf16"),
    synth.Config(115, "decode-fused-single-expert", T=16, H=64, I=64, E=1, k=1, act="bf16", expert="bf16"),
    # MXFP4 decode with the scales staged in LDS (E > 64, so not fused): K tails in both products;
    # then the largest MXFP4 K (4992, 156 scale groups per row)
    synth.Config(116, "decode-mxfp4-staged-scales", T=24, H=192, I=320, E=80, k=2, act="bf16", expert="mxfp4"),
    synth.Config(117, "decode-mxfp4-max-K", T=4, H=4992, I=64, E=66, k=1, act="bf16", expert="mxfp4"),
]


def test_mxfp4_prefill_integer_decode_matches_hardware_decode():
    """The prefill GEMMs decode an MXFP4 tile with the hardware scaled
    conversion when every scale of its live weight rows is in 2..252, else
    on the integer path.  Scale group 1 of a few weight rows gets all-zero
    codes (it contributes exactly nothing) and scale 0 (integer path for the
    tiles holding those rows) or 120 (hardware path): the outputs must be
    bitwise equal, so the integer path reproduces the hardware decode on
    every other group, and both match the fp64 reference.  Gate row 3 of
    experts 0-4 (gate/up column tile 0 only) and down row 70 of experts 5-8
    are changed, so both paths run in each launch."""
    cfg = next(c for c in EDGE if c.name == "mxfp4-small")
    L = synth.make_layer(cfg)
    base = L.stacked()
    outs = []
    for scale in (0, 120):
        st = {n: a.copy() for n, a in base.items()}
        for e in range(cfg.E):
            n, row = ("gate", 3) if e < 5 else ("down", 70)
            st[n][e, row, 16:32] = 0      # packed codes of K elements 32..63
            st["s_" + n][e, row, 1] = scale
        m, g = check_layer(L, st)
        print(scale, m)
        outs.append(g["out_raw"])
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


@pytest.mark.parametrize("cfg", EDGE, ids=[c.name for c in EDGE])
def test_edge_shapes(cfg):
    L = synth.make_layer(cfg)
    check_layer(L, L.stacked())


def test_gpt_oss_20b_layer_2048_tokens_all_outputs():
    """Several row tiles per expert and a ragged last tile, all tokens compared."""
    L, st = layer_full(2)
    m, _ = check_layer(with_T(L, 2048), st)
    print(m)


def test_gpt_oss_20b_decode_64_tokens():
    L, st = layer_full(2)
    check_layer(with_T(L, 64), st)


@pytest.mark.parametrize("T", [512, 64], ids=["prefill-kernels", "decode-fused-routing"])
def test_deterministic_run_to_run(T):
    """Bitwise-identical outputs and routing tables on repeated calls (no
    atomics decide an order anywhere, including the routing that every decode
    workgroup computes for itself)."""
    L, st = layer_full(2)
    prob = problem(L.cfg, T)
    w = device_weights(L, st)
    h = to_dev(L.h[:T], "bf16")
    a = run(prob, w, h, "bf16", byte=0xFF)
    b = run(prob, w, h, "bf16", byte=0x7F)   # a second, differently poisoned workspace
    assert torch.equal(a["out_raw"].view(torch.int16), b["out_raw"].view(torch.int16))
    for n in ("logits", "topk_idx", "topk_w", "perm_src"):
        np.testing.assert_array_equal(a[n], b[n])


# --------------------------------------------------------------- full sizes --

def test_gpt_oss_20b_prefill_4096_all_tokens():
    L, st = layer_full(2)
    m, _ = check_layer(L, st)
    print(m)


@pytest.mark.parametrize("M", [2, 3])
def test_silent_expansion_identity(M):
    """64a8 / 96a12: the expanded layer equals the 32a4 layer (GPU vs GPU and
    GPU vs the fp64 reference), copies of a router row give bitwise-equal
    logits, and the selected set is the copies of the base selection."""
    L, st = layer_full(2)
    c = L.cfg
    base = problem(c, L.T)
    w = device_weights(L, st)
    big = smoe.Problem(L.T, c.H, c.I, M * c.E, M * c.k, base.act_dtype, base.expert_dtype)
    wx = {n: torch.empty((M * t.shape[0],) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
          for n, t in w.items()}
    smoe.moe_expand_silent(base, w, M, wx)
    torch.cuda.synchronize()
    for n in w:
        for m in range(M):
            assert torch.equal(wx[n][m * c.E:(m + 1) * c.E], w[n])
    h = to_dev(L.h, "bf16")
    gb = run(base, w, h, "bf16")
    gx = run(big, wx, h, "bf16")
    # duplicated router rows: bitwise-equal logits
    for m in range(1, M):
        np.testing.assert_array_equal(gx["logits"][:, m * c.E:(m + 1) * c.E], gx["logits"][:, :c.E])
    np.testing.assert_array_equal(gx["logits"][:, :c.E], gb["logits"])
    # selection: the M copies of each base choice (ascending ids)
    want = np.sort(np.concatenate([gb["topk_idx"] + m * c.E for m in range(M)], axis=1), axis=1)
    np.testing.assert_array_equal(gx["topk_idx"], want)
    # outputs: expanded GPU vs base GPU over all tokens, and vs the fp64 base layer
    r = rel_l2(gx["out"], gb["out"])
    assert r <= 5e-3 and np.abs(gx["out"] - gb["out"]).max() <= 1e-2 * np.abs(gb["out"]).max()
    # every token against the fp64 base layer, near-ties of the base layer excluded
    ow = oracle_weights(L, st)
    h64 = oracle.widen(L.h, "bf16")
    s = oracle.router_logits(h64, ow.w_router, ow.b_router)
    near = oracle.topk_gap(s, c.k) < 1e-5
    ref = reference_out(L, st, L.T, oracle.select_topk(s, c.k))
    check_out(gx["out"][~near], ref[~near], "bf16")
    print({"M": M, "gpu_vs_gpu_rel_l2": r})


@pytest.mark.parametrize("M,kp,T", [(2, 4, 256), (3, 4, 256), (2, 2, 256), (2, 4, 4096), (3, 4, 4096)],
                         ids=["64a4", "96a4", "64a2", "64a4-prefill-4096", "96a4-prefill-4096"])
def test_silent_expansion_narrow_k(M, kp, T):
    """Deploy-narrow shapes: the 32a4 layer expanded M times, run with k' = kp
    at T tokens.  Copies of a router row give bitwise-equal logits, so where
    the k'-th pick is one of several copies (96a4: three copies of the best
    expert and one of the second) the lower index must win exactly as in the
    reference.  Routing bit-exact and outputs within tolerance against the
    fp64 reference on the expanded layer; where kp = M j the expanded GPU
    layer also matches the base GPU layer at top-j."""
    L, st = layer_full(2)
    c = L.cfg
    base = problem(c, T)
    w = device_weights(L, st)
    wx = {n: torch.empty((M * t.shape[0],) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
          for n, t in w.items()}
    smoe.moe_expand_silent(base, w, M, wx)
    big = smoe.Problem(T, c.H, c.I, M * c.E, kp, base.act_dtype, base.expert_dtype)
    h = to_dev(L.h[:T], "bf16")
    gx = run(big, wx, h, "bf16")
    ow = oracle_weights(L, st)
    cmap = np.arange(M * c.E) % c.E
    wr = oracle.expand_silent(ow.w_router, M, cmap)
    br = oracle.expand_silent(ow.b_router, M, cmap)
    owx = oracle.LayerWeights(wr, br, lambda j: ow.expert(cmap[j]))
    h64 = oracle.widen(L.h[:T], "bf16")
    # distinct base experts near a selection boundary would make the pick
    # legitimately ambiguous; this draw has none among any token's top three
    sb = -np.sort(-oracle.router_logits(h64, ow.w_router, ow.b_router), axis=1)
    j = -(-kp // M)
    assert np.min(sb[:, :j] - sb[:, 1:j + 1]) >= 1e-5
    s = oracle.router_logits(h64, wr, br)
    ref_idx = oracle.select_topk(s, kp)
    np.testing.assert_array_equal(gx["topk_idx"], ref_idx)
    md = oracle.routing_metadata(ref_idx, M * c.E)
    np.testing.assert_array_equal(gx["expert_offsets"], md["offsets"])
    np.testing.assert_array_equal(gx["perm_src"], md["perm_src"])
    ref = oracle.moe_forward(h64, owx, kp, idx=ref_idx, workers=workers())
    m = check_out(gx["out"], ref["out"], "bf16")
    if kp % M == 0:
        gb = run(problem(c, T, k=kp // M), w, h, "bf16")
        r = rel_l2(gx["out"], gb["out"])
        assert r <= 5e-3 and np.abs(gx["out"] - gb["out"]).max() <= 1e-2 * np.abs(gb["out"]).max()
        m["gpu_vs_base_top_j"] = r
    print(m)


@pytest.mark.parametrize("kp", [8, 20], ids=["248-rows-top8", "248-rows-top20"])
def test_nonuniform_expansion_248_rows(kp):
    """The 248 expert rows of the 220a20b layer (its page, Model Details: 128
    base rows plus 120 added rows) built by moe_expand_copies from the
    128-expert MXFP4 layer, added row 128 + j starting as a copy of base row j:
    the expanded tensors equal their sources, copies of a router row give
    bitwise-equal logits, routing is bit-exact against the fp64 reference
    of the expanded layer (exact ties between copies go to the lower id) and
    every token's output is within tolerance; where a token's base top-(kp/2)
    experts all have two copies the expanded layer equals the base layer at
    top-(kp/2) (the silent-init identity)."""
    L, st = layer_full(4)
    c = L.cfg
    T = 2048
    cmap = np.concatenate([np.arange(128), np.arange(120)])
    base = problem(c, T)
    w = device_weights(L, st)
    wx = {n: torch.empty((len(cmap),) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device) for n, t in w.items()}
    smoe.moe_expand_copies(base, w, cmap, wx)
    torch.cuda.synchronize()
    for n in w:
        assert torch.equal(wx[n][:128], w[n]) and torch.equal(wx[n][128:], w[n][:120])
    big = smoe.Problem(T, c.H, c.I, len(cmap), kp, base.act_dtype, base.expert_dtype)
    h = to_dev(L.h[:T], "bf16")
    gx = run(big, wx, h, "bf16")
    np.testing.assert_array_equal(gx["logits"][:, 128:], gx["logits"][:, :120])
    ow = oracle_weights(L, st)
    owx = oracle.LayerWeights(oracle.expand_rows(ow.w_router, cmap), oracle.expand_rows(ow.b_router, cmap),
                              lambda j: ow.expert(int(cmap[j])))
    h64 = oracle.widen(L.h[:T], "bf16")
    s = oracle.router_logits(h64, owx.w_router, owx.b_router)
    ref_idx = oracle.select_topk(s, kp)
    gap = oracle.topk_gap(s, kp)
    eff, n_near, _ = reconcile(ref_idx, s, gap, gx["topk_idx"].astype(np.int64), kp)
    np.testing.assert_array_equal(gx["topk_idx"], eff)
    # where the boundary is an exact tie between copies of one expert that is
    # clear of every other expert, the pick is unique (lower copy first)
    sb = oracle.router_logits(h64, ow.w_router, ow.b_router)
    kth = cmap[np.argsort(-s, axis=1, kind="stable")[:, kp - 1]]
    clear = np.array([np.min(np.abs(np.delete(sb[t], kth[t]) - sb[t, kth[t]])) >= 1e-5 for t in range(T)])
    copy_tie = (gap == 0) & clear
    assert copy_tie.sum() > 100
    np.testing.assert_array_equal(gx["topk_idx"][copy_tie], ref_idx[copy_tie])
    md = oracle.routing_metadata(eff, len(cmap))
    np.testing.assert_array_equal(gx["expert_offsets"], md["offsets"])
    np.testing.assert_array_equal(gx["perm_src"], md["perm_src"])
    ref = oracle.moe_forward(h64, owx, kp, idx=eff, workers=workers())
    m = check_out(gx["out"], ref["out"], "bf16")
    # silent identity on the tokens whose base top-(kp/2) all have copies
    j = kp // 2
    gb = run(problem(c, T, k=j), w, h, "bf16")
    both = np.all(gb["topk_idx"] < 120, axis=1) & (oracle.topk_gap(sb, j) >= 1e-5)
    assert both.sum() > T // 4
    r = rel_l2(gx["out"][both], gb["out"][both])
    assert r <= 5e-3 and np.abs(gx["out"][both] - gb["out"][both]).max() <= 1e-2 * np.abs(gb["out"][both]).max()
    m.update(n_near=n_near, exact_copy_ties=int(copy_tie.sum()), identity_tokens=int(both.sum()), gpu_vs_base_rel_l2=r)
    print(m)


def test_random_64a8_prefill_4096_all_tokens():
    L, st = layer_full(3)
    m, _ = check_layer(L, st)
    print(m)


def test_gpt_oss_120b_mxfp4_skewed_8192_all_tokens():
    L, st = layer_full(4)
    m, g = check_layer(L, st)
    counts = np.diff(g["expert_offsets"])
    hot = counts[L.hot_set].sum() / counts.sum()
    assert 0.49 <= hot <= 0.51
    print(m, {"hot_share": float(hot)})


def test_220a20b_mxfp4_prefill_2048_all_tokens():
    L, st = layer_full(5)
    m, _ = check_layer(L, st)
    print(m)


def test_220a20b_mxfp4_decode_32_tokens():
    L, st = layer_full(5)
    m, _ = check_layer(with_T(L, 32), st)
    print(m)


# -------------------------------------------------------------- MXFP4 decode --

def _bf16_bits_of(x64: np.ndarray) -> np.ndarray:
    """bf16 bits of values that bf16 represents exactly (low half is zero)."""
    b = x64.astype(np.float32).view(np.uint32)
    assert not np.any(b[np.isfinite(x64)] & 0xFFFF)
    return (b >> 16).astype(np.uint16)


@pytest.mark.parametrize("name", ["decode-mxfp4-staged-scales", "mxfp4-small"])
def test_mxfp4_codes_off_the_line_grid(name):
    """MXFP4 code blocks that start 16, 48 and 80 bytes past a 128-byte memory
    line (views into larger buffers; the API asks for 16-byte alignment only).
    The decode kernels copy codes along the memory's line grid, so these
    starts take their line-offset arithmetic; the outputs must be bitwise
    those of the same layer with line-aligned weights, and the layer must
    still match the fp64 oracle."""
    cfg = next(c for c in EDGE if c.name == name)
    L = synth.make_layer(cfg)
    st = L.stacked()
    w = device_weights(L, st)
    shifted = dict(w)
    for n, off in (("w_gate", 48), ("w_up", 80), ("w_down", 16)):
        t = w[n]
        buf = torch.zeros(t.numel() + 256, dtype=torch.uint8, device=t.device)
        v = buf[off:off + t.numel()].view(t.shape)
        v.copy_(t)
        assert v.data_ptr() % 128 == off
        shifted[n] = v
    prob = problem(cfg, L.T)
    h = to_dev(L.h, cfg.act)
    g0 = run(prob, w, h, cfg.act)
    g1 = run(prob, shifted, h, cfg.act)
    assert torch.equal(g0["out_raw"].view(torch.int16), g1["out_raw"].view(torch.int16))
    check_layer(L, st, w_dev=shifted)


def test_mxfp4_decode_bit_exact_every_code_and_scale():
    # every byte (two codes) with every scale 0..254: 16 groups of 16 bytes per scale
    packed = np.tile(np.arange(256, dtype=np.uint8).reshape(16, 16), (255, 1))
    scales = np.repeat(np.arange(255, dtype=np.uint8), 16)
    ref = oracle.mxfp4_dequant(packed.reshape(-1, 16), scales.reshape(-1, 1))
    out = torch.empty(packed.size * 2, dtype=torch.int16, device="cuda")
    smoe.moe_mxfp4_decode(to_dev(packed, "u8"), to_dev(scales, "u8"), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16).reshape(ref.shape)
    finite = np.abs(ref) <= float.fromhex("0x1.fep127")   # bf16 max
    np.testing.assert_array_equal(got[finite], _bf16_bits_of(ref[finite]))
    over = ~finite
    assert np.all((got[over] & 0x7FFF) == 0x7F80)        # beyond bf16 range: +-inf
    assert np.all((got[over] >> 15) == (ref[over] < 0))


def test_mxfp4_decode_bit_exact_workload_weights():
    L, st = layer_full(4)
    for n in ("gate", "down"):
        packed, scales = st[n][5], st["s_" + n][5]
        ref = oracle.mxfp4_dequant(packed, scales)
        out = torch.empty(ref.size, dtype=torch.int16, device="cuda")
        smoe.moe_mxfp4_decode(to_dev(packed, "u8"), to_dev(scales, "u8"), out)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16), _bf16_bits_of(ref).ravel())


# ---------------------------------------------------------------- interface --

def test_zero_tokens_is_a_noop_and_errors_leave_outputs_untouched():
    L, st = layer_full(1)
    w = device_weights(L, st)
    prob0 = problem(L.cfg, 0)
    out = torch.full((4, 64), 7.0, device="cuda")
    smoe.moe_forward(prob0, w, None, None, workspace=torch.empty(1, dtype=torch.uint8, device="cuda"),
                     workspace_bytes=0)
    prob = problem(L.cfg, 4)
    h = to_dev(L.h[:4], "f32")
    need = smoe.moe_workspace_bytes(prob)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    with pytest.raises(smoe.MoeError) as ei:
        smoe.moe_forward(prob, w, h, out, workspace=ws, workspace_bytes=need - 1)
    assert ei.value.status == -4
    with pytest.raises(smoe.MoeError) as ei:
        smoe.moe_forward(prob, w, h.view(-1)[1:].data_ptr(), out, workspace=ws)
    assert ei.value.status == -5
    bad = dataclasses.replace(prob, k=5)
    with pytest.raises(smoe.MoeError) as ei:
        smoe.moe_forward(bad, w, h, out, workspace=ws)
    assert ei.value.status == -2
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_profile_hooks_report_every_stage():
    L, st = layer_full(1)
    prob = problem(L.cfg, 64)
    w = device_weights(L, st)
    h = to_dev(L.h, "f32")
    out = torch.empty((64, 64), device="cuda")
    smoe.moe_profile_begin(3)
    for _ in range(5):
        smoe.moe_forward(prob, w, h, out)
    ms, calls = smoe.moe_profile_end()
    assert calls == 3 and len(ms) == 5 and all(x > 0 for x in ms)
    with pytest.raises(smoe.MoeError):
        smoe.moe_profile_end()


def test_profile_mask_records_only_selected_stages():
    L, st = layer_full(1)
    prob = problem(L.cfg, 64)
    w = device_weights(L, st)
    h = to_dev(L.h, "f32")
    out = torch.empty((64, 64), device="cuda")
    smoe.moe_profile_begin_mask(2, (1 << 2) | (1 << 3))   # the gate/up stage only
    for _ in range(2):
        smoe.moe_forward(prob, w, h, out)
    ms, calls = smoe.moe_profile_end()
    assert calls == 2 and ms[2] > 0 and all(ms[i] == 0 for i in (0, 1, 3, 4))
