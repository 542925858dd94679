"""The C interface without a GPU: the library loads, exports every function
include/moe.h declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

import sparse_mixture_experts_token_amd as smoe

HEADER = os.path.join(os.path.dirname(__file__), "..", "include", "moe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*(moe_[a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = smoe.load()
    names = declared_functions()
    assert len(names) == 17, names
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(smoe.EXPORTED) == names


def test_status_strings():
    for code in range(-9, 1):
        assert smoe.moe_status_string(code) and smoe.moe_status_string(code) != "unknown status"
    assert smoe.moe_status_string(-99) == "unknown status"
    assert smoe.moe_stage_name(2) == "gateup_swiglu_gemm"


def _ws(**kw):
    base = dict(T=16, H=64, I=128, E=4, k=2, act_dtype=smoe.MOE_F32, expert_dtype=smoe.MOE_F32)
    base.update(kw)
    return smoe.moe_workspace_bytes(smoe.Problem(**base))


def test_workspace_size_and_shape_limits():
    assert _ws() > 0
    assert _ws(T=32) > _ws(T=16)
    assert _ws(T=0) > 0
    for bad in (dict(k=0), dict(k=5), dict(E=0), dict(E=1025, k=2), dict(H=96), dict(I=100), dict(T=-1),
                dict(act_dtype=smoe.MOE_BF16, expert_dtype=smoe.MOE_F32), dict(expert_dtype=smoe.MOE_MXFP4),
                dict(T=1 << 20, k=4, H=1024)):
        assert _ws(**bad) == 0, bad
    assert _ws(E=1024, k=1024, T=2) > 0
    assert _ws(act_dtype=smoe.MOE_BF16, expert_dtype=smoe.MOE_MXFP4) > 0


def _call(problem, weights=None, h=0x1000, out=0x2000, ws=0x3000, ws_bytes=1 << 40):
    lib = smoe.load()
    w = smoe._Weights(*[weights.get(n) if weights else 0x4000 for n in smoe._WEIGHT_FIELDS])
    p = problem._c() if problem is not None else None
    return lib.moe_forward(ctypes.byref(p) if p is not None else None, ctypes.byref(w), h, out, None, ws,
                           ws_bytes, None)


def test_forward_argument_errors_return_before_any_launch():
    P = smoe.Problem(16, 64, 128, 4, 2, smoe.MOE_F32, smoe.MOE_F32)
    assert _call(None) == -1
    assert _call(smoe.Problem(16, 64, 128, 4, 5, smoe.MOE_F32, smoe.MOE_F32)) == -2
    assert _call(smoe.Problem(16, 64, 128, 4, 2, smoe.MOE_F32, smoe.MOE_BF16)) == -3
    assert _call(P, h=0) == -1
    assert _call(P, h=0x1004) == -5
    assert _call(P, ws_bytes=16) == -4
    w = {n: 0x4000 for n in smoe._WEIGHT_FIELDS}
    w["w_down"] = 0
    assert _call(P, weights=w) == -1
    mx = smoe.Problem(16, 64, 128, 4, 2, smoe.MOE_BF16, smoe.MOE_MXFP4)
    w = {n: 0x4000 for n in smoe._WEIGHT_FIELDS}
    w["s_up"] = 0
    assert _call(mx, weights=w) == -1
    # T = 0 is a no-op even with no buffers at all
    assert _call(smoe.Problem(0, 64, 128, 4, 2, smoe.MOE_F32, smoe.MOE_F32), h=0, out=0, ws=0, ws_bytes=0) == 0


def _block(problem, g=0x5000, eps=1e-5, x=0x1000, out=0x2000, ws=0x3000, ws_bytes=1 << 40):
    lib = smoe.load()
    w = smoe._Weights(*[0x4000 for _ in smoe._WEIGHT_FIELDS])
    p = problem._c()
    return lib.moe_block_forward(ctypes.byref(p), ctypes.byref(w), g, eps, x, out, None, ws, ws_bytes, None)


def test_block_argument_errors_return_before_any_launch():
    P = smoe.Problem(16, 64, 128, 4, 2, smoe.MOE_BF16, smoe.MOE_BF16)
    lib = smoe.load()
    need = lib.moe_block_workspace_bytes(ctypes.byref(P._c()))
    # the normalised input (fp32 and bf16) and the widened router come on top of the routing tables
    assert need > lib.moe_workspace_bytes(ctypes.byref(P._c())) > 0
    assert _block(P, g=0) == -1
    assert _block(P, g=0x5004) == -5
    assert _block(P, x=0) == -1
    for eps in (-1e-6, float("nan"), float("inf")):
        assert _block(P, eps=eps) == -2, eps
    assert _block(P, ws_bytes=need - 1) == -4
    assert _block(smoe.Problem(16, 64, 128, 4, 5, smoe.MOE_BF16, smoe.MOE_BF16)) == -2
    # T = 0 is a no-op even with no buffers at all
    assert _block(smoe.Problem(0, 64, 128, 4, 2, smoe.MOE_BF16, smoe.MOE_BF16), g=0, x=0, out=0, ws=0,
                  ws_bytes=0) == 0


def test_backward_argument_errors_return_before_any_launch():
    lib = smoe.load()
    P = smoe.Problem(8, 64, 128, 4, 2, smoe.MOE_BF16, smoe.MOE_BF16)
    w = smoe._Weights(0x1000, 0x1100, 0x2000, 0x3000, 0x4000, None, None, None)
    r = smoe._Routing(None, 0x5000, 0x5100, 0x5200, 0x5300)
    g = smoe._Grads(0x6000, 0x6100, 0x6200, 0x6300, 0x6400)
    need = lib.moe_backward_workspace_bytes(ctypes.byref(P._c()))
    assert need > 0

    def call(p=P, w=w, h=0x7000, d=0x7100, r=r, tr=None, dh=0x7200, g=g, ws=0x8000, nb=need):
        return lib.moe_backward(ctypes.byref(p._c()), ctypes.byref(w) if w is not None else None, h, d,
                                ctypes.byref(r) if r is not None else None, tr, dh, ctypes.byref(g), ws, nb, None)

    assert call(p=smoe.Problem(8, 64, 128, 4, 2, smoe.MOE_F32, smoe.MOE_F32)) == -3
    assert call(p=smoe.Problem(8, 64, 128, 4, 2, smoe.MOE_BF16, smoe.MOE_MXFP4)) == -3
    assert call(p=smoe.Problem(8, 60, 128, 4, 2)) == -2
    assert call(h=0) == -1 and call(d=0) == -1 and call(r=None) == -1 and call(ws=0) == -1
    assert call(r=smoe._Routing(None, 0x5000, None, 0x5200, 0x5300)) == -1
    assert call(nb=need - 1) == -4
    assert call(h=0x7008) == -5 and call(dh=0x7208) == -5
    assert call(g=smoe._Grads(0x6002, None, None, None, None)) == -5
    # T = 0 writes nothing and needs no buffers
    assert call(p=smoe.Problem(0, 64, 128, 4, 2), h=0, d=0, r=None, dh=0, ws=0, nb=0) == 0
    # switched off: a call that passes every check enqueues nothing
    assert call() == -8
    assert "switched off" in smoe.moe_status_string(-8)


def test_attention_argument_errors_return_before_any_launch():
    lib = smoe.load()

    def call(P, q=0x1000, k=0x2000, v=0x3000, s=0x4000, lens=None, out=0x5000, ws=0x7000, ws_bytes=1 << 40):
        p = P._c()
        return lib.moe_attn_sink_decode(ctypes.byref(p), q, k, v, s, lens, out, ws, ws_bytes, None)

    P = smoe.AttnProblem(4, 64, 8, 300, 64, 128)
    assert lib.moe_attn_sink_decode(None, 1, 1, 1, 1, None, 1, 1, 1, None) == -1
    need = lib.moe_attn_workspace_bytes(ctypes.byref(P._c()))
    assert need > 0 and lib.moe_attn_workspace_bytes(ctypes.byref(smoe.AttnProblem(4, 60, 8, 300, 64)._c())) == 0
    assert call(P, ws_bytes=need - 1) == -4
    assert call(P, ws=0) == -1
    assert call(P, ws=0x7004) == -5
    for bad in (dict(Hq=60), dict(Hq=128, Hkv=8), dict(D=12), dict(D=72), dict(Tk=0), dict(window=-1), dict(Hkv=0)):
        kw = dict(B=4, Hq=64, Hkv=8, Tk=300, D=64, window=0)
        kw.update(bad)
        assert call(smoe.AttnProblem(**kw)) == -2, bad
    assert call(smoe.AttnProblem(4, 64, 8, 300, 64, 0, float("nan"))) == -2
    assert call(P, q=0) == -1
    assert call(P, s=0) == -1
    assert call(P, k=0x2008) == -5
    assert call(P, lens=0x6002) == -5
    # B = 0 is a no-op even with no buffers
    assert call(smoe.AttnProblem(0, 64, 8, 300, 64), q=0, k=0, v=0, s=0, out=0, ws=0, ws_bytes=0) == 0


def test_expand_and_decode_argument_errors():
    lib = smoe.load()
    P = smoe.Problem(0, 64, 128, 4, 2, smoe.MOE_BF16, smoe.MOE_BF16)._c()
    w = smoe._Weights(*([0x4000] * 8))
    assert lib.moe_expand_silent(ctypes.byref(P), ctypes.byref(w), 0, ctypes.byref(w), None) == -2
    assert lib.moe_expand_silent(ctypes.byref(P), ctypes.byref(w), 257, ctypes.byref(w), None) == -2
    w0 = smoe._Weights(*([0] * 8))
    assert lib.moe_expand_silent(ctypes.byref(P), ctypes.byref(w0), 2, ctypes.byref(w), None) == -1
    assert lib.moe_expand_silent(None, ctypes.byref(w), 2, ctypes.byref(w), None) == -1
    ids = (ctypes.c_int32 * 3)(0, 3, 1)
    assert lib.moe_expand_copies(ctypes.byref(P), ctypes.byref(w), None, 3, ctypes.byref(w), None) == -1
    assert lib.moe_expand_copies(ctypes.byref(P), ctypes.byref(w), ids, 0, ctypes.byref(w), None) == -2
    assert lib.moe_expand_copies(ctypes.byref(P), ctypes.byref(w), ids, 1025, ctypes.byref(w), None) == -2
    bad = (ctypes.c_int32 * 3)(0, 4, 1)   # expert 4 of a 4-expert layer
    assert lib.moe_expand_copies(ctypes.byref(P), ctypes.byref(w), bad, 3, ctypes.byref(w), None) == -2
    neg = (ctypes.c_int32 * 3)(0, -1, 1)
    assert lib.moe_expand_copies(ctypes.byref(P), ctypes.byref(w), neg, 3, ctypes.byref(w), None) == -2
    assert lib.moe_expand_copies(ctypes.byref(P), ctypes.byref(w0), ids, 3, ctypes.byref(w), None) == -1
    assert lib.moe_mxfp4_decode(0x1000, 0x2000, -1, 0x3000, None) == -2
    assert lib.moe_mxfp4_decode(0, 0x2000, 4, 0x3000, None) == -1
    assert lib.moe_mxfp4_decode(0x1008, 0x2000, 4, 0x3000, None) == -5
    assert lib.moe_mxfp4_decode(0, 0, 0, 0, None) == 0


def test_profile_end_without_begin_is_a_state_error():
    lib = smoe.load()
    assert lib.moe_profile_end(None, None) == -7
    assert lib.moe_profile_begin(0) == -2


def test_profile_mask_argument_errors():
    lib = smoe.load()
    assert lib.moe_profile_begin_mask(4, 0) == -2                                  # empty mask
    assert lib.moe_profile_begin_mask(4, smoe.MOE_PROFILE_ALL + 1) == -2          # bit beyond the last boundary
    assert lib.moe_profile_begin_mask(0, smoe.MOE_PROFILE_ALL) == -2              # no calls


def test_noalloc_argument_errors_return_before_any_launch():
    """moe_forward_noalloc checks its arguments, and the problem's workspace
    against the static scratch limit, before it touches the device."""
    lib = smoe.load()

    def call(p, h=0x1000, out=0x2000, weights=None):
        w = smoe._Weights(*[weights.get(n) if weights else 0x4000 for n in smoe._WEIGHT_FIELDS])
        return lib.moe_forward_noalloc(ctypes.byref(p._c()) if p is not None else None, ctypes.byref(w), h, out,
                                       None, None)

    P = smoe.Problem(16, 64, 128, 4, 2, smoe.MOE_BF16, smoe.MOE_BF16)
    assert call(None) == -1
    assert call(P, h=0) == -1 and call(P, out=0) == -1
    assert call(P, h=0x1004) == -5
    assert call(smoe.Problem(16, 64, 128, 4, 5)) == -2
    assert call(smoe.Problem(16, 64, 128, 4, 2, smoe.MOE_F32, smoe.MOE_BF16)) == -3
    big = smoe.Problem(4096, 2880, 2880, 32, 4)   # the gpt-oss-20b layer at prefill: ~285 MB of workspace
    assert smoe.moe_workspace_bytes(big) > smoe.MOE_NOALLOC_SCRATCH_BYTES
    assert call(big) == -9
    assert "scratch" in smoe.moe_status_string(-9)
    assert call(smoe.Problem(0, 64, 128, 4, 2), h=0, out=0) == 0
