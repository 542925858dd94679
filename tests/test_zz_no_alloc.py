"""moe_forward_noalloc (the layer on the library's static per-GPU scratch, for
callers that cannot allocate) against moe_forward on the same inputs: outputs
and routing tables bitwise equal, on two calls in a row with the second one
smaller, so the second runs on scratch that still holds the first call's
tables and intermediates.  Both calls' outputs are filled with 0xFF bytes
first; moe_forward gets a freshly poisoned workspace."""
import numpy as np
import pytest
import torch

import sparse_mixture_experts_token_amd as smoe
import synth
from gpu_util import check_canaries, device_weights, poisoned, problem, routing_outputs, run, to_dev

pytestmark = pytest.mark.gpu


def _noalloc(prob, w, h):
    T, E, k, H = prob.T, prob.E, prob.k, prob.H
    out = poisoned((T, H), h.dtype, 0xFF, h.device)
    r = routing_outputs(T, E, k, h.device)
    smoe.moe_forward_noalloc(prob, w, h, out, routing=r)
    torch.cuda.synchronize()
    check_canaries()
    res = {n: t.cpu().numpy() for n, t in r.items()}
    res["out_raw"] = out.cpu()
    return res


MXFP4_SMALL = synth.Config(106, "mxfp4-small", T=200, H=128, I=256, E=9, k=2, act="bf16", expert="mxfp4")
CASES = [(2, (512, 64)),             # gpt-oss-20b layer: prefill kernels, then the fused decode path
         (MXFP4_SMALL, (200, 50)),   # MXFP4 experts, ragged
         (1, (64, 17))]              # fp32 fixture


@pytest.mark.parametrize("key,Ts", CASES, ids=["gpt-oss-20b-512-then-64", "mxfp4-200-then-50", "fixture-fp32-64-then-17"])
def test_noalloc_matches_moe_forward_on_two_calls(key, Ts):
    L = synth.make_layer(key)
    st = L.stacked()
    c = L.cfg
    w = device_weights(L, st)
    for T in Ts:
        assert T <= L.T
        prob = problem(c, T)
        assert smoe.moe_workspace_bytes(prob) <= smoe.MOE_NOALLOC_SCRATCH_BYTES
        h = to_dev(L.h[:T], c.act)
        want = run(prob, w, h, c.act)
        got = _noalloc(prob, w, h)
        assert torch.equal(got["out_raw"].view(torch.uint8), want["out_raw"].view(torch.uint8)), f"T={T}: out differs"
        for n in ("logits", "topk_idx", "topk_w", "expert_offsets", "perm_src"):
            np.testing.assert_array_equal(got[n].view(np.uint32), want[n].view(np.uint32), err_msg=f"T={T}: {n}")


def test_noalloc_rejects_problems_beyond_the_scratch():
    L = synth.make_layer(2, T=64)
    st = L.stacked()
    w = device_weights(L, st)
    big = smoe.Problem(4096, 2880, 2880, 32, 4)
    h = torch.zeros((4096, 2880), dtype=torch.bfloat16, device="cuda")
    out = torch.full((4096, 2880), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(smoe.MoeError) as ei:
        smoe.moe_forward_noalloc(big, w, h, out)
    assert ei.value.status == -9
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
