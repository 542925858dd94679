"""fp64 CPU reference of the sparse mixture-of-experts feed-forward layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link
or execute anything in this package; only ``tests/``, the smoke check in
``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` use it.  It
shares no code with the HIP library: the two meet only in the seeded inputs of
``synth``, which carry none of the layer's arithmetic.

It is plain and slow on purpose: NumPy in float64 on the exact values of the
stored inputs (bf16 and fp32 widen exactly; MXFP4 decodes exactly), with no
blocking, fusion or reordering beyond the definitions it follows.

Sources (web pages; cited by title and section):

* "gpt-oss-40b-64a8-init" (LLM-surgery model page), section 2 "Mathematical
  Foundation: Silent Init", Proof: the layer
  ``FFN(h) = sum_{i in top-k(s)} p_i(h) E_i(h)`` with router logits
  ``s_i = W_r[i].h + b_r[i]`` and softmax taken over the selected set only;
  the M-fold expansion and why it leaves the output unchanged.  Section 3
  "Combinatorial Routing Analysis", Per-Layer table: the C(E, k) counts.
  Section 5.2: original experts keep indices 0..E-1, copies follow.
* "gpt-oss 20B" field guide, cutaway 03 "Sparse Mixture of Experts": SwiGLU
  experts, top four of 32, the selected scores normalised, weighted sum.
  Cutaway 04 "One decoder block": RMSNorm before the MoE sublayer, whose
  output is added back to the residual stream.
* "openai/gpt-oss-20b" fixture comparison page, Preserved properties and
  Config changes tables: ``hidden_act = silu``; the fixture shape.
* "gpt-oss-20b and gpt-oss-120b" explainer, "Two attention savings, and a
  sink": the learned per-head sink in the attention normalisation and its
  worked example.  "Four-bit expert weights": MXFP4
  groups share a scale, 4.25 bits per parameter, decoded exactly.  The element
  and scale encodings (E2M1, E8M0, 32-element groups) are those of the OCP
  Microscaling Formats (MX) v1.0 specification.

Parity status per function is listed in each module's header.
"""
from .mxfp4 import e2m1_value, e8m0_value, mxfp4_dequant, mxfp4_bits_per_param
from .moe import (
    widen,
    router_logits,
    select_topk,
    topk_gap,
    selected_softmax,
    silu,
    swiglu_expert,
    moe_forward,
    moe_forward_per_token,
    routing_metadata,
    expand_silent,
    expand_rows,
    LayerWeights,
)
from .block import rms_norm, block_forward, block_forward_per_token
from .attention import sink_softmax, attn_sink_decode
from .backward import silu_grad, moe_backward

__all__ = [
    "e2m1_value", "e8m0_value", "mxfp4_dequant", "mxfp4_bits_per_param",
    "widen", "router_logits", "select_topk", "topk_gap", "selected_softmax",
    "silu", "swiglu_expert", "moe_forward", "moe_forward_per_token",
    "routing_metadata", "expand_silent", "expand_rows", "LayerWeights",
    "rms_norm", "block_forward", "block_forward_per_token",
    "sink_softmax", "attn_sink_decode",
    "silu_grad", "moe_backward",
]
