"""Seeded synthetic inputs for the sparse mixture-of-experts feed-forward layer.

This module is the one piece that both sides of the parity check share: the
fp64 reference (``oracle/``) and the HIP library are fed the same arrays from
here.  It holds none of the layer's arithmetic (no router, no top-k, no
softmax, no expert network, no dequantisation).  It only draws numbers and
stores them in the layer's input formats:

* activations and router parameters: fp32, or bf16 kept as raw ``uint16`` bits
  (rounded once from an fp32 draw, round-to-nearest-even);
* expert weights: the same, or MXFP4 (OCP Microscaling v1.0: E2M1 elements,
  32-element groups along the input dimension, one E8M0 scale byte per group),
  packed two elements per byte, element ``2j`` in the low nibble of byte ``j``.

Streams: every tensor (and every expert of a per-expert tensor) has its own
``numpy`` PCG64 stream, seeded from ``SeedSequence([20261203, cid, tensor_id,
index])``.  Per-expert streams keep generation parallel and memory-bounded and
let a checker draw only the experts it needs.

Workloads (``CONFIGS``) follow the shapes of the pages: the tiny two-layer test
fixture of gpt-oss-20b (hidden 64, intermediate 128, 4 experts, top-2), the
gpt-oss-20b MoE layer (hidden and intermediate 2,880, 32 experts, top-4), an
independently drawn layer of the 64a8 shape (64 experts, top-8), a
gpt-oss-120b-shaped layer (128 experts, top-4) with MXFP4 experts and a skewed
router bias, and the 248-row top-20 layer of
gpt-oss-220a20b with MXFP4 experts.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

ROOT_SEED = 20261203

# tensor ids of the per-tensor streams
TID_H, TID_WR, TID_BR, TID_GATE, TID_UP, TID_DOWN, TID_HOT, TID_ROWSCALE, TID_NORM, TID_ATTN, TID_DOUT = range(11)


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    T: int            # prefill tokens
    H: int            # hidden_size
    I: int            # intermediate_size
    E: int            # num_local_experts
    k: int            # num_experts_per_tok
    act: str          # "f32" | "bf16": h, out, router weight and bias
    expert: str       # "f32" | "bf16" | "mxfp4"
    router_std: float = 0.02
    bias_std: float = 0.01
    expert_std: float = 0.02
    T_decode: int = 0  # decode tokens (first rows of the prefill h); 0 = none
    hot: int = 0       # number of hot experts (router-bias skew); 0 = none
    hot_beta: float = 0.0  # bias added to the hot experts' router rows


# Router-bias offset for the skewed 128-expert layer.  It was found by
# bisection (tests/golden/find_c4_beta.py) so that the 8 hot experts receive
# half of the T*k routing assignments after the bias is rounded to bf16; the
# share itself is re-checked by the CPU test suite.
C4_HOT_BETA = 1.576

CONFIGS = {
    1: Config(1, "fixture-64h-128i-4e-top2-f32", T=64, H=64, I=128, E=4, k=2,
              act="f32", expert="f32", bias_std=0.0),
    2: Config(2, "gpt-oss-20b-moe-32e-top4-bf16", T=4096, H=2880, I=2880, E=32, k=4,
              act="bf16", expert="bf16", T_decode=64),
    3: Config(3, "random-64a8-bf16", T=4096, H=2880, I=2880, E=64, k=8,
              act="bf16", expert="bf16"),
    4: Config(4, "gpt-oss-120b-moe-128e-top4-mxfp4-skewed", T=8192, H=2880, I=2880,
              E=128, k=4, act="bf16", expert="mxfp4", hot=8, hot_beta=C4_HOT_BETA),
    5: Config(5, "220a20b-moe-248e-top20-mxfp4", T=2048, H=2880, I=2880, E=248, k=20,
              act="bf16", expert="mxfp4", T_decode=32),
}


def rng_for(cid: int, tid: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, cid, tid, index])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the raw uint16 bits.
    Inputs are finite draws, so no NaN handling is needed."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
    return (b >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------
# MXFP4 encoder (generation side only; the reference keeps its own decoder)
# --------------------------------------------------------------------------

def _e2m1_code(v: np.ndarray) -> np.ndarray:
    """Nearest-even E2M1 code (4 bits incl. sign) of ``v``; magnitudes above 6
    saturate to 6.  The E2M1 grid is 0, .5, 1, 1.5 (step .5), 2, 3 (step 1),
    4, 6 (step 2); the code of magnitude ``q`` counts the grid points below it."""
    a = np.abs(v)
    q = np.where(a < 2.0, np.round(a * 2.0) * 0.5,
                 np.where(a < 4.0, np.round(a), 2.0 * np.round(a * 0.5)))
    q = np.minimum(q, 6.0)
    # grid position: 0,.5,1,1.5 -> 0..3 ; 2,3 -> 4,5 ; 4 -> 6 ; 6 -> 7
    code = np.where(q < 2.0, q * 2.0, np.where(q < 4.0, q + 2.0, np.where(q < 6.0, 6.0, 7.0)))
    code = code.astype(np.uint8)
    return code | np.where(v < 0, np.uint8(8), np.uint8(0))


def mxfp4_encode(x: np.ndarray):
    """Quantise an fp32 matrix ``[N, K]`` (K % 32 == 0) to MXFP4.

    Per group of 32 consecutive elements of a row, the shared E8M0 exponent is
    ``floor(log2(max|x|)) - 2`` (2 is the largest E2M1 exponent), stored as a
    byte with bias 127; elements are rounded to the nearest E2M1 value of
    ``x / 2**exponent``.  Returns ``(packed uint8 [N, K/2], scales uint8 [N, K/32])``.
    """
    N, K = x.shape
    assert K % 32 == 0
    g = np.ascontiguousarray(x, dtype=np.float32).reshape(N, K // 32, 32)
    amax = np.abs(g).max(axis=-1)
    _, ex = np.frexp(amax)               # amax = m * 2**ex, m in [0.5, 1)
    e = np.where(amax > 0, ex.astype(np.int32) - 1 - 2, -127)
    e = np.clip(e, -127, 127)
    v = np.ldexp(g, (-e)[..., None].astype(np.int32))
    codes = _e2m1_code(v).reshape(N, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << np.uint8(4))).astype(np.uint8)
    scales = (e + 127).astype(np.uint8)
    return packed, scales


# --------------------------------------------------------------------------
# Layer inputs
# --------------------------------------------------------------------------

def _store(x32: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if fmt == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(fmt)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


@dataclass
class Layer:
    """Inputs of one MoE layer in storage format.

    ``h`` is ``[T, H]``; ``w_router`` ``[E, H]``; ``b_router`` ``[E]`` (all in
    the activation format).  Expert weights are produced per expert by
    ``expert(e)`` or stacked by ``stacked()``: gate/up ``[I, H]``, down
    ``[H, I]`` (``[out, in]``, row-major), or for MXFP4 packed ``[out, in/2]``
    with scales ``[out, in/32]``.
    """
    cfg: Config
    T: int
    h: np.ndarray
    w_router: np.ndarray
    b_router: np.ndarray
    hot_set: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))

    @property
    def E(self):
        return self.cfg.E

    @property
    def k(self):
        return self.cfg.k

    def expert(self, e: int) -> dict:
        c = self.cfg
        out = {}
        for name, tid, shape in (("gate", TID_GATE, (c.I, c.H)),
                                 ("up", TID_UP, (c.I, c.H)),
                                 ("down", TID_DOWN, (c.H, c.I))):
            x = rng_for(c.cid, tid, e).standard_normal(shape, dtype=np.float32)
            x *= np.float32(c.expert_std)
            if c.expert == "mxfp4":
                out[name], out["s_" + name] = mxfp4_encode(x)
            else:
                out[name] = _store(x, c.expert)
        return out

    def stacked(self, threads: int | None = None) -> dict:
        """All experts' weights stacked along a leading expert axis."""
        c = self.cfg
        first = self.expert(0)
        arrs = {n: np.empty((c.E,) + a.shape, a.dtype) for n, a in first.items()}
        for n, a in first.items():
            arrs[n][0] = a

        def fill(e):
            for n, a in self.expert(e).items():
                arrs[n][e] = a

        with ThreadPoolExecutor(threads or _threads()) as ex:
            list(ex.map(fill, range(1, c.E)))
        return arrs


def make_layer(key, T: int | None = None, hot_beta: float | None = None) -> Layer:
    """Inputs of workload ``key`` (a key of ``CONFIGS``, or a ``Config`` for
    an extra shape) with the first ``T`` tokens (default: the workload's
    prefill T).  ``hot_beta`` overrides the hot experts' router-bias offset
    (used only to choose that offset)."""
    c = key if isinstance(key, Config) else CONFIGS[key]
    beta = c.hot_beta if hot_beta is None else hot_beta
    T = c.T if T is None else T
    if T > c.T:
        raise ValueError(f"T={T} exceeds the workload's {c.T} tokens")
    h32 = rng_for(c.cid, TID_H).standard_normal((c.T, c.H), dtype=np.float32)[:T]
    wr32 = rng_for(c.cid, TID_WR).standard_normal((c.E, c.H), dtype=np.float32) * np.float32(c.router_std)
    br32 = rng_for(c.cid, TID_BR).standard_normal(c.E, dtype=np.float32) * np.float32(c.bias_std)
    hot = np.zeros(0, np.int64)
    if c.hot:
        hot = np.sort(rng_for(c.cid, TID_HOT).choice(c.E, size=c.hot, replace=False))
        br32[hot] += np.float32(beta)
    return Layer(cfg=c, T=T, h=_store(h32, c.act), w_router=_store(wr32, c.act),
                 b_router=_store(br32, c.act), hot_set=hot)


def block_inputs(layer: Layer) -> tuple[np.ndarray, np.ndarray]:
    """Inputs of the pre-normalised block built on ``layer``, in the
    activation format: the residual stream ``x`` (``h`` with each row scaled
    by a seeded factor drawn log-uniformly from [0.5, 2], so rows differ in
    mean square) and the norm gain ``g`` ``[H]`` drawn uniformly from
    [0.5, 1.5]."""
    c = layer.cfg
    scale = np.exp2(rng_for(c.cid, TID_ROWSCALE).uniform(-1.0, 1.0, c.T).astype(np.float32))[:layer.T]
    if c.act == "bf16":
        h32 = (np.asarray(layer.h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    else:
        h32 = np.asarray(layer.h, dtype=np.float32)
    g32 = rng_for(c.cid, TID_NORM).uniform(0.5, 1.5, c.H).astype(np.float32)
    return _store(h32 * scale[:, None], c.act), _store(g32, c.act)


def attn_inputs(seed: int, B: int, Hq: int, Hkv: int, Tk: int, D: int) -> dict:
    """Seeded decode-attention inputs in bf16 bits: q [B, Hq, D], k and v
    [B, Hkv, Tk, D] with N(0, 1) entries, sinks [Hq] ~ N(0, 1), and per-sequence
    lengths [B] (int32) drawn uniformly from 1..Tk, the first sequence full and,
    for B > 2, the second of length 1."""
    r = rng_for(seed, TID_ATTN)
    out = {"q": f32_to_bf16_bits(r.standard_normal((B, Hq, D), dtype=np.float32)),
           "k": f32_to_bf16_bits(r.standard_normal((B, Hkv, Tk, D), dtype=np.float32)),
           "v": f32_to_bf16_bits(r.standard_normal((B, Hkv, Tk, D), dtype=np.float32)),
           "sinks": f32_to_bf16_bits(r.standard_normal(Hq, dtype=np.float32))}
    lens = r.integers(1, Tk + 1, size=B).astype(np.int32)
    if B > 0:
        lens[0] = Tk
    if B > 2:
        lens[1] = 1
    out["lens"] = lens
    return out


def grad_output(seed: int, T: int, H: int) -> np.ndarray:
    """Seeded upstream gradient of the layer output: [T, H] N(0, 1) in bf16 bits."""
    return f32_to_bf16_bits(rng_for(seed, TID_DOUT).standard_normal((T, H), dtype=np.float32))


def decode_T(key: int) -> int:
    return CONFIGS[key].T_decode
