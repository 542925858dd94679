"""Python binding of libmoe, the MI355X (gfx950) sparse mixture-of-experts
feed-forward layer.

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libmoe.so`` (built in place by ``sparse_mixture_experts_token_amd.build``).
PyTorch supplies device memory and the current HIP stream.  If the library is
missing, ``load()`` raises: there is no fallback implementation.

The functions mirror the C entry points of ``include/moe.h``:

* ``moe_workspace_bytes(problem)``
* ``moe_forward(problem, weights, h, out, routing=None, workspace=None)``
* ``moe_forward_noalloc(problem, weights, h, out, routing=None)``
* ``moe_block_workspace_bytes(problem)``
* ``moe_block_forward(problem, weights, norm_weight, eps, x, out, routing=None, workspace=None)``
* ``moe_backward_workspace_bytes(problem)``
* ``moe_backward(problem, weights, h, d_out, routing, d_h=None, grads=None, trainable=None, workspace=None)``
* ``moe_attn_workspace_bytes(problem)``
* ``moe_attn_sink_decode(problem, q, k_cache, v_cache, sinks, lens, out, workspace=None)``
* ``moe_expand_silent(base, src, M, dst)``
* ``moe_expand_copies(base, src, copy_of, dst)``
* ``moe_status_string(status)``
* ``moe_profile_begin(max_calls)`` / ``moe_profile_begin_mask(max_calls, mask)`` / ``moe_profile_end()``

``problem`` is a ``Problem``; ``weights`` / ``src`` / ``dst`` are dicts of
device tensors keyed ``w_router, b_router, w_gate, w_up, w_down`` (and
``s_gate, s_up, s_down`` for MXFP4); ``routing`` is a dict with any of
``logits, topk_idx, topk_w, expert_offsets, perm_src``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_BF16, MOE_MXFP4 = 0, 1, 2
MOE_NUM_STAGES = 5
STATUS = {0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_DTYPE",
          -4: "MOE_ERR_WORKSPACE", -5: "MOE_ERR_ALIGN", -6: "MOE_ERR_HIP", -7: "MOE_ERR_STATE",
          -8: "MOE_ERR_DISABLED", -9: "MOE_ERR_SCRATCH"}
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20
EXPORTED = ("moe_workspace_bytes", "moe_forward", "moe_forward_noalloc", "moe_block_workspace_bytes", "moe_block_forward",
            "moe_backward_workspace_bytes", "moe_backward", "moe_attn_workspace_bytes", "moe_attn_sink_decode", "moe_expand_silent", "moe_expand_copies", "moe_mxfp4_decode", "moe_status_string",
            "moe_profile_begin", "moe_profile_begin_mask", "moe_profile_end", "moe_stage_name")
MOE_PROFILE_ALL = (1 << (MOE_NUM_STAGES + 1)) - 1


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class _Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("act_dtype", ctypes.c_int32), ("expert_dtype", ctypes.c_int32)]


_WEIGHT_FIELDS = ("w_router", "b_router", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")
_ROUTING_FIELDS = ("logits", "topk_idx", "topk_w", "expert_offsets", "perm_src")


_GRAD_FIELDS = ("d_w_router", "d_b_router", "d_w_gate", "d_w_up", "d_w_down")


class _Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _GRAD_FIELDS]


class _AttnProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("Tk", ctypes.c_int32),
                ("D", ctypes.c_int32), ("window", ctypes.c_int32), ("scale", ctypes.c_float)]


@dataclass
class AttnProblem:
    """Sizes of decode attention with sinks (``moe_attn_problem``)."""
    B: int
    Hq: int
    Hkv: int
    Tk: int
    D: int
    window: int = 0
    scale: float = 0.0  # 0: 1/sqrt(D)

    def _c(self) -> _AttnProblem:
        sc = self.scale if self.scale else 1.0 / float(self.D) ** 0.5
        return _AttnProblem(self.B, self.Hq, self.Hkv, self.Tk, self.D, self.window, sc)


class _Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _WEIGHT_FIELDS]


class _Routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _ROUTING_FIELDS]


@dataclass(frozen=True)
class Problem:
    """Sizes and formats of one layer call (see ``moe_problem`` in moe.h)."""
    T: int
    H: int
    I: int
    E: int
    k: int
    act_dtype: int = MOE_BF16
    expert_dtype: int = MOE_BF16

    def _c(self) -> _Problem:
        return _Problem(self.T, self.H, self.I, self.E, self.k, self.act_dtype, self.expert_dtype)


_lib = None


def load() -> ctypes.CDLL:
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sparse_mixture_experts_token_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.moe_workspace_bytes.argtypes = [ctypes.POINTER(_Problem)]
    lib.moe_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_forward.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_Weights), ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.POINTER(_Routing), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.moe_forward.restype = ctypes.c_int
    lib.moe_forward_noalloc.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_Weights), ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.POINTER(_Routing), ctypes.c_void_p]
    lib.moe_forward_noalloc.restype = ctypes.c_int
    lib.moe_block_workspace_bytes.argtypes = [ctypes.POINTER(_Problem)]
    lib.moe_block_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_block_forward.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_Weights), ctypes.c_void_p,
                                      ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.moe_block_forward.restype = ctypes.c_int
    lib.moe_backward_workspace_bytes.argtypes = [ctypes.POINTER(_Problem)]
    lib.moe_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_backward.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_Weights), ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.POINTER(_Routing), ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.POINTER(_Grads), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.moe_backward.restype = ctypes.c_int
    lib.moe_attn_workspace_bytes.argtypes = [ctypes.POINTER(_AttnProblem)]
    lib.moe_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_attn_sink_decode.argtypes = [ctypes.POINTER(_AttnProblem)] + [ctypes.c_void_p] * 7 + [
        ctypes.c_size_t, ctypes.c_void_p]
    lib.moe_attn_sink_decode.restype = ctypes.c_int
    lib.moe_expand_silent.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_Weights), ctypes.c_int32,
                                      ctypes.POINTER(_Weights), ctypes.c_void_p]
    lib.moe_expand_silent.restype = ctypes.c_int
    lib.moe_expand_copies.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_Weights),
                                      ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, ctypes.POINTER(_Weights),
                                      ctypes.c_void_p]
    lib.moe_expand_copies.restype = ctypes.c_int
    lib.moe_mxfp4_decode.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                     ctypes.c_void_p]
    lib.moe_mxfp4_decode.restype = ctypes.c_int
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_profile_begin.argtypes = [ctypes.c_int32]
    lib.moe_profile_begin.restype = ctypes.c_int
    lib.moe_profile_begin_mask.argtypes = [ctypes.c_int32, ctypes.c_uint32]
    lib.moe_profile_begin_mask.restype = ctypes.c_int
    lib.moe_profile_end.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32)]
    lib.moe_profile_end.restype = ctypes.c_int
    lib.moe_stage_name.argtypes = [ctypes.c_int]
    lib.moe_stage_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        raise MoeError(status, moe_status_string(status))


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensors passed to libmoe must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _weights(d: dict) -> _Weights:
    unknown = set(d) - set(_WEIGHT_FIELDS)
    if unknown:
        raise KeyError(f"unknown weight fields {sorted(unknown)}")
    return _Weights(*[_ptr(d.get(n)) for n in _WEIGHT_FIELDS])


def moe_status_string(status: int) -> str:
    return load().moe_status_string(status).decode()


def moe_stage_name(stage: int) -> str:
    return load().moe_stage_name(stage).decode()


def moe_workspace_bytes(problem: Problem) -> int:
    p = problem._c()
    return int(load().moe_workspace_bytes(ctypes.byref(p)))


def _routing(routing: dict | None):
    if routing is None:
        return None
    unknown = set(routing) - set(_ROUTING_FIELDS)
    if unknown:
        raise KeyError(f"unknown routing fields {sorted(unknown)}")
    return _Routing(*[_ptr(routing.get(n)) for n in _ROUTING_FIELDS])


def _workspace(size_fn, p, like, workspace, workspace_bytes):
    if workspace is None:
        nbytes = int(size_fn(ctypes.byref(p)))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=like.device if like is not None else "cuda")
        return workspace, nbytes
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    return workspace, workspace_bytes


def moe_forward(problem: Problem, weights: dict, h, out, routing: dict | None = None, workspace=None,
                workspace_bytes: int | None = None, stream=None) -> None:
    """Enqueue the layer on ``stream`` (default: torch's current stream).
    ``workspace`` defaults to a fresh torch allocation of the required size."""
    lib = load()
    p = problem._c()
    w = _weights(weights)
    r = _routing(routing)
    workspace, workspace_bytes = _workspace(lib.moe_workspace_bytes, p, h, workspace, workspace_bytes)
    st = lib.moe_forward(ctypes.byref(p), ctypes.byref(w), _ptr(h), _ptr(out),
                         ctypes.byref(r) if r is not None else None, _ptr(workspace), int(workspace_bytes),
                         _stream(stream))
    _check(st)


def moe_forward_noalloc(problem: Problem, weights: dict, h, out, routing: dict | None = None, stream=None) -> None:
    """``moe_forward`` on the library's static per-GPU scratch (no workspace,
    nothing allocated by the call); problems needing more than
    ``MOE_NOALLOC_SCRATCH_BYTES`` of workspace raise MOE_ERR_SCRATCH.  Calls
    that overlap on one GPU share the scratch and race."""
    lib = load()
    p = problem._c()
    w = _weights(weights)
    r = _routing(routing)
    _check(lib.moe_forward_noalloc(ctypes.byref(p), ctypes.byref(w), _ptr(h), _ptr(out),
                                   ctypes.byref(r) if r is not None else None, _stream(stream)))


def moe_block_workspace_bytes(problem: Problem) -> int:
    p = problem._c()
    return int(load().moe_block_workspace_bytes(ctypes.byref(p)))


def moe_block_forward(problem: Problem, weights: dict, norm_weight, eps: float, x, out,
                      routing: dict | None = None, workspace=None, workspace_bytes: int | None = None,
                      stream=None) -> None:
    """Enqueue ``out = x + MoE(RMSNorm(x))`` on ``stream`` (default: torch's
    current stream); ``norm_weight`` is the [H] gain in the activation format."""
    lib = load()
    p = problem._c()
    w = _weights(weights)
    r = _routing(routing)
    workspace, workspace_bytes = _workspace(lib.moe_block_workspace_bytes, p, x, workspace, workspace_bytes)
    st = lib.moe_block_forward(ctypes.byref(p), ctypes.byref(w), _ptr(norm_weight), float(eps), _ptr(x), _ptr(out),
                               ctypes.byref(r) if r is not None else None, _ptr(workspace), int(workspace_bytes),
                               _stream(stream))
    _check(st)


def moe_backward_workspace_bytes(problem: Problem) -> int:
    p = problem._c()
    return int(load().moe_backward_workspace_bytes(ctypes.byref(p)))


def moe_backward(problem: Problem, weights: dict, h, d_out, routing: dict, d_h=None, grads: dict | None = None,
                 trainable=None, workspace=None, workspace_bytes: int | None = None, stream=None) -> None:
    """Enqueue the layer's gradients on ``stream`` (default: torch's current
    stream).  ``routing`` holds the forward's ``topk_idx``, ``topk_w``,
    ``expert_offsets`` and ``perm_src``; ``grads`` maps ``d_w_router``,
    ``d_b_router``, ``d_w_gate``, ``d_w_up``, ``d_w_down`` to fp32 tensors
    (missing: not computed); ``trainable`` is an [E] uint8 tensor or None."""
    lib = load()
    p = problem._c()
    w = _weights(weights)
    r = _routing(routing)
    grads = grads or {}
    unknown = set(grads) - set(_GRAD_FIELDS)
    if unknown:
        raise KeyError(f"unknown gradient fields {sorted(unknown)}")
    g = _Grads(*[_ptr(grads.get(n)) for n in _GRAD_FIELDS])
    workspace, workspace_bytes = _workspace(lib.moe_backward_workspace_bytes, p, h, workspace, workspace_bytes)
    _check(lib.moe_backward(ctypes.byref(p), ctypes.byref(w), _ptr(h), _ptr(d_out),
                            ctypes.byref(r) if r is not None else None, _ptr(trainable), _ptr(d_h), ctypes.byref(g),
                            _ptr(workspace), int(workspace_bytes), _stream(stream)))


def moe_attn_workspace_bytes(problem: AttnProblem) -> int:
    p = problem._c()
    return int(load().moe_attn_workspace_bytes(ctypes.byref(p)))


def moe_attn_sink_decode(problem: AttnProblem, q, k_cache, v_cache, sinks, lens, out, workspace=None,
                         workspace_bytes: int | None = None, stream=None) -> None:
    """Enqueue decode attention with sinks on ``stream`` (default: torch's
    current stream); ``lens`` may be None (every sequence has Tk keys);
    ``workspace`` defaults to a fresh torch allocation of the required size."""
    lib = load()
    p = problem._c()
    workspace, workspace_bytes = _workspace(lib.moe_attn_workspace_bytes, p, q, workspace, workspace_bytes)
    _check(lib.moe_attn_sink_decode(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(sinks),
                                    _ptr(lens), _ptr(out), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def moe_expand_silent(base: Problem, src: dict, M: int, dst: dict, stream=None) -> None:
    p = base._c()
    _check(load().moe_expand_silent(ctypes.byref(p), ctypes.byref(_weights(src)), int(M),
                                    ctypes.byref(_weights(dst)), _stream(stream)))


def moe_expand_copies(base: Problem, src: dict, copy_of, dst: dict, stream=None) -> None:
    """dst row j = src row copy_of[j] for every per-expert tensor; ``copy_of``
    is a host sequence of original expert ids (its length is the new E)."""
    ids = [int(x) for x in copy_of]
    arr = (ctypes.c_int32 * max(len(ids), 1))(*ids)
    p = base._c()
    _check(load().moe_expand_copies(ctypes.byref(p), ctypes.byref(_weights(src)), arr, len(ids),
                                    ctypes.byref(_weights(dst)), _stream(stream)))


def moe_mxfp4_decode(packed, scales, out_bf16, stream=None) -> None:
    """Decode an MXFP4 tensor (uint8 codes, uint8 scales) into ``out_bf16``
    (``packed.numel() * 2`` bfloat16 elements)."""
    n_groups = packed.numel() // 16
    if scales.numel() != n_groups or out_bf16.numel() != n_groups * 32:
        raise ValueError("packed, scales and out_bf16 sizes do not match")
    _check(load().moe_mxfp4_decode(_ptr(packed), _ptr(scales), n_groups, _ptr(out_bf16), _stream(stream)))


def moe_profile_begin(max_calls: int) -> None:
    _check(load().moe_profile_begin(int(max_calls)))


def moe_profile_begin_mask(max_calls: int, boundary_mask: int) -> None:
    """Record only the stage boundaries in ``boundary_mask`` (bit i: the event
    before stage i; bit MOE_NUM_STAGES: the one after the last)."""
    _check(load().moe_profile_begin_mask(int(max_calls), int(boundary_mask)))


def moe_profile_end():
    """Returns ``(stage_ms, calls)``: summed per-stage milliseconds and the
    number of recorded calls."""
    arr = (ctypes.c_float * MOE_NUM_STAGES)()
    n = ctypes.c_int32(0)
    _check(load().moe_profile_end(arr, ctypes.byref(n)))
    return [float(x) for x in arr], int(n.value)


# ---------------------------------------------------------------- helpers --

def expanded_shapes(problem: Problem, M: int) -> dict:
    """Shapes and dtypes of the tensors of the M-fold expanded layer."""
    E2 = problem.E * M
    return weight_shapes(Problem(problem.T, problem.H, problem.I, E2, problem.k * M, problem.act_dtype,
                                 problem.expert_dtype))


def weight_shapes(problem: Problem) -> dict:
    """``{name: (shape, torch dtype)}`` of the weight tensors of ``problem``."""
    adt = torch.float32 if problem.act_dtype == MOE_F32 else torch.bfloat16
    E, H, I = problem.E, problem.H, problem.I
    out = {"w_router": ((E, H), adt), "b_router": ((E,), adt)}
    if problem.expert_dtype == MOE_MXFP4:
        out.update(w_gate=((E, I, H // 2), torch.uint8), w_up=((E, I, H // 2), torch.uint8),
                   w_down=((E, H, I // 2), torch.uint8), s_gate=((E, I, H // 32), torch.uint8),
                   s_up=((E, I, H // 32), torch.uint8), s_down=((E, H, I // 32), torch.uint8))
    else:
        edt = torch.float32 if problem.expert_dtype == MOE_F32 else torch.bfloat16
        out.update(w_gate=((E, I, H), edt), w_up=((E, I, H), edt), w_down=((E, H, I), edt))
    return out
