"""Python binding of libspava (approximate-attention prefill on gfx950).

Argument marshalling only: every step runs in the HIP library
(``libspava.so``, built in-tree by ``sequence_approximate_attention_amd.build``).
PyTorch supplies device memory and the current stream.  The functions carry
the C names of ``include/spava.h``; ``prefill`` chains the four calls.

Layouts (rows = tokens [anchor | V blocks of L | n_q query tokens]):
  q [N, Hq, d]; k, v [N, Hkv, d]; kp, vp [Hkv, V, lp, d]; o [N, Hq, d];
  lse [Hq, N]; scores [V, Hkv, L] f32; idx [V, Hkv, lp] i32;
  o_part [V+1, n_q, Hq, d] f32; lse_part [V+1, Hq, n_q] f32.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# SPAVA_LIBRARY names another build of the same library to load instead of
# the in-tree one (the host-sanitizer build of the CPU tests).
LIB_PATH = os.environ.get("SPAVA_LIBRARY") or os.path.join(HERE, "libspava.so")

SPAVA_OK, SPAVA_EINVAL, SPAVA_EUNSUPPORTED, SPAVA_EWORKSPACE, SPAVA_ELAUNCH = range(5)
SPAVA_BF16, SPAVA_F32 = 0, 1
SPAVA_PHASE_ALL, SPAVA_PHASE_LOCAL, SPAVA_PHASE_PASSING = 0, 1, 2
EXPORTS = ("spava_version", "spava_last_error", "spava_plan_check", "spava_score_topk_ws_bytes",
           "spava_score_topk", "spava_gather_passing", "spava_attn_fwd",
           "spava_lse_merge", "spava_score_topk_context_ws_bytes", "spava_score_topk_context",
           "spava_kv_overlap", "spava_attn_fwd_phase", "spava_score_topk_from_partials",
           "spava_score_topk_noalloc")
SPAVA_NOALLOC_SCRATCH_BYTES = 64 << 20


class SpavaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"spava error {code}: {msg}")
        self.code = code


class spava_plan(ctypes.Structure):
    _fields_ = [("n_anchor", ctypes.c_int32), ("n_hosts", ctypes.c_int32),
                ("host_len", ctypes.c_int32), ("n_query", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("lp", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("q_stride_tok", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
                ("kv_stride_tok", ctypes.c_int64), ("kv_stride_head", ctypes.c_int64)]


_lib = None


def lib():
    """Load libspava.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sequence_approximate_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(spava_plan)
        vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
        L.spava_version.restype = ctypes.c_int
        L.spava_last_error.restype = ctypes.c_char_p
        L.spava_plan_check.argtypes = [P]
        L.spava_score_topk_ws_bytes.argtypes = [P]
        L.spava_score_topk_ws_bytes.restype = sz
        L.spava_score_topk.argtypes = [P, vp, vp, vp, vp, vp, sz, vp]
        L.spava_score_topk_noalloc.argtypes = [P, vp, vp, vp, vp, vp]
        L.spava_score_topk_context_ws_bytes.argtypes = [P]
        L.spava_score_topk_context_ws_bytes.restype = sz
        L.spava_score_topk_context.argtypes = [P, vp, vp, vp, vp, vp, sz, vp]
        L.spava_kv_overlap.argtypes = [i32, i32, vp, vp, vp, vp]
        L.spava_attn_fwd_phase.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.spava_score_topk_from_partials.argtypes = [P, vp, vp, vp, vp, vp, vp]
        L.spava_gather_passing.argtypes = [P, vp, vp, vp, vp, vp, vp]
        L.spava_attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.spava_lse_merge.argtypes = [i32, i32, i32, i32, vp, vp, vp, i64, vp, i64, i32, vp]
        _lib = L
    return _lib


@dataclass(frozen=True)
class Plan:
    """One layer's split and head geometry (mirrors ``spava_plan``).  Strides
    are in elements; 0 means the dense layout."""
    n_anchor: int
    n_hosts: int
    host_len: int
    n_query: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    lp: int
    dtype: int = SPAVA_BF16
    scale: float = 0.0
    q_stride_tok: int = 0
    q_stride_head: int = 0
    kv_stride_tok: int = 0
    kv_stride_head: int = 0

    @property
    def n_tokens(self) -> int:
        return self.n_anchor + self.n_hosts * self.host_len + self.n_query

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == SPAVA_BF16 else torch.float32

    def c(self) -> spava_plan:
        return spava_plan(self.n_anchor, self.n_hosts, self.host_len, self.n_query,
                          self.n_q_heads, self.n_kv_heads, self.head_dim, self.lp,
                          self.dtype, float(self.scale), self.q_stride_tok, self.q_stride_head,
                          self.kv_stride_tok, self.kv_stride_head)

    def q_strides(self):
        return (self.q_stride_tok or self.n_q_heads * self.head_dim, self.q_stride_head or self.head_dim, 1)

    def kv_strides(self):
        return (self.kv_stride_tok or self.n_kv_heads * self.head_dim, self.kv_stride_head or self.head_dim, 1)

    def with_strides(self, q, k, v) -> "Plan":
        """The plan with the element strides of the views q [N, Hq, d] and
        k, v [N, Hkv, d] (k and v must share theirs; channels contiguous)."""
        if tuple(k.stride()) != tuple(v.stride()):
            raise ValueError("k and v must have the same strides")
        if q.stride(2) != 1 or k.stride(2) != 1:
            raise ValueError("channels must be contiguous")
        return dataclasses.replace(self, q_stride_tok=q.stride(0), q_stride_head=q.stride(1),
                                   kv_stride_tok=k.stride(0), kv_stride_head=k.stride(1))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(rc: int):
    if rc != SPAVA_OK:
        raise SpavaError(rc, lib().spava_last_error().decode())


def _expect(t, shape, dtype, name, strides=None):
    """Device tensor of this shape and dtype, contiguous or (q, k, v) with the
    plan's strides."""
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if strides is not None:
        if t.numel() and tuple(t.stride()) != tuple(strides):
            raise ValueError(f"{name} has strides {tuple(t.stride())}, the plan says {tuple(strides)}")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _reach(t, n_elems, name):
    """Raise unless the n_elems elements from t's first element lie inside its
    storage (a strided output written through a plain pointer)."""
    end = (t.storage_offset() + n_elems) * t.element_size()
    if n_elems > 0 and end > t.untyped_storage().nbytes():
        raise ValueError(f"{name}: {n_elems} elements from its first element run past the end of its storage")


def spava_plan_check(plan: Plan) -> int:
    return lib().spava_plan_check(ctypes.byref(plan.c()))


def spava_score_topk_ws_bytes(plan: Plan) -> int:
    return lib().spava_score_topk_ws_bytes(ctypes.byref(plan.c()))


def spava_score_topk_context_ws_bytes(plan: Plan) -> int:
    return lib().spava_score_topk_context_ws_bytes(ctypes.byref(plan.c()))


def spava_score_topk(plan: Plan, q, k, scores, idx, ws, stream=None):
    p = plan
    _expect(q, (p.n_tokens, p.n_q_heads, p.head_dim), p.torch_dtype, "q", p.q_strides())
    _expect(k, (p.n_tokens, p.n_kv_heads, p.head_dim), p.torch_dtype, "k", p.kv_strides())
    _expect(scores, (p.n_hosts, p.n_kv_heads, p.host_len), torch.float32, "scores")
    _expect(idx, (p.n_hosts, p.n_kv_heads, p.lp), torch.int32, "idx")
    _check(lib().spava_score_topk(ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(scores), _ptr(idx),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def spava_score_topk_noalloc(plan: Plan, q, k, scores, idx, stream=None):
    """spava_score_topk with the library's static scratch in place of a
    workspace (no allocation; calls overlapping on one GPU race).  scores may
    be None."""
    p = plan
    _expect(q, (p.n_tokens, p.n_q_heads, p.head_dim), p.torch_dtype, "q", p.q_strides())
    _expect(k, (p.n_tokens, p.n_kv_heads, p.head_dim), p.torch_dtype, "k", p.kv_strides())
    _expect(scores, (p.n_hosts, p.n_kv_heads, p.host_len), torch.float32, "scores")
    _expect(idx, (p.n_hosts, p.n_kv_heads, p.lp), torch.int32, "idx")
    _check(lib().spava_score_topk_noalloc(ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(scores), _ptr(idx),
                                          _stream(stream)))


def spava_score_topk_context(plan: Plan, q, k, scores, idx, ws, stream=None):
    """Context-driven selection: the block's own tokens score its keys."""
    p = plan
    _expect(q, (p.n_tokens, p.n_q_heads, p.head_dim), p.torch_dtype, "q", p.q_strides())
    _expect(k, (p.n_tokens, p.n_kv_heads, p.head_dim), p.torch_dtype, "k", p.kv_strides())
    _expect(scores, (p.n_hosts, p.n_kv_heads, p.host_len), torch.float32, "scores")
    _expect(idx, (p.n_hosts, p.n_kv_heads, p.lp), torch.int32, "idx")
    _check(lib().spava_score_topk_context(ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(scores), _ptr(idx),
                                          _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def spava_kv_overlap(idx_a, idx_b, counts, stream=None):
    """idx_a, idx_b [..., lp] int32 (strictly ascending lists); counts [...]
    int32 receives the size of each pair's intersection (-1 if a list is not
    strictly ascending)."""
    if tuple(idx_a.shape) != tuple(idx_b.shape) or idx_a.dim() < 1:
        raise ValueError("idx_a and idx_b must have the same shape [..., lp]")
    lp = idx_a.shape[-1]
    _expect(idx_a, idx_a.shape, torch.int32, "idx_a")
    _expect(idx_b, idx_b.shape, torch.int32, "idx_b")
    _expect(counts, idx_a.shape[:-1], torch.int32, "counts")
    _check(lib().spava_kv_overlap(counts.numel(), lp, _ptr(idx_a), _ptr(idx_b), _ptr(counts),
                                  _stream(stream)))


def spava_gather_passing(plan: Plan, k, v, idx, kp, vp, stream=None):
    p = plan
    _expect(k, (p.n_tokens, p.n_kv_heads, p.head_dim), p.torch_dtype, "k", p.kv_strides())
    _expect(v, (p.n_tokens, p.n_kv_heads, p.head_dim), p.torch_dtype, "v", p.kv_strides())
    _expect(idx, (p.n_hosts, p.n_kv_heads, p.lp), torch.int32, "idx")
    _expect(kp, (p.n_kv_heads, p.n_hosts, p.lp, p.head_dim), p.torch_dtype, "kp")
    _expect(vp, (p.n_kv_heads, p.n_hosts, p.lp, p.head_dim), p.torch_dtype, "vp")
    _check(lib().spava_gather_passing(ctypes.byref(p.c()), _ptr(k), _ptr(v), _ptr(idx), _ptr(kp),
                                      _ptr(vp), _stream(stream)))


def spava_attn_fwd(plan: Plan, q, k, v, kp, vp, o, lse, o_part, lse_part, stream=None):
    spava_attn_fwd_phase(plan, SPAVA_PHASE_ALL, q, k, v, kp, vp, o, lse, o_part, lse_part, stream)


def spava_attn_fwd_phase(plan: Plan, phase: int, q, k, v, kp, vp, o, lse, o_part, lse_part, stream=None):
    """SPAVA_PHASE_LOCAL: anchor rows, host 0's context rows and the query
    partials; SPAVA_PHASE_PASSING: context rows of hosts 1..V-1;
    SPAVA_PHASE_ALL: everything."""
    p = plan
    N = p.n_tokens
    _expect(q, (N, p.n_q_heads, p.head_dim), p.torch_dtype, "q", p.q_strides())
    _expect(k, (N, p.n_kv_heads, p.head_dim), p.torch_dtype, "k", p.kv_strides())
    _expect(v, (N, p.n_kv_heads, p.head_dim), p.torch_dtype, "v", p.kv_strides())
    _expect(kp, (p.n_kv_heads, p.n_hosts, p.lp, p.head_dim), p.torch_dtype, "kp")
    _expect(vp, (p.n_kv_heads, p.n_hosts, p.lp, p.head_dim), p.torch_dtype, "vp")
    _expect(o, (N, p.n_q_heads, p.head_dim), p.torch_dtype, "o")
    _expect(lse, (p.n_q_heads, N), torch.float32, "lse")
    _expect(o_part, (p.n_hosts + 1, p.n_query, p.n_q_heads, p.head_dim), torch.float32, "o_part")
    _expect(lse_part, (p.n_hosts + 1, p.n_q_heads, p.n_query), torch.float32, "lse_part")
    _check(lib().spava_attn_fwd_phase(ctypes.byref(p.c()), phase, _ptr(q), _ptr(k), _ptr(v), _ptr(kp),
                                      _ptr(vp), _ptr(o), _ptr(lse), _ptr(o_part), _ptr(lse_part), _stream(stream)))


def spava_score_topk_from_partials(plan: Plan, q, k, lse_part, scores, idx, stream=None):
    """Scores and top-lp with the row normalisers taken from the query
    partials that spava_attn_fwd_phase(LOCAL) wrote."""
    p = plan
    _expect(q, (p.n_tokens, p.n_q_heads, p.head_dim), p.torch_dtype, "q", p.q_strides())
    _expect(k, (p.n_tokens, p.n_kv_heads, p.head_dim), p.torch_dtype, "k", p.kv_strides())
    _expect(lse_part, (p.n_hosts + 1, p.n_q_heads, p.n_query), torch.float32, "lse_part")
    _expect(scores, (p.n_hosts, p.n_kv_heads, p.host_len), torch.float32, "scores")
    _expect(idx, (p.n_hosts, p.n_kv_heads, p.lp), torch.int32, "idx")
    _check(lib().spava_score_topk_from_partials(ctypes.byref(p.c()), _ptr(q), _ptr(k), _ptr(lse_part),
                                                _ptr(scores), _ptr(idx), _stream(stream)))


def spava_lse_merge(o_part, lse_part, o, o_row_stride, lse, lse_head_stride, stream=None):
    """o_part [P, R, H, D] f32, lse_part [P, H, R] f32; o / lse are the first
    element of the strided outputs (views into larger tensors are fine)."""
    P, R, H, D = o_part.shape
    if tuple(lse_part.shape) != (P, H, R):
        raise ValueError("lse_part must be [P, H, R]")
    for t, n in ((o_part, "o_part"), (lse_part, "lse_part")):
        if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous float32 device tensor")
    if o.dtype not in (torch.bfloat16, torch.float32) or lse.dtype != torch.float32:
        raise ValueError("o must be bf16/f32 and lse f32")
    if not o.is_cuda or not lse.is_cuda:
        raise ValueError("o and lse must be device tensors")
    if R > 0:
        _reach(o, (R - 1) * int(o_row_stride) + H * D, "o")
        _reach(lse, (H - 1) * int(lse_head_stride) + R, "lse")
    out_dtype = SPAVA_BF16 if o.dtype == torch.bfloat16 else SPAVA_F32
    _check(lib().spava_lse_merge(P, R, H, D, _ptr(o_part), _ptr(lse_part), _ptr(o), int(o_row_stride),
                                 _ptr(lse), int(lse_head_stride), out_dtype, _stream(stream)))


@dataclass
class Buffers:
    """Device buffers of one prefill layer (allocated once, reusable)."""
    scores: torch.Tensor
    idx: torch.Tensor
    kp: torch.Tensor
    vp: torch.Tensor
    o: torch.Tensor
    lse: torch.Tensor
    o_part: torch.Tensor
    lse_part: torch.Tensor
    ws_score: torch.Tensor


def alloc_buffers(plan: Plan, device="cuda") -> Buffers:
    p = plan
    dt = p.torch_dtype
    N = p.n_tokens
    f32 = torch.float32
    return Buffers(
        scores=torch.empty((p.n_hosts, p.n_kv_heads, p.host_len), dtype=f32, device=device),
        idx=torch.empty((p.n_hosts, p.n_kv_heads, p.lp), dtype=torch.int32, device=device),
        kp=torch.empty((p.n_kv_heads, p.n_hosts, p.lp, p.head_dim), dtype=dt, device=device),
        vp=torch.empty((p.n_kv_heads, p.n_hosts, p.lp, p.head_dim), dtype=dt, device=device),
        o=torch.empty((N, p.n_q_heads, p.head_dim), dtype=dt, device=device),
        lse=torch.empty((p.n_q_heads, N), dtype=f32, device=device),
        o_part=torch.empty((p.n_hosts + 1, p.n_query, p.n_q_heads, p.head_dim), dtype=f32, device=device),
        lse_part=torch.empty((p.n_hosts + 1, p.n_q_heads, p.n_query), dtype=f32, device=device),
        ws_score=torch.empty(max(256, spava_score_topk_ws_bytes(p)), dtype=torch.uint8, device=device),
    )


def prefill(plan: Plan, q, k, v, bufs: Buffers | None = None, idx=None, stream=None,
            partials_first: bool = False) -> Buffers:
    """One layer of approximate-attention prefill: score + top-lp (unless
    ``idx`` is given), gather, fused attention, LSE merge.  Returns the
    buffers; ``bufs.o`` / ``bufs.lse`` hold the layer output.

    partials_first: run the rows that need no passing block first (query
    partials, anchor, host 0) and score from the query partials' LSEs, then
    gather and run the remaining context rows (Figure 5 ordering); same
    results."""
    p = plan
    if bufs is None:
        bufs = alloc_buffers(p, q.device)
    attn = lambda phase: spava_attn_fwd_phase(p, phase, q, k, v, bufs.kp, bufs.vp, bufs.o, bufs.lse,
                                              bufs.o_part, bufs.lse_part, stream)
    if partials_first:
        attn(SPAVA_PHASE_LOCAL)
        if idx is None:
            spava_score_topk_from_partials(p, q, k, bufs.lse_part, bufs.scores, bufs.idx, stream)
            idx = bufs.idx
        spava_gather_passing(p, k, v, idx, bufs.kp, bufs.vp, stream)
        attn(SPAVA_PHASE_PASSING)
    else:
        if idx is None:
            spava_score_topk(p, q, k, bufs.scores, bufs.idx, bufs.ws_score, stream)
            idx = bufs.idx
        spava_gather_passing(p, k, v, idx, bufs.kp, bufs.vp, stream)
        attn(SPAVA_PHASE_ALL)
    if p.n_query:
        q0 = p.n_anchor + p.n_hosts * p.host_len
        spava_lse_merge(bufs.o_part, bufs.lse_part, bufs.o[q0:], p.n_q_heads * p.head_dim,
                        bufs.lse[:, q0:], p.n_tokens, stream)
    return bufs


def plan_for(w, lp: int | None = None) -> Plan:
    """Plan of a workload object with the fields of ``workloads.Workload``."""
    return Plan(w.n_anchor, w.n_hosts, w.host_len, w.n_query, w.n_q_heads, w.n_kv_heads,
                w.head_dim, w.lp if lp is None else lp,
                SPAVA_BF16 if w.dtype == "bf16" else SPAVA_F32)
