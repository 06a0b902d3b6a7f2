"""Seeded synthetic inputs for the approximate-attention prefill path.

This module holds the workload shapes and the input generator shared by the
tests, the benchmark and the smoke check.  It contains none of the method's
arithmetic: no scoring, selection, attention or merging happens here.  It only
draws Q, K and V and plants the key structure each workload calls for.

Workload shapes follow the long-video setting of "Spava / APB-V:
Accelerating Long-Video Understanding via Sequence-Parallelism-aware
Approximate Attention" (Figure 2 caption: anchor block, virtual-host context
blocks, query block).  The head counts mimic Qwen2.5-VL attention layers, the
base models named in that paper's experiments.  The pages measure on
LongVideoBench / VNBench videos; no dataset is used here: these seeded inputs
stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
import math

import numpy as np

BF16 = "bf16"
F32 = "f32"


@dataclass(frozen=True)
class Workload:
    """Shape of one prefill layer.

    Token layout (rows of Q/K/V): anchor ``[0, la)``, then ``V`` context blocks
    of ``L`` tokens each, then ``n_q`` query tokens.
    """

    name: str
    dtype: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_anchor: int      # la
    n_hosts: int       # V (virtual hosts)
    host_len: int      # L
    n_query: int       # n_q
    lp: int            # passing length
    structure: str     # "planted_count", "planted_frac", "needle", "frames", "none"
    structure_arg: float = 0.0
    seed: int = 0

    @property
    def n_tokens(self) -> int:
        return self.n_anchor + self.n_hosts * self.host_len + self.n_query

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads.  Index i uses seed i.
TINY_F32 = Workload("tiny_f32", F32, 2, 1, 64, 32, 4, 128, 16, 16,
                    "planted_count", 4, seed=0)
QWEN3B_32K = Workload("qwen2.5vl3b_32k", BF16, 16, 2, 128, 2048, 8, 3840, 128,
                      1024, "planted_frac", 0.01, seed=1)
QWEN7B_64K = Workload("qwen2.5vl7b_64k", BF16, 28, 4, 128, 2048, 16, 3968, 256,
                      2048, "planted_frac", 0.01, seed=2)
QWEN3B_128K = Workload("qwen2.5vl3b_128k", BF16, 16, 2, 128, 2048, 16, 8064, 128,
                       512, "needle", 64, seed=3)
QWEN7B_256K = Workload("qwen2.5vl7b_256k_frames", BF16, 28, 4, 128, 4096, 32, 8128,
                       512, 4096, "frames", 1024, seed=4)

WORKLOADS = [TINY_F32, QWEN3B_32K, QWEN7B_64K, QWEN3B_128K, QWEN7B_256K]
QWEN3B_128K_LP_SWEEP = (512, 2048, 8064)

# The pages' default hyper-parameters (APB-V review, free-parameter ledger:
# anchor length la = n/64, passing length lp = n/128, H = 8 hosts), with n the
# whole input length, on two shapes:
#  * the 32K video layer above, re-split at n = 32768 (la 512, lp 256);
#  * a text-shaped layer standing in for the pages' long-context NLP transfer
#    (RULER at 128K input, Llama-3.1-8B, 8 GPUs): 128K tokens, 32 query / 8 KV
#    heads of width 128 (the public Llama-3.1-8B configuration; the pages give
#    no head counts) and a 64-key needle in place of the benchmark's
#    needle-in-a-haystack items (no RULER data is used).
# The pages give no query length; both use a 512-token query block, which
# makes the host blocks whole 64-key tiles (L = 3968 and 16064).
QWEN3B_32K_PAGE_DEFAULTS = Workload("qwen2.5vl3b_32k_page_defaults", BF16, 16, 2, 128,
                                    32768 // 64, 8, 3968, 512, 32768 // 128,
                                    "planted_frac", 0.01, seed=5)
LLAMA8B_128K_TEXT = Workload("llama3.1-8b_128k_text", BF16, 32, 8, 128,
                             131072 // 64, 8, 16064, 512, 131072 // 128,
                             "needle", 64, seed=6)
# The same 32K re-split with a 128-token query block: host blocks of 4016
# keys, not whole tiles.
QWEN3B_32K_PAGE_DEFAULTS_Q128 = QWEN3B_32K_PAGE_DEFAULTS.with_(
    name="qwen2.5vl3b_32k_page_defaults_q128", host_len=4016, n_query=128)
PAGE_DEFAULT_WORKLOADS = [QWEN3B_32K_PAGE_DEFAULTS, LLAMA8B_128K_TEXT]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns float32 values whose low 16 bits are zero.  Inputs are finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x_rounded: np.ndarray) -> np.ndarray:
    """High 16 bits of already-rounded float32 values (the bfloat16 encoding)."""
    return (np.ascontiguousarray(x_rounded, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _mean_query_dir(q: np.ndarray, w: Workload, g: int) -> np.ndarray:
    """Unit vector along the mean of the query-block rows of KV group ``g``."""
    q0 = w.n_anchor + w.n_hosts * w.host_len
    qs = q[q0:q0 + w.n_query, g * w.group:(g + 1) * w.group, :].astype(np.float64)
    m = qs.reshape(-1, w.head_dim).mean(axis=0) if qs.size else np.ones(w.head_dim)
    n = np.linalg.norm(m)
    if n == 0.0:
        m = np.ones(w.head_dim)
        n = np.linalg.norm(m)
    return m / n


def make_inputs(w: Workload, seed: int | None = None):
    """Draw Q, K, V for workload ``w``.

    Recipe: ``numpy.random.Generator(PCG64(seed))``; Q ``[N, Hq, d]``, K and V
    ``[N, Hkv, d]`` drawn in that order as float32 standard normals; then the
    key structure; then (bf16 workloads) one round-to-nearest-even cast.

    Key structure (applied to K rows of the anchor and context blocks only,
    except "planted" which touches context blocks only):
      * planted_count / planted_frac: per (block h, KV head g), in h-major
        order, ``n`` block-local positions drawn without replacement are set
        to ``3*sqrt(d)*u_g`` where ``u_g`` is the unit mean direction of the
        query-block rows of group g.  ``n`` is the count, or round(frac*L).
      * needle: 64 consecutive context keys starting uniformly in
        ``[la, la+V*L-64]`` are set to ``3*sqrt(d)*u_g`` for every g.
      * frames: for token t < la+V*L, ``K[t] += o[t // 1024]`` with
        ``o ~ N(0, 0.5)`` (variance 0.5) per (frame, g, channel).

    Returns a dict with float32 arrays ``q, k, v`` (already rounded for bf16
    workloads) and, for bf16 workloads, the uint16 encodings ``q16, k16, v16``.
    """
    if seed is None:
        seed = w.seed
    rng = np.random.Generator(np.random.PCG64(seed))
    N, Hq, Hkv, d = w.n_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim
    q = rng.standard_normal((N, Hq, d), dtype=np.float32)
    k = rng.standard_normal((N, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((N, Hkv, d), dtype=np.float32)
    la, L, V = w.n_anchor, w.host_len, w.n_hosts
    amp = 3.0 * math.sqrt(d)
    if w.structure in ("planted_count", "planted_frac"):
        n = int(w.structure_arg) if w.structure == "planted_count" else int(round(w.structure_arg * L))
        n = max(0, min(n, L))
        dirs = [(_mean_query_dir(q, w, g) * amp).astype(np.float32) for g in range(Hkv)]
        for h in range(V):
            for g in range(Hkv):
                pos = rng.choice(L, n, replace=False) if n else np.zeros(0, dtype=np.int64)
                k[la + h * L + pos, g, :] = dirs[g]
    elif w.structure == "needle":
        span = int(w.structure_arg)
        lo, hi = la, la + V * L - span
        if hi >= lo and span > 0:
            start = int(rng.integers(lo, hi + 1))
            for g in range(Hkv):
                k[start:start + span, g, :] = (_mean_query_dir(q, w, g) * amp).astype(np.float32)
    elif w.structure == "frames":
        flen = int(w.structure_arg)
        nctx = la + V * L
        nf = (nctx + flen - 1) // flen
        o = (rng.standard_normal((nf, Hkv, d), dtype=np.float32) * np.float32(math.sqrt(0.5)))
        k[:nctx] += np.repeat(o, flen, axis=0)[:nctx]
    elif w.structure != "none":
        raise ValueError(f"unknown structure {w.structure!r}")
    out = {"q": q, "k": k, "v": v}
    if w.dtype == BF16:
        for name in ("q", "k", "v"):
            r = bf16_round(out[name])
            out[name] = r
            out[name + "16"] = bf16_bits(r)
    return out


def small_workload(dtype=BF16, *, Hq=4, Hkv=2, d=128, la=48, V=3, L=100, n_q=20,
                   lp=24, structure="planted_count", arg=3, seed=7) -> Workload:
    """A small ragged workload (sizes not multiples of the kernels' tiles)."""
    return Workload(f"small_{dtype}_{Hq}x{Hkv}x{d}_la{la}_V{V}_L{L}_q{n_q}_lp{lp}", dtype,
                    Hq, Hkv, d, la, V, L, n_q, lp, structure, arg, seed=seed)


def random_small_workloads(count: int = 120, seed: int = 2026) -> list[Workload]:
    """A fixed, seeded list of small ragged shapes drawn at random (head
    grouping, width, anchor, hosts, block length, query length, passing
    length with extra weight on 0, 1 and L; a few float32), sized so that the
    oracle finishes each in well under a second."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 3, 7]))
        while Hkv * G > 16:
            G = int(rng.choice([1, 2, 3]))
        d = int(rng.choice([64, 128]))
        la = int(rng.choice([0, int(rng.integers(1, 300))]))
        V = int(rng.integers(1, 7))
        L = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 700))]))
        n_q = int(rng.choice([0, int(rng.integers(1, 49))]))
        lp = int(rng.choice([0, 1, L, int(rng.integers(0, L + 1))]))
        dtype = F32 if rng.random() < 0.15 else BF16
        out.append(small_workload(dtype, Hq=Hkv * G, Hkv=Hkv, d=d, la=la, V=V, L=L, n_q=n_q, lp=lp,
                                  seed=1000 + i))
    return out
