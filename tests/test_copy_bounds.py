"""Every direct-to-LDS copy of the bf16 kernels addresses memory inside its
tensor, on every workload shape, without relying on the buffer range check.

The kernels' tile walks are re-derived here from their definitions (the unit
order, each unit's key runs, the tile cursors of the attention kernel, the key
chunks of the row statistics, the query-row chunks of the column sums) and
every copy's byte range is checked against the tensor it reads.  Host logic
only: no GPU is used.  A tensor whose size is a multiple of the allocator's
2 MiB granule has no slack behind it, so a read past its end can fault; this
is the check that would have caught such reads.
"""
import numpy as np
import pytest

import workloads as W

KT = 64          # keys per tile
BM = 256         # query rows per attention unit
CS_ROWS = 32     # query rows per column-sum chunk


def cdiv(a, b):
    return -(-a // b)


class Extent:
    def __init__(self, name, nbytes):
        self.name, self.nbytes = name, nbytes

    def check(self, lo, hi, what):
        assert 0 <= lo and hi <= self.nbytes, f"{what}: {self.name} bytes [{lo}, {hi}) outside [0, {self.nbytes})"


def layout(w, D, strides):
    """Element strides (q token, q head, kv token, kv head) and the element
    extents of q and k under them; strides=None is the dense layout,
    "packed" a QKV projection output [N][Hq+2Hkv][d], "heads_major" [H][N][d]."""
    N, Hq, Hkv = w.n_tokens, w.n_q_heads, w.n_kv_heads
    if strides is None:
        st = (Hq * D, D, Hkv * D, D)
    elif strides == "packed":
        st = ((Hq + 2 * Hkv) * D, D, (Hq + 2 * Hkv) * D, D)
    else:
        st = (D, N * D, D, N * D)
    q_ext = (N - 1) * st[0] + (Hq - 1) * st[1] + D
    k_ext = (N - 1) * st[2] + (Hkv - 1) * st[3] + D
    return st, q_ext, k_ext


def attention_copies(w, D, past_walk="stay", strides=None):
    """Walk the attention kernel's K and V cursors of every unit (V tiles are
    copied row-major from v and vp exactly as K tiles from k and kp).  With
    past_walk="advance" a cursor keeps stepping over whole tiles after the
    walk (what a cursor whose remaining byte count had gone negative, read as
    an unsigned range, would do); the kernels keep it on its last tile."""
    la, V, L, nq, lp, Hq, Hkv = w.n_anchor, w.n_hosts, w.host_len, w.n_query, w.lp, w.n_q_heads, w.n_kv_heads
    G = Hq // Hkv
    N = la + V * L + nq
    (_, _, kv_st, kv_sh), _, k_ext = layout(w, D, strides)
    ext = {"k": Extent("k", k_ext * 2), "kp": Extent("kp", Hkv * V * lp * D * 2),
           "v": Extent("v", k_ext * 2), "vp": Extent("vp", Hkv * V * lp * D * 2)}
    n_ctx_h = cdiv(L, BM) * Hq
    n_q = cdiv(nq * G, BM) * Hkv
    qt = n_q // Hkv
    n_units = V * n_ctx_h + V * n_q + n_q + cdiv(la, BM) * Hq
    tiles = 0
    for b in range(n_units):
        if b < V * n_ctx_h:
            kind, host = "ctx", V - 1 - b // n_ctx_h
            r = b % n_ctx_h
            head, tile = r % Hq, cdiv(L, BM) - 1 - r // Hq
            g = head // G
        elif b < V * n_ctx_h + V * n_q:
            bb = b - V * n_ctx_h
            kind, host, g, tile = "qblock", bb // n_q, (bb % n_q) // qt, (bb % n_q) % qt
        elif b < V * n_ctx_h + V * n_q + n_q:
            bb = b - V * n_ctx_h - V * n_q
            kind, host, g, tile = "qhead", 0, bb // qt, bb % qt
        else:
            bb = b - V * n_ctx_h - V * n_q - n_q
            kind, host = "anchor", 0
            head, tile = bb % Hq, cdiv(la, BM) - 1 - bb // Hq
            g = head // G
        if kind in ("ctx", "anchor"):
            base, n = (0, la) if kind == "anchor" else (la + host * L, L)
            toks = [base + r for r in range(tile * BM, min(n, tile * BM + BM))]
        else:
            R = nq * G
            toks = [la + V * L + r % nq for r in range(tile * BM, min(R, tile * BM + BM))]
        if not toks:
            continue
        gmax = max(toks)

        def main(tok0, n, causal):
            return dict(kbuf="k", k=(tok0 * kv_st + g * kv_sh) * 2, vbuf="v", v=(tok0 * kv_st + g * kv_sh) * 2,
                        kstr=kv_st * 2, len=n, causal=causal, tok0=tok0)
        runs = [main(0, 0, 0)] * 3
        if kind == "anchor":
            runs = [main(0, la, 1), dict(runs[1], len=0), dict(runs[2], len=0)]
        elif kind == "ctx":
            pas = dict(kbuf="kp", k=g * V * lp * D * 2, vbuf="vp", v=g * V * lp * D * 2,
                       kstr=D * 2, len=host * lp if lp else 0, causal=0, tok0=0)
            runs = [main(0, la, 0), pas if host > 0 else dict(pas, len=0), main(la + host * L, L, 1)]
        elif kind == "qhead":
            runs = [main(0, la, 0), main(la + V * L, nq, 1), dict(runs[2], len=0)]
        else:
            runs = [main(la + host * L, L, 0), dict(runs[1], len=0), dict(runs[2], len=0)]
        nts = []
        for x in runs:
            n = min(x["len"], gmax - x["tok0"] + 1) if x["causal"] else x["len"]
            nts.append(cdiv(n, KT) if n > 0 else 0)
        T = sum(nts)

        def walk(is_k):
            """Byte ranges [lo, hi) and buffer of the copies issued for tiles
            0 .. T+3 of the K (is_k) or V cursor: both walk the same rows, K
            from k / kp and V from v / vp."""
            out = []
            addr, stride, buf = runs[0]["k" if is_k else "v"], runs[0]["kstr"], "k" if is_k else "v"
            s, left, rows = 0, 0, 0

            def enter(s0):
                nonlocal s, left, rows, addr, stride, buf
                s = s0
                while s < 3 and nts[s] == 0:
                    s += 1
                if s >= 3:
                    if past_walk == "stay":
                        left, rows = 1, 0      # stays on its last tile
                    else:
                        left, rows = 1 << 30, 1 << 30
                    return
                x = runs[s]
                left = nts[s]
                addr, stride, rows = (x["k"] if is_k else x["v"]), x["kstr"], x["len"]
                buf = x["kbuf"] if is_k else x["vbuf"]
            enter(0)
            for _ in range(T + 4):
                last = max(0, min(KT, rows) - 1)
                out.append((buf, addr, addr + last * stride + D * 2))
                if left > 1:
                    left -= 1
                    addr += KT * stride
                    rows -= KT
                else:
                    enter(s + 1)
            return out
        for is_k in (True, False):
            for buf, lo, hi in walk(is_k):
                ext[buf].check(lo, hi, f"{w.name} unit {b} ({kind}) {'K' if is_k else 'V'} copy")
                tiles += 1
    return tiles


RS_ROWS = 256    # rows per row-statistics workgroup


def score_copies(w, D, ctx=False, strides=None):
    """Row statistics: K tiles of each key chunk; column sums: Q rows of each
    chunk.  ctx=True walks the context selector: the scoring rows are each
    block's own tokens, and a row-statistics workgroup stops at the tile of
    its last token (possibly before its chunk's first tile)."""
    la, V, L, nq, Hq, Hkv = w.n_anchor, w.n_hosts, w.host_len, w.n_query, w.n_q_heads, w.n_kv_heads
    G = Hq // Hkv
    N = la + V * L + nq
    ntok = L if ctx else nq
    R = ntok * G
    (q_st, q_sh, kv_st, kv_sh), q_ext, k_ext = layout(w, D, strides)
    k = Extent("k", k_ext * 2)
    q = Extent("q", q_ext * 2)
    if R == 0:
        return 0
    T = cdiv(L, KT)
    tpc = T if ctx else max(8, cdiv(T, 16))   # the context selector takes all keys in one chunk
    kc_n = cdiv(T, tpc)
    kstr = kv_st * 2
    n = 0
    for h in range(V):
        for g in range(Hkv):
            kblk = ((la + h * L) * kv_st + g * kv_sh) * 2
            for kc in range(kc_n):
                t0 = kc * tpc
                nts = [min(T, t0 + tpc) - t0]
                if ctx:
                    nts = []
                    for rt in range(cdiv(R, RS_ROWS)):
                        r_lo, r_hi = rt * RS_ROWS, min(R, rt * RS_ROWS + RS_ROWS) - 1
                        last = ntok - 1 if r_lo // ntok != r_hi // ntok else r_hi % ntok
                        nts.append(max(0, min(min(T, t0 + tpc) - t0, cdiv(last + 1, KT) - t0)))
                for nt in sorted(set(nts)):
                    for t in range(nt + 3):
                        tt = t0 + (t if t < nt else 0)
                        first, last = tt * KT, min(tt * KT + KT - 1, L - 1)
                        k.check(kblk + first * kstr, kblk + last * kstr + D * 2,
                                f"{w.name} row statistics h{h} g{g}")
                        n += 1
    # Column sums: a chunk copy starts at any row r0 < R of a split (or at R
    # for the look-ahead past a split's last chunk) and covers rows r0..r0+31;
    # row r < R is token r % ntok of head g*G + r // ntok, rows >= R read row 0.
    r = np.arange(R + CS_ROWS)
    tok = np.where(r < R, r % ntok, 0)
    head = np.where(r < R, r // ntok, 0)
    for h in range(V if ctx else 1):
        q0 = ((la + h * L) if ctx else (la + V * L)) * q_st * 2
        q_end = q0 + ((ntok - 1) * q_st + (Hq - 1) * q_sh + D) * 2   # the column sums' Q range ends here
        for g in range(Hkv):
            off = q0 + (tok * q_st + (g * G + head) * q_sh) * 2
            lo, hi = int(off.min()), int(off.max()) + D * 2
            q.check(lo, hi, f"{w.name} column sums h{h} g{g}")
            assert hi <= q_end, f"{w.name}: column-sum copy past its range"
            n += len(r)
    return n


SMALL = [
    W.small_workload("bf16"),
    W.small_workload("bf16", Hq=8, Hkv=2, d=64, la=0, V=4, L=77, n_q=9, lp=77, seed=8),
    W.small_workload("bf16", Hq=7, Hkv=1, d=128, la=130, V=2, L=200, n_q=33, lp=0, seed=9),
    W.small_workload("bf16", Hq=4, Hkv=4, d=128, la=5, V=5, L=64, n_q=1, lp=1, seed=10),
    W.small_workload("bf16", Hq=2, Hkv=1, d=128, la=64, V=1, L=300, n_q=0, lp=17, seed=11),
]
FULL = [W.QWEN3B_32K, W.QWEN7B_64K, W.QWEN3B_128K, W.QWEN3B_128K.with_(lp=8064),
        W.QWEN3B_32K_PAGE_DEFAULTS, W.QWEN3B_32K_PAGE_DEFAULTS_Q128, W.LLAMA8B_128K_TEXT]


@pytest.mark.parametrize("w", SMALL + FULL, ids=lambda w: f"{w.name}_lp{w.lp}")
def test_score_copies_in_bounds(w):
    assert score_copies(w, w.head_dim) > 0 or w.n_query == 0


@pytest.mark.parametrize("w", SMALL + [W.QWEN3B_32K, W.QWEN3B_32K_PAGE_DEFAULTS_Q128, W.LLAMA8B_128K_TEXT],
                         ids=lambda w: w.name)
def test_context_score_copies_in_bounds(w):
    assert score_copies(w, w.head_dim, ctx=True) > 0


@pytest.mark.parametrize("w", SMALL + FULL, ids=lambda w: f"{w.name}_lp{w.lp}")
def test_attention_copies_in_bounds(w):
    assert attention_copies(w, w.head_dim) > 0


@pytest.mark.parametrize("strides", ["packed", "heads_major"])
@pytest.mark.parametrize("w", SMALL[:4] + [W.QWEN3B_32K], ids=lambda w: w.name)
def test_strided_copies_in_bounds(w, strides):
    # q, k, v as views of a packed QKV buffer or of head-major tensors.
    assert attention_copies(w, w.head_dim, strides=strides) > 0
    assert score_copies(w, w.head_dim, strides=strides) > 0 or w.n_query == 0
    assert score_copies(w, w.head_dim, ctx=True, strides=strides) > 0


@pytest.mark.parametrize("w", [W.QWEN3B_32K_PAGE_DEFAULTS_Q128, W.LLAMA8B_128K_TEXT], ids=lambda w: w.name)
def test_walk_catches_a_cursor_that_runs_past_the_walk(w):
    # The query partials' last run ends at token N: stepping on past it reads
    # beyond k.  Both of these shapes have k ending on a 2 MiB granule.
    assert (w.n_tokens * w.n_kv_heads * w.head_dim * 2) % (2 << 20) == 0
    with pytest.raises(AssertionError, match="outside"):
        attention_copies(w, w.head_dim, past_walk="advance")


RANDOM_BF16 = [w for w in W.random_small_workloads() if w.dtype == W.BF16]


RANDOM_ALL = W.random_small_workloads()


@pytest.mark.parametrize("w", RANDOM_BF16, ids=lambda w: w.name)
def test_random_shapes_copies_in_bounds(w):
    # The seeded random shapes of the GPU parity sweep, before any GPU runs
    # them, in the layout the sweep also gives them (dense for all; packed
    # QKV or head-major for shape index 1 or 2 modulo 3).
    layouts = [None, [None, "packed", "heads_major"][RANDOM_ALL.index(w) % 3]]
    for strides in dict.fromkeys(layouts):
        assert attention_copies(w, w.head_dim, strides=strides) > 0
        assert score_copies(w, w.head_dim, strides=strides) > 0 or w.n_query == 0
        assert score_copies(w, w.head_dim, ctx=True, strides=strides) > 0
