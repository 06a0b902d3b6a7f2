"""Plain CPU oracle for the approximate-attention prefill path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline use it.  It shares no code with the HIP library.

Everything is float64 numpy, written step by step in the order the method
takes them, so that each step can be checked against the pages by eye.  A
matrix product (``@``) and a stable sort are the only library primitives.

Source pages (cited by title and section/figure):
  [Spava]  "Spava: Accelerating Long-Video Understanding via
           Sequence-Parallelism-aware Approximate Attention" (sciencestack):
           abstract; Figure 2 caption (anchor block B_a, context blocks B^(h),
           passing blocks B_p, query block B_qr); Figure 3 caption (fused
           context and query forward); Figure 5 caption (the query block's
           logits against block h rank its keys; query attention and its merging).
  [APB-V]  "APB-V: ..." machine review (pith.science): "Core claim" and
           "What carries the argument" (top-lp KVs per block ranked by the
           query block's attention scores, all-gathered as passing blocks from
           earlier hosts; attention over anchor, passing blocks and local
           context); Referee Report, major comment 1 and minor comment 2
           (Eq. (4): context attention keys [K_a, K_p, K^(h)]); "Axiom &
           Free-Parameter Ledger" (ArgTop_lp selection; exact LSE merging of
           partial query attention, Eq. 5 / Appendix A).
  [gist-nl] "Technische Samenvatting: APB-V" (gist.science/nl):
           Methodologie (context splitting) and "Systeem-niveau
           Optimalisaties" (fused context and query forward with lse merge);
           Beperkingen (one host degrades to standard attention).

Readings where the pages leave a step open (each is also a test case):
  * Scoring: for block h and KV head g, score[j] is the sum, over every
    query-block token and every query head of group g, of the softmax of
    q.k/sqrt(d) taken over the L keys of block h only.
  * Selection: the lp keys first in the order (score descending, index
    ascending); emitted as ascending block-local indices.
  * GQA: query head a reads KV head a // (Hq/Hkv).
  * Context token of host h attends to: the whole anchor, the passing blocks
    of hosts 0..h-1 (not its own), and its own block causally (diagonal
    included).  Anchor tokens attend causally within the anchor.
  * Query tokens: partial 0 covers anchor + query block (causal); partial
    h+1 covers block h in full; partials are merged by log-sum-exp.
  * Q and K are taken as given (post positional encoding).
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


def split_sequence(la: int, V: int, L: int, n_q: int) -> dict:
    """Token ranges of the anchor, the V context blocks and the query block.

    [Spava] Figure 2 caption; [gist-nl] Methodologie, context splitting.
    """
    return {
        "anchor": (0, la),
        "blocks": [(la + h * L, la + (h + 1) * L) for h in range(V)],
        "query": (la + V * L, la + V * L + n_q),
        "n_tokens": la + V * L + n_q,
    }


def block_scores(q, k, la, V, L, n_q, scale=None):
    """Query-to-context importance of every key of every block.

    [Spava] Figure 5 caption (the query block's logits Q_qr K^(h)T rank
    the keys of block h);
    [APB-V] "What carries the argument" (ranking by query-to-context
    attention scores).  Softmax restricted to block h, summed over query
    tokens and the query heads of the group.

    q: [N, Hq, d], k: [N, Hkv, d].  Returns float64 [V, Hkv, L].
    """
    Hq, d = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    seg = split_sequence(la, V, L, n_q)
    q0, q1 = seg["query"]
    qq = np.asarray(q[q0:q1], dtype=np.float64)                    # query block only
    out = np.zeros((V, Hkv, L), dtype=np.float64)
    for h, (b0, b1) in enumerate(seg["blocks"]):
        for g in range(Hkv):
            keys = np.asarray(k[b0:b1, g, :], dtype=np.float64)    # [L, d]
            for a in range(g * G, (g + 1) * G):
                rows = qq[:, a, :]                                 # [n_q, d]
                s = (rows @ keys.T) * scale                        # [n_q, L]
                s = s - s.max(axis=1, keepdims=True)
                p = np.exp(s)
                p = p / p.sum(axis=1, keepdims=True)
                out[h, g] += p.sum(axis=0)
    return out


def context_block_scores(q, k, la, V, L, n_q, scale=None):
    """Context-driven importance of every key of every block: the referee's
    alternative selector.

    [APB-V] Referee Report, major comment 1 (select the top-lp KVs of a block
    by cumulative attention from all tokens in the context block, and compare
    that selection with the query-based one) and "What would settle it" (the
    overlap of the two selected sets).  Reading: every token t of block h and
    every query head a of group g attends causally over the block's own keys
    (j <= t, diagonal included), the softmax taken over those keys only;
    score[j] sums these probabilities over the block's tokens and the group's
    heads.  Selection then follows select_passing unchanged.

    q: [N, Hq, d], k: [N, Hkv, d].  Returns float64 [V, Hkv, L].
    """
    Hq, d = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    seg = split_sequence(la, V, L, n_q)
    visible = np.tril(np.ones((L, L), dtype=bool))                  # token t sees keys j <= t
    out = np.zeros((V, Hkv, L), dtype=np.float64)
    for h, (b0, b1) in enumerate(seg["blocks"]):
        for g in range(Hkv):
            keys = np.asarray(k[b0:b1, g, :], dtype=np.float64)     # [L, d]
            for a in range(g * G, (g + 1) * G):
                rows = np.asarray(q[b0:b1, a, :], dtype=np.float64)  # the block's own tokens
                s = np.where(visible, (rows @ keys.T) * scale, NEG_INF)
                s = s - s.max(axis=1, keepdims=True)
                p = np.exp(s)
                p = p / p.sum(axis=1, keepdims=True)
                out[h, g] += p.sum(axis=0)
    return out


def kv_overlap(idx_a, idx_b):
    """Number of keys two selections share, per (block, KV head).

    [APB-V] "What would settle it": the overlap between the query-selected
    and the context-selected KV sets.  idx_*: [V, Hkv, lp].  Returns int64
    [V, Hkv].
    """
    idx_a = np.asarray(idx_a)
    idx_b = np.asarray(idx_b)
    V, Hkv, _ = idx_a.shape
    out = np.zeros((V, Hkv), dtype=np.int64)
    for h in range(V):
        for g in range(Hkv):
            out[h, g] = len(set(idx_a[h, g].tolist()) & set(idx_b[h, g].tolist()))
    return out


def select_passing(scores, lp: int):
    """ArgTop_lp per (block, KV head), ties to the lower index, ascending.

    [APB-V] "Axiom & Free-Parameter Ledger" (ArgTop_lp of the query scores
    builds the passing blocks); "Core claim" (top-lp key-value pairs).

    scores: [V, Hkv, L].  Returns int32 [V, Hkv, lp] of block-local indices.
    """
    scores = np.asarray(scores, dtype=np.float64)
    V, Hkv, L = scores.shape
    if not 0 <= lp <= L:
        raise ValueError("lp must lie in [0, L]")
    idx = np.zeros((V, Hkv, lp), dtype=np.int32)
    for h in range(V):
        for g in range(Hkv):
            order = np.argsort(-scores[h, g], kind="stable")       # desc, index asc on ties
            idx[h, g] = np.sort(order[:lp])
    return idx


def gather_passing(k, v, idx, la: int, L: int):
    """The passing blocks: selected K and V rows of every block.

    [Spava] Figure 2 caption (each context block is compressed, then
    communicated); [APB-V] "What carries the argument".

    Returns kp, vp of shape [Hkv, V, lp, d] (input dtype preserved).
    """
    V, Hkv, lp = idx.shape
    d = k.shape[2]
    kp = np.zeros((Hkv, V, lp, d), dtype=k.dtype)
    vp = np.zeros((Hkv, V, lp, d), dtype=v.dtype)
    for h in range(V):
        for g in range(Hkv):
            rows = la + h * L + idx[h, g].astype(np.int64)
            kp[g, h] = k[rows, g, :]
            vp[g, h] = v[rows, g, :]
    return kp, vp


def attend(qrows, keys, vals, visible, scale):
    """Softmax attention of query rows over a key list with a visibility mask.

    Returns O [R, d] and the natural-log LSE [R] of the scaled logits
    (the FlashAttention ``lse``: [APB-V] axiom on Eq. 5).  A row with no
    visible key gets O = 0 and LSE = -inf.
    """
    qrows = np.asarray(qrows, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    vals = np.asarray(vals, dtype=np.float64)
    R, d = qrows.shape
    if keys.shape[0] == 0:
        return np.zeros((R, vals.shape[1] if vals.ndim == 2 else d)), np.full(R, NEG_INF)
    s = (qrows @ keys.T) * scale
    s = np.where(visible, s, NEG_INF)
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.exp(s - m_safe[:, None])
    l = p.sum(axis=1)
    l_safe = np.where(empty, 1.0, l)
    o = (p @ vals) / l_safe[:, None]
    lse = np.where(empty, NEG_INF, m_safe + np.log(l_safe))
    o[empty] = 0.0
    return o, lse


def _causal(n_rows, row_tok0, n_keys, key_tok0):
    """visible[r, j] = key token (key_tok0 + j) <= row token (row_tok0 + r)."""
    rt = row_tok0 + np.arange(n_rows)[:, None]
    kt = key_tok0 + np.arange(n_keys)[None, :]
    return kt <= rt


def anchor_rows(q, k, v, la, scale):
    """Anchor tokens: causal attention within the anchor block.

    [Spava] Figure 2 caption (every host holds B_a); reading: computed once.
    Returns O [la, Hq, d], LSE [Hq, la].
    """
    Hq, d = q.shape[1], q.shape[2]
    G = Hq // k.shape[1]
    O = np.zeros((la, Hq, d))
    LSE = np.zeros((Hq, la))
    vis = _causal(la, 0, la, 0)
    for a in range(Hq):
        g = a // G
        O[:, a], LSE[a] = attend(q[:la, a], k[:la, g], v[:la, g], vis, scale)
    return O, LSE


def context_rows(q, k, v, kp, vp, la, V, L, h, scale):
    """Context tokens of virtual host h.

    Keys: anchor (all visible), passing blocks of hosts 0..h-1 (all
    visible), then host h's own block causally.  [APB-V] "Core claim"
    (passing blocks from earlier hosts; anchor, local context and passing
    blocks), Referee Report major comment 1 and minor comment 2 (Eq. (4)
    key list [K_a, K_p, K^(h)]).
    Returns O [L, Hq, d], LSE [Hq, L].
    """
    Hq, d = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    G = Hq // Hkv
    lp = kp.shape[2]
    b0 = la + h * L
    n_pass = h * lp
    n_keys = la + n_pass + L
    vis = np.ones((L, n_keys), dtype=bool)
    vis[:, la + n_pass:] = _causal(L, b0, L, b0)
    O = np.zeros((L, Hq, d))
    LSE = np.zeros((Hq, L))
    for a in range(Hq):
        g = a // G
        keys = np.concatenate([k[:la, g], kp[g, :h].reshape(n_pass, d), k[b0:b0 + L, g]], axis=0)
        vals = np.concatenate([v[:la, g], vp[g, :h].reshape(n_pass, vp.shape[-1]), v[b0:b0 + L, g]], axis=0)
        O[:, a], LSE[a] = attend(q[b0:b0 + L, a], keys, vals, vis, scale)
    return O, LSE


def query_partials(q, k, v, la, V, L, n_q, scale):
    """Partial attention of the query block, one partial per key group.

    Partial 0: anchor (all visible) + query block (causal).  Partial h+1:
    all of block h.  [Spava] Figure 3 caption (fused context and query
    forward) and Figure 5 caption ("query" then "merge"); [gist-nl]
    "Fused Context and Query Forward".
    Returns O_part [V+1, n_q, Hq, d], LSE_part [V+1, Hq, n_q].
    """
    Hq, d = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    G = Hq // Hkv
    q0 = la + V * L
    O = np.zeros((V + 1, n_q, Hq, d))
    LSE = np.zeros((V + 1, Hq, n_q))
    vis0 = np.ones((n_q, la + n_q), dtype=bool)
    vis0[:, la:] = _causal(n_q, q0, n_q, q0)
    visb = np.ones((n_q, L), dtype=bool)
    for a in range(Hq):
        g = a // G
        rows = q[q0:q0 + n_q, a]
        keys = np.concatenate([k[:la, g], k[q0:q0 + n_q, g]], axis=0)
        vals = np.concatenate([v[:la, g], v[q0:q0 + n_q, g]], axis=0)
        O[0, :, a], LSE[0, a] = attend(rows, keys, vals, vis0, scale)
        for h in range(V):
            b0 = la + h * L
            O[h + 1, :, a], LSE[h + 1, a] = attend(rows, k[b0:b0 + L, g], v[b0:b0 + L, g], visb, scale)
    return O, LSE


def lse_merge(o_parts, lse_parts):
    """Log-sum-exp merge of partial attention results.

    [APB-V] "Axiom & Free-Parameter Ledger": merging partial query
    attention through the FlashAttention lse is exact (Eq. 5, Appendix A).

    o_parts: [P, ..., d]; lse_parts: [P, ...] (same leading shape as
    o_parts without d).  Returns O [..., d], LSE [...].
    A row whose partials all have LSE = -inf gets O = 0, LSE = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse_parts - m_safe[None])
    wsum = w.sum(axis=0)
    wsum_safe = np.where(empty, 1.0, wsum)
    o = (w[..., None] * o_parts).sum(axis=0) / wsum_safe[..., None]
    o[empty] = 0.0
    lse = np.where(empty, NEG_INF, m_safe + np.log(wsum_safe))
    return o, lse


def approx_prefill(q, k, v, la, V, L, n_q, lp, scale=None, idx=None, with_scores=True):
    """The whole path: score, select, gather, attention, merge.

    q: [N, Hq, d]; k, v: [N, Hkv, d] (any float dtype; computed in float64).
    ``idx`` may be given to skip scoring/selection (e.g. to probe a chosen
    index set); otherwise it is computed from the scores.

    Returns dict: scores [V,Hkv,L] (or None), idx [V,Hkv,lp], kp, vp
    [Hkv,V,lp,d], O [N,Hq,d], LSE [Hq,N], O_part [V+1,n_q,Hq,d],
    LSE_part [V+1,Hq,n_q].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, Hq, d = q.shape
    if N != la + V * L + n_q:
        raise ValueError("token count does not match the split")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    scores = None
    if idx is None:
        scores = block_scores(q, k, la, V, L, n_q, scale)
        idx = select_passing(scores, lp)
    elif with_scores:
        scores = block_scores(q, k, la, V, L, n_q, scale)
    kp, vp = gather_passing(k, v, idx, la, L)
    O = np.zeros((N, Hq, d))
    LSE = np.zeros((Hq, N))
    if la:
        O[:la], LSE[:, :la] = anchor_rows(q, k, v, la, scale)
    for h in range(V):
        b0 = la + h * L
        O[b0:b0 + L], LSE[:, b0:b0 + L] = context_rows(q, k, v, kp, vp, la, V, L, h, scale)
    q0 = la + V * L
    O_part, LSE_part = query_partials(q, k, v, la, V, L, n_q, scale)
    if n_q:
        Oq, Lq = lse_merge(O_part, LSE_part.transpose(0, 2, 1))  # [n_q, Hq, d], [n_q, Hq]
        O[q0:] = Oq
        LSE[:, q0:] = Lq.T
    return {"scores": scores, "idx": idx, "kp": kp, "vp": vp, "O": O, "LSE": LSE,
            "O_part": O_part, "LSE_part": LSE_part}


def sampled_rows(q, k, v, kp, vp, la, V, L, n_q, rows, scale=None):
    """Outputs of chosen (token, head) pairs.

    For full-size workloads where the whole oracle is too slow.  Each row is
    computed from its own key list exactly as in ``approx_prefill``: a
    context token t of host h sees [anchor, passing blocks 0..h-1, own block
    up to t] -- a prefix of host h's full list, so the chosen rows of one
    (KV head, host) go through ``attend`` together, each masked to its own
    prefix; anchor tokens see the anchor up to themselves.  Query tokens go
    through their V+1 partials and the merge.  Inputs are converted to
    float64 one KV head at a time.
    Returns O [len(rows), d], LSE [len(rows)].
    """
    Hq, d = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    G = Hq // Hkv
    lp = kp.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q0 = la + V * L
    outO = np.zeros((len(rows), vp.shape[-1]))
    outL = np.zeros(len(rows))
    for g in range(Hkv):
        mine = [n for n, (t, a) in enumerate(rows) if a // G == g]
        if not mine:
            continue
        kg = np.asarray(k[:, g], dtype=np.float64)
        vg = np.asarray(v[:, g], dtype=np.float64)
        kpg = np.asarray(kp[g], dtype=np.float64).reshape(V * lp, d)
        vpg = np.asarray(vp[g], dtype=np.float64).reshape(V * lp, -1)
        # Rows that share a key list: the anchor ("a"), host h's context
        # tokens (h), and each query token on its own.
        groups = {}
        for n in mine:
            t = rows[n][0]
            key = "a" if t < la else ((t - la) // L if t < q0 else ("q", n))
            groups.setdefault(key, []).append(n)
        for key, ns in groups.items():
            toks = np.array([rows[n][0] for n in ns])
            qr = np.stack([np.asarray(q[rows[n][0], rows[n][1]], dtype=np.float64) for n in ns])
            if key == "a":                                          # anchor tokens: causal
                keys, vals = kg[:la], vg[:la]
                n_vis = toks + 1
            elif not isinstance(key, tuple):                        # context tokens of host h
                h = key
                b0 = la + h * L
                keys = np.concatenate([kg[:la], kpg[:h * lp], kg[b0:b0 + L]], axis=0)
                vals = np.concatenate([vg[:la], vpg[:h * lp], vg[b0:b0 + L]], axis=0)
                n_vis = la + h * lp + (toks - b0) + 1
            else:                                                   # query token: partials + merge
                t = toks[0]
                parts_o, parts_l = [], []
                keys = np.concatenate([kg[:la], kg[q0:t + 1]], axis=0)
                vals = np.concatenate([vg[:la], vg[q0:t + 1]], axis=0)
                o0, l0 = attend(qr, keys, vals, np.ones((1, keys.shape[0]), bool), scale)
                parts_o.append(o0[0]); parts_l.append(l0[0])
                for h in range(V):
                    b0 = la + h * L
                    oh, lh = attend(qr, kg[b0:b0 + L], vg[b0:b0 + L], np.ones((1, L), bool), scale)
                    parts_o.append(oh[0]); parts_l.append(lh[0])
                o, lse = lse_merge(np.stack(parts_o)[:, None, :], np.stack(parts_l)[:, None])
                outO[ns[0]], outL[ns[0]] = o[0], lse[0]
                continue
            vis = np.arange(keys.shape[0])[None, :] < n_vis[:, None]
            o, lse = attend(qr, keys, vals, vis, scale)
            outO[ns], outL[ns] = o, lse
    return outO, outL


def dense_causal(q, k, v, scale=None):
    """Exact causal softmax attention over the whole sequence (the textbook
    definition; GQA head a reads KV head a // G).  Used as the reference for
    the cases where the method must reduce to it: [gist-nl] Beperkingen (one
    host degrades to standard attention).

    Returns O [N, Hq, d], LSE [Hq, N].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, Hq, d = q.shape
    G = Hq // k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    vis = _causal(N, 0, N, 0)
    O = np.zeros((N, Hq, d))
    LSE = np.zeros((Hq, N))
    for a in range(Hq):
        O[:, a], LSE[a] = attend(q[:, a], k[:, a // G], v[:, a // G], vis, scale)
    return O, LSE
