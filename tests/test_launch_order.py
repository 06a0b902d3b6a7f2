"""The attention kernel's launch order (re-derived here from its definition:
context units of the first n_ctx_first hosts from V-1 down, the query-block
partials, the remaining hosts' context units, query partial 0, the anchor)
visits every unit exactly once for any split point, and the host rule that
picks the split point puts the query-block partials after exactly the hosts
whose shortest unit is at least as long.  Host logic only: no GPU is used.
"""
import pytest

import workloads as W

KT, BM = 64, 256


def cdiv(a, b):
    return -(-a // b)


def decode(w, n_first, b):
    V, L, Hq, Hkv, nq = w.n_hosts, w.host_len, w.n_q_heads, w.n_kv_heads, w.n_query
    G = Hq // Hkv
    n_ctx_h = cdiv(L, BM) * Hq
    qt = cdiv(nq * G, BM)
    n_q = qt * Hkv
    nctx, nqb, n1 = V * n_ctx_h, V * n_q, n_first * n_ctx_h
    if b < n1 or n1 + nqb <= b < nctx + nqb:
        c = b if b < n1 else b - nqb
        r = c % n_ctx_h
        return ("ctx", V - 1 - c // n_ctx_h, r % Hq, cdiv(L, BM) - 1 - r // Hq)
    if b < n1 + nqb:
        b -= n1
        return ("qblock", b // n_q, (b % n_q) // qt, (b % n_q) % qt)
    b -= nctx + nqb
    if b < n_q:
        return ("qhead", b // qt, b % qt)
    b -= n_q
    na = cdiv(w.n_anchor, BM)
    return ("anchor", b % Hq, na - 1 - b // Hq)


def all_units(w):
    V, L, Hq, Hkv, nq, la = w.n_hosts, w.host_len, w.n_q_heads, w.n_kv_heads, w.n_query, w.n_anchor
    G = Hq // Hkv
    qt = cdiv(nq * G, BM)
    u = {("ctx", h, a, t) for h in range(V) for a in range(Hq) for t in range(cdiv(L, BM))}
    u |= {("qblock", h, g, t) for h in range(V) for g in range(Hkv) for t in range(qt)}
    u |= {("qhead", g, t) for g in range(Hkv) for t in range(qt)}
    u |= {("anchor", a, t) for a in range(Hq) for t in range(cdiv(la, BM))}
    return u


def n_ctx_first(w):
    """Hosts whose shortest context unit (first row tile) walks at least the
    ceil(L/64) tiles of a query-block partial."""
    t_q = cdiv(w.host_len, KT)
    return sum(1 for h in range(w.n_hosts)
               if cdiv(w.n_anchor, KT) + (cdiv(h * w.lp, KT) if h else 0) + cdiv(min(w.host_len, BM), KT) >= t_q)


SHAPES = [W.small_workload("bf16", Hq=7, Hkv=1, d=128, la=130, V=2, L=200, n_q=33, lp=0, seed=9),
          W.small_workload("bf16", Hq=8, Hkv=2, d=64, la=0, V=4, L=77, n_q=9, lp=77, seed=8),
          W.small_workload("bf16", Hq=2, Hkv=1, d=128, la=64, V=1, L=300, n_q=0, lp=17, seed=11),
          W.QWEN3B_32K, W.QWEN3B_32K_PAGE_DEFAULTS_Q128, W.QWEN3B_128K]


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_every_split_point_visits_every_unit_once(w):
    want = all_units(w)
    for nf in range(w.n_hosts + 1):
        got = [decode(w, nf, b) for b in range(len(want))]
        assert len(set(got)) == len(got) and set(got) == want, nf


def test_split_point_rule():
    # 32K: the first row tile of host h walks 32 + 16h + 4 tiles against 60
    # for a query-block partial, so hosts 7..2 go first.
    assert n_ctx_first(W.QWEN3B_32K) == 6
    # No passing blocks and a short anchor: every host's first tiles are
    # shorter than a whole block, so the partials lead.
    assert n_ctx_first(W.QWEN3B_32K.with_(lp=0, n_anchor=0)) == 0
    # Longer anchors than blocks: every host goes first (the previous order).
    w = W.small_workload("bf16", Hq=2, Hkv=1, d=128, la=512, V=3, L=128, n_q=8, lp=8, seed=1)
    assert n_ctx_first(w) == 3
