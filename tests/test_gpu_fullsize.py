"""Full-size workloads (32K-256K tokens): every score and selected index is
compared with the oracle; gathered rows on a sample; attention on sampled
(token, head) rows that the oracle computes one by one, in the same launch
configuration the benchmark uses.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import sequence_approximate_attention_amd as S
import workloads as W
from gpu_helpers import TOL, check_close, check_idx, dev_inputs, np64, sample_rows

pytestmark = pytest.mark.gpu

_cache = {}


def inputs(w):
    key = (w.name, w.seed)
    if key not in _cache:
        _cache.clear()
        x = W.make_inputs(w)
        sc = O.block_scores(x["q"], x["k"], w.n_anchor, w.n_hosts, w.host_len, w.n_query)
        _cache[key] = (x, sc)
    return _cache[key]


def heads_to_sample(w):
    """The first query head of every KV group, and the last head."""
    G = w.group
    return sorted({0, w.n_q_heads - 1} | {g * G for g in range(w.n_kv_heads)})


def run_case(w, query_stride=7, dense_check=False, stride=61, heads=None, partials_first=False):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    x, sc = inputs(w)
    print(f"[fullsize] {w.name} lp={w.lp} N={w.n_tokens} partials_first={partials_first}", flush=True)
    idx_o = O.select_passing(sc, w.lp)
    plan = S.plan_for(w)
    q, k, v = dev_inputs(x, w)
    # 1. Scores and selection, full.
    bufs = S.prefill(plan, q, k, v, partials_first=partials_first)
    torch.cuda.synchronize()
    got_sc = np64(bufs.scores)
    rel = np.abs(got_sc - sc) / np.maximum(sc, 1e-30)
    assert rel.max() < 1e-5, f"scores rel err {rel.max():.2e}"
    idx_g = bufs.idx.cpu().numpy()
    n_diff = check_idx(sc, idx_g, idx_o, w.lp)
    print(f"[fullsize] scores max rel err {rel.max():.2e}; index differences at near-ties: {n_diff}")
    # 2. Gather + attention with the oracle's own selection.
    bufs2 = S.prefill(plan, q, k, v, idx=torch.from_numpy(idx_o).to(q.device), partials_first=partials_first)
    torch.cuda.synchronize()
    kp_o, vp_o = O.gather_passing(x["k"], x["v"], idx_o, w.n_anchor, w.host_len)
    rng = np.random.default_rng(0)
    sel = rng.choice(kp_o.shape[2], size=min(64, kp_o.shape[2]), replace=False) if w.lp else []
    np.testing.assert_array_equal(np64(bufs2.kp[:, :, sel]), kp_o[:, :, sel])
    np.testing.assert_array_equal(np64(bufs2.vp[:, :, sel]), vp_o[:, :, sel])
    rows = sample_rows(w, heads if heads is not None else heads_to_sample(w), stride=stride,
                       query_stride=query_stride)
    o_ref, l_ref = O.sampled_rows(x["q"], x["k"], x["v"], kp_o, vp_o, w.n_anchor, w.n_hosts,
                                  w.host_len, w.n_query, rows)
    t = torch.tensor([r[0] for r in rows], device=q.device)
    a = torch.tensor([r[1] for r in rows], device=q.device)
    o_got = np64(bufs2.o[t, a])
    l_got = np64(bufs2.lse[a, t])
    tol = TOL[w.dtype]
    mx = check_close(o_got, o_ref, tol["o_max"], tol["o_mean"], f"{w.name} O")
    check_close(l_got, l_ref, tol["lse_max"], None, f"{w.name} LSE")
    print(f"[fullsize] {len(rows)} sampled rows: O max-abs {mx:.2e}")
    # 3. The GPU's own selection end to end (differs only at allowed near-ties).
    if n_diff:
        o_own = np64(bufs.o[t, a])
        check_close(o_own, o_ref, tol["o_max"], tol["o_mean"], f"{w.name} O (own idx)")
    else:
        assert torch.equal(bufs.o.view(torch.int16), bufs2.o.view(torch.int16))
    if dense_check:
        # lp = L keeps every key: exact causal attention (definition written out).
        scale = 1.0 / math.sqrt(w.head_dim)
        G = w.group
        dense_o = np.zeros_like(o_ref)
        dense_l = np.zeros_like(l_ref)
        for n, (tk, hd) in enumerate(rows):
            kk = x["k"][:tk + 1, hd // G].astype(np.float64)
            vv = x["v"][:tk + 1, hd // G].astype(np.float64)
            oo, ll = O.attend(x["q"][tk, hd][None].astype(np.float64), kk, vv,
                              np.ones((1, tk + 1), bool), scale)
            dense_o[n], dense_l[n] = oo[0], ll[0]
        check_close(o_got, dense_o, tol["o_max"], tol["o_mean"], "lp=L vs dense O")
        check_close(l_got, dense_l, tol["lse_max"], None, "lp=L vs dense LSE")


def test_qwen3b_32k():
    run_case(W.QWEN3B_32K, query_stride=1)


def test_qwen7b_64k():
    run_case(W.QWEN7B_64K, query_stride=3)


@pytest.mark.parametrize("lp", W.QWEN3B_128K_LP_SWEEP)
def test_qwen3b_128k_lp_sweep(lp):
    run_case(W.QWEN3B_128K.with_(lp=lp), query_stride=5, dense_check=(lp == W.QWEN3B_128K.host_len))


def test_qwen7b_256k_frames():
    # One query head of every KV group (0, 7, 14, 21) and the last head; every
    # 127th token keeps the oracle's share of the run to about a minute.
    w = W.QWEN7B_256K
    run_case(w, query_stride=17, stride=127)


# The pages' default hyper-parameters (la = n/64, lp = n/128).
def test_qwen3b_32k_page_defaults():
    run_case(W.QWEN3B_32K_PAGE_DEFAULTS, query_stride=3)


# Host blocks of 4016 keys (not whole tiles), 128-token query block.
def test_qwen3b_32k_page_defaults_q128():
    run_case(W.QWEN3B_32K_PAGE_DEFAULTS_Q128, query_stride=1)


def test_llama8b_128k_text():
    # One query head of each of the 8 KV groups and the last head.
    w = W.LLAMA8B_128K_TEXT
    run_case(w, query_stride=5, stride=127)
