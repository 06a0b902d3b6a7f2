"""Parity of the context-driven selector and of the selection overlap (through
the C ABI) with the oracle.

Small workloads compare every score and index with
oracle.context_block_scores / select_passing; the full-size 32K workload
compares every score and index of sampled (block, KV head) pairs, which the
oracle scores on those pairs' slices of q and k.  The overlap kernel is
compared exactly with oracle.kv_overlap on the oracle's own two selections.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import sequence_approximate_attention_amd as S
import workloads as W
from gpu_helpers import check_idx, dev_inputs, np64

pytestmark = pytest.mark.gpu

REL_TOL = 1e-5   # scores: float32 probabilities summed in float64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()
    yield


def run_context(w, x):
    plan = S.plan_for(w)
    q, k, _ = dev_inputs(x, w)
    scores = torch.empty((w.n_hosts, w.n_kv_heads, w.host_len), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.n_hosts, w.n_kv_heads, w.lp), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(256, S.spava_score_topk_context_ws_bytes(plan)), dtype=torch.uint8, device="cuda")
    S.spava_score_topk_context(plan, q, k, scores, idx, ws)
    torch.cuda.synchronize()
    return np64(scores), idx.cpu().numpy()


def check_rel(got, want, what):
    err = np.abs(got - want) / np.maximum(np.abs(want), 1e-30)
    assert err.max() < REL_TOL, f"{what}: scores rel err {err.max():.2e}"
    return float(err.max())


SMALL = [
    W.small_workload("bf16"),
    W.small_workload("bf16", Hq=8, Hkv=2, d=64, la=0, V=4, L=77, n_q=9, lp=77, seed=8),
    W.small_workload("bf16", Hq=7, Hkv=1, d=128, la=130, V=2, L=200, n_q=33, lp=0, seed=9),
    W.small_workload("bf16", Hq=4, Hkv=4, d=128, la=5, V=5, L=64, n_q=1, lp=1, seed=10),
    W.small_workload("bf16", Hq=2, Hkv=1, d=128, la=64, V=1, L=300, n_q=0, lp=17, seed=11),
    # several key chunks of 512 and more than 4096 scoring rows (L * G = 5600)
    W.small_workload("bf16", Hq=8, Hkv=1, d=128, la=16, V=2, L=700, n_q=5, lp=100, seed=13),
    W.small_workload("bf16", Hq=16, Hkv=2, d=64, la=0, V=1, L=1100, n_q=0, lp=275, seed=14),
    # fewer block tokens than one 32-row chunk: chunks span several heads
    W.small_workload("bf16", Hq=6, Hkv=1, d=128, la=3, V=3, L=5, n_q=2, lp=2, seed=15),
    W.small_workload("f32", Hq=4, Hkv=2, d=128, la=40, V=3, L=90, n_q=12, lp=30, seed=12),
    W.small_workload("f32", Hq=2, Hkv=1, d=64, la=0, V=2, L=130, n_q=0, lp=64, seed=16),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_context_selection(w):
    print(f"[context] {w.name}", flush=True)
    x = W.make_inputs(w)
    want = O.context_block_scores(x["q"], x["k"], w.n_anchor, w.n_hosts, w.host_len, w.n_query)
    got, idx = run_context(w, x)
    check_rel(got, want, w.name)
    check_idx(want, idx, O.select_passing(want, w.lp), w.lp)


def test_context_first_and_last_keys():
    # Closed forms of the causal sums: token 0 sees only key 0, so key 0
    # collects at least G (one per head); the last key is seen by the last
    # token only.  Checked on the GPU scores, beside the full comparison.
    w = W.small_workload("bf16", Hq=4, Hkv=2, d=128, la=8, V=2, L=96, n_q=4, lp=8, seed=17)
    x = W.make_inputs(w)
    got, _ = run_context(w, x)
    assert (got[:, :, 0] >= w.group * (1 - 1e-6)).all()
    assert (got[:, :, -1] <= w.group * (1 + 1e-6)).all()
    # Every token's probabilities sum to one: sum over keys = L * G.
    np.testing.assert_allclose(got.sum(axis=2), w.host_len * w.group, rtol=1e-5)


FULL = [W.QWEN3B_32K, W.QWEN3B_32K_PAGE_DEFAULTS]


@pytest.mark.parametrize("w", FULL, ids=lambda w: w.name)
def test_fullsize_context_selection_sampled_pairs(w):
    """All V * Hkv lists are computed in the benchmark's launch; the oracle
    scores the first and last blocks on KV heads 0 and Hkv - 1."""
    print(f"[context] {w.name} full size", flush=True)
    x = W.make_inputs(w)
    got, idx = run_context(w, x)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got.sum(axis=2), w.host_len * w.group, rtol=1e-5)
    G, L, d = w.group, w.host_len, w.head_dim
    for h in sorted({0, w.n_hosts - 1}):
        for g in sorted({0, w.n_kv_heads - 1}):
            b0 = w.n_anchor + h * L
            qs = x["q"][b0:b0 + L, g * G:(g + 1) * G]
            ks = x["k"][b0:b0 + L, g:g + 1]
            want = O.context_block_scores(qs, ks, 0, 1, L, 0, scale=1.0 / math.sqrt(d))
            err = check_rel(got[h:h + 1, g:g + 1], want, f"{w.name} block {h} head {g}")
            n_diff = check_idx(want, idx[h:h + 1, g:g + 1], O.select_passing(want, w.lp), w.lp)
            print(f"[context] block {h} KV head {g}: rel err {err:.2e}, near-tie index differences {n_diff}",
                  flush=True)


def _overlap(a, b):
    counts = torch.empty(a.shape[:-1], dtype=torch.int32, device="cuda")
    S.spava_kv_overlap(torch.from_numpy(np.ascontiguousarray(a)).cuda(),
                       torch.from_numpy(np.ascontiguousarray(b)).cuda(), counts)
    torch.cuda.synchronize()
    return counts.cpu().numpy()


@pytest.mark.parametrize("w", [SMALL[0], SMALL[5], SMALL[6]], ids=lambda w: w.name)
def test_overlap_of_the_two_selections(w):
    x = W.make_inputs(w)
    idx_q = O.select_passing(O.block_scores(x["q"], x["k"], w.n_anchor, w.n_hosts, w.host_len, w.n_query), w.lp)
    idx_c = O.select_passing(O.context_block_scores(x["q"], x["k"], w.n_anchor, w.n_hosts, w.host_len,
                                                    w.n_query), w.lp)
    got = _overlap(idx_q, idx_c)
    np.testing.assert_array_equal(got, O.kv_overlap(idx_q, idx_c))
    np.testing.assert_array_equal(_overlap(idx_q, idx_q), np.full(idx_q.shape[:2], w.lp))


def test_overlap_random_lists_and_invalid_order():
    rng = np.random.default_rng(21)
    n, L, lp = 37, 5000, 1000
    a = np.stack([np.sort(rng.choice(L, lp, replace=False)) for _ in range(n)]).astype(np.int32)
    b = np.stack([np.sort(rng.choice(L, lp, replace=False)) for _ in range(n)]).astype(np.int32)
    b[3] = a[3]                              # identical
    b[4] = np.arange(L - lp, L)              # top of the range
    want = O.kv_overlap(a[:, None], b[:, None])[:, 0]
    np.testing.assert_array_equal(_overlap(a, b), want)
    # A list that is not strictly ascending is reported as -1.
    bad = b.copy()
    bad[7, [10, 11]] = bad[7, [11, 10]]
    bad[9, 20] = bad[9, 19]
    got = _overlap(a, bad)
    assert got[7] == -1 and got[9] == -1
    keep = [i for i in range(n) if i not in (7, 9)]
    np.testing.assert_array_equal(got[keep], want[keep])
    # lp = 1 and lp = 0
    np.testing.assert_array_equal(_overlap(a[:, :1], a[:, :1]), np.ones(n, dtype=np.int32))
    np.testing.assert_array_equal(_overlap(a[:, :0], b[:, :0]), np.zeros(n, dtype=np.int32))
