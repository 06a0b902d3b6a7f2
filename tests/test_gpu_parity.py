"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small workloads are compared element by element on every output; the
full-size workloads compare every score and index, and attention on sampled
(token, head) rows computed one by one by the oracle.
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()
    yield


def run_full(w, x, idx=None):
    plan = S.plan_for(w)
    q, k, v = dev_inputs(x, w)
    bufs = S.prefill(plan, q, k, v, idx=idx)
    torch.cuda.synchronize()
    return plan, bufs


def check_scores(bufs, ref, rel_tol=1e-5):
    sc = np64(bufs.scores)
    want = ref["scores"]
    err = np.abs(sc - want) / np.maximum(np.abs(want), 1e-30)
    assert err.max() < rel_tol, f"scores rel err {err.max():.2e}"
    return float(err.max())


def compare_all(w, x, bufs, ref, with_scores=True):
    tol = TOL[w.dtype]
    if with_scores and ref["scores"] is not None:
        check_scores(bufs, ref)
    check_close(np64(bufs.o), ref["O"], tol["o_max"], tol["o_mean"], "O")
    check_close(np64(bufs.lse), ref["LSE"], tol["lse_max"], None, "LSE")
    if w.n_query:
        check_close(np64(bufs.o_part), ref["O_part"], tol["o_max"], tol["o_mean"], "O_part")
        check_close(np64(bufs.lse_part), ref["LSE_part"], tol["lse_max"], None, "LSE_part")


SMALL = [
    W.small_workload("bf16"),
    W.small_workload("bf16", Hq=8, Hkv=2, d=64, la=0, V=4, L=77, n_q=9, lp=77, seed=8),
    W.small_workload("bf16", Hq=7, Hkv=1, d=128, la=130, V=2, L=200, n_q=33, lp=0, seed=9),
    W.small_workload("bf16", Hq=4, Hkv=4, d=128, la=5, V=5, L=64, n_q=1, lp=1, seed=10),
    W.small_workload("bf16", Hq=2, Hkv=1, d=128, la=64, V=1, L=300, n_q=0, lp=17, seed=11),
    W.small_workload("f32", Hq=4, Hkv=2, d=128, la=40, V=3, L=90, n_q=12, lp=30, seed=12),
    # d = 64 with walks of up to 27 key tiles (both V ring slots reused many
    # times, ragged run ends inside tiles)
    W.small_workload("bf16", Hq=4, Hkv=2, d=64, la=300, V=3, L=1000, n_q=40, lp=200, seed=13),
    # blocks of one and two tokens: every walk a single ragged tile
    W.small_workload("bf16", Hq=4, Hkv=2, d=64, la=7, V=6, L=1, n_q=3, lp=1, seed=14),
    W.small_workload("bf16", Hq=6, Hkv=3, d=128, la=0, V=3, L=2, n_q=5, lp=1, seed=15),
]


def test_tiny_f32_full_pipeline():
    w = W.TINY_F32
    x = W.make_inputs(w)
    plan, bufs = run_full(w, x)
    ref = O.approx_prefill(x["q"], x["k"], x["v"], w.n_anchor, w.n_hosts, w.host_len,
                           w.n_query, w.lp)
    check_idx(ref["scores"], bufs.idx.cpu().numpy(), ref["idx"], w.lp)
    if not np.array_equal(bufs.idx.cpu().numpy(), ref["idx"]):
        # A near-tie swap: the attention is compared on the oracle's selection.
        plan, bufs = run_full(w, x, idx=torch.from_numpy(ref["idx"]).cuda())
    np.testing.assert_array_equal(np64(bufs.kp), ref["kp"])
    np.testing.assert_array_equal(np64(bufs.vp), ref["vp"])
    compare_all(w, x, bufs, ref)


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_full_pipeline(w):
    x = W.make_inputs(w)
    ref = O.approx_prefill(x["q"], x["k"], x["v"], w.n_anchor, w.n_hosts, w.host_len,
                           w.n_query, w.lp)
    plan, bufs = run_full(w, x)
    check_idx(ref["scores"], bufs.idx.cpu().numpy(), ref["idx"], w.lp)
    check_scores(bufs, ref)
    # Attention parity on the oracle's own selection (inputs flow oracle -> GPU only).
    plan, bufs2 = run_full(w, x, idx=torch.from_numpy(ref["idx"]).cuda())
    np.testing.assert_array_equal(np64(bufs2.kp), ref["kp"])
    np.testing.assert_array_equal(np64(bufs2.vp), ref["vp"])
    compare_all(w, x, bufs2, ref, with_scores=False)


def test_merge_kernel_matches_oracle():
    rng = np.random.default_rng(3)
    P, R, H, D = 5, 37, 3, 64
    o_part = rng.standard_normal((P, R, H, D)).astype(np.float32)
    lse_part = (rng.standard_normal((P, H, R)) * 3).astype(np.float32)
    lse_part[1, 0, :5] = -np.inf
    lse_part[:, 2, 7] = -np.inf
    o = torch.empty((R, H, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((H, R), dtype=torch.float32, device="cuda")
    S.spava_lse_merge(torch.from_numpy(o_part).cuda(), torch.from_numpy(lse_part).cuda(), o, H * D, lse, R)
    torch.cuda.synchronize()
    ro, rl = O.lse_merge(o_part, lse_part.transpose(0, 2, 1))
    check_close(np64(o), ro, 1e-5, None, "merge O")
    check_close(np64(lse).T, rl, 1e-5, None, "merge LSE")
    assert torch.isneginf(lse[2, 7]).item() and (o[7, 2] == 0).all().item()


def test_uniform_keys_closed_form_bf16():
    # Zero queries: every score ties, the lower indices win, every visible key
    # has weight 1/n: LSE = ln(n) exactly and O = mean of visible values.
    w = W.small_workload("bf16", Hq=4, Hkv=2, d=128, la=32, V=4, L=128, n_q=16, lp=16, seed=5)
    x = W.make_inputs(w)
    for key in ("q", "q16"):
        x[key] = np.zeros_like(x[key])
    plan, bufs = run_full(w, x)
    idx = bufs.idx.cpu().numpy()
    np.testing.assert_array_equal(idx, np.broadcast_to(np.arange(w.lp, dtype=np.int32), idx.shape))
    lse = np64(bufs.lse)
    la, L, lp = w.n_anchor, w.host_len, w.lp
    for t in range(w.n_tokens):
        if t < la:
            n = t + 1
        elif t < la + w.n_hosts * L:
            h = (t - la) // L
            n = la + h * lp + (t - la - h * L) + 1
        else:
            n = t + 1
        assert abs(lse[0, t] - math.log(n)) < 2e-5, (t, lse[0, t], math.log(n))


def test_dense_mode_matches_dense_oracle():
    # One host, no anchor, no query, no passing: plain causal attention.
    w = W.small_workload("bf16", Hq=8, Hkv=2, d=128, la=0, V=1, L=700, n_q=0, lp=0, seed=6)
    x = W.make_inputs(w)
    plan, bufs = run_full(w, x)
    od, ld = O.dense_causal(x["q"], x["k"], x["v"])
    tol = TOL["bf16"]
    check_close(np64(bufs.o), od, tol["o_max"], tol["o_mean"], "dense O")
    check_close(np64(bufs.lse), ld, tol["lse_max"], None, "dense LSE")


def test_bitwise_determinism():
    w = W.small_workload("bf16", Hq=8, Hkv=2, d=128, la=100, V=3, L=260, n_q=40, lp=70, seed=13)
    x = W.make_inputs(w)
    _, b1 = run_full(w, x)
    _, b2 = run_full(w, x)
    for name in ("scores", "idx", "kp", "vp", "o", "lse", "o_part", "lse_part"):
        t1, t2 = getattr(b1, name), getattr(b2, name)
        assert torch.equal(t1.view(torch.uint8) if t1.dtype == torch.bfloat16 else t1,
                           t2.view(torch.uint8) if t2.dtype == torch.bfloat16 else t2), name


def test_scores_may_be_null():
    # Without a scores buffer the selection is the same (scores live in ws).
    w = W.small_workload("bf16", Hq=8, Hkv=2, d=128, la=40, V=3, L=300, n_q=24, lp=50, seed=23)
    x = W.make_inputs(w)
    plan = S.plan_for(w)
    q, k, _ = dev_inputs(x, w)
    ws = torch.empty(S.spava_score_topk_ws_bytes(plan), dtype=torch.uint8, device="cuda")
    scores = torch.empty((w.n_hosts, w.n_kv_heads, w.host_len), dtype=torch.float32, device="cuda")
    idx_a = torch.empty((w.n_hosts, w.n_kv_heads, w.lp), dtype=torch.int32, device="cuda")
    idx_b = torch.empty_like(idx_a)
    S.spava_score_topk(plan, q, k, scores, idx_a, ws)
    S.spava_score_topk(plan, q, k, None, idx_b, ws)
    ctx_ws = torch.empty(S.spava_score_topk_context_ws_bytes(plan), dtype=torch.uint8, device="cuda")
    idx_c = torch.empty_like(idx_a)
    S.spava_score_topk_context(plan, q, k, None, idx_c, ctx_ws)
    torch.cuda.synchronize()
    assert torch.equal(idx_a, idx_b)
    sc = O.block_scores(x["q"], x["k"], w.n_anchor, w.n_hosts, w.host_len, w.n_query)
    check_idx(sc, idx_b.cpu().numpy(), O.select_passing(sc, w.lp), w.lp)
    scc = O.context_block_scores(x["q"], x["k"], w.n_anchor, w.n_hosts, w.host_len, w.n_query)
    check_idx(scc, idx_c.cpu().numpy(), O.select_passing(scc, w.lp), w.lp)


@pytest.mark.parametrize("lp", [0, 37, 256])
def test_exact_rows_match_the_dense_plan_on_gpu(lp):
    # Anchor, host-0 and query rows see their whole prefix, so the
    # approximate run and the library's own dense plan (one host over the
    # same N tokens) agree there for any lp; with lp = L every row agrees.
    w = W.small_workload("bf16", Hq=8, Hkv=2, d=128, la=90, V=3, L=256, n_q=40, lp=lp, seed=29)
    x = W.make_inputs(w)
    plan, approx = run_full(w, x)
    N = w.n_tokens
    dense_plan = S.Plan(0, 1, N, 0, w.n_q_heads, w.n_kv_heads, w.head_dim, 0, S.SPAVA_BF16)
    q, k, v = dev_inputs(x, w)
    dense = S.prefill(dense_plan, q, k, v)
    torch.cuda.synchronize()
    L, la = w.host_len, w.n_anchor
    rows = np.r_[0:la + L, la + w.n_hosts * L:N] if lp < L else np.arange(N)
    tol = TOL["bf16"]
    check_close(np64(approx.o)[rows], np64(dense.o)[rows], tol["o_max"], tol["o_mean"], "O vs dense plan")
    check_close(np64(approx.lse)[:, rows], np64(dense.lse)[:, rows], tol["lse_max"], None, "LSE vs dense plan")
    od, ld = O.dense_causal(x["q"], x["k"], x["v"])
    check_close(np64(dense.o), od, tol["o_max"], tol["o_mean"], "dense plan O vs oracle")


@pytest.mark.parametrize("L,lp", [(1000, 333), (5000, 700), (9000, 64), (16384, 4096), (17000, 300)])
def test_selection_across_list_lengths(L, lp):
    # The top-lp kernel keeps up to 4, 8 or 16 keys per thread in registers
    # (lists of up to 4096, 8192, 16384 keys) and reads longer lists again
    # per pass; every size class against the oracle's scores and selection.
    w = W.small_workload("bf16", Hq=4, Hkv=2, d=64, la=0, V=1, L=L, n_q=6, lp=lp, seed=31)
    x = W.make_inputs(w)
    plan = S.plan_for(w)
    q, k, _ = dev_inputs(x, w)
    ws = torch.empty(S.spava_score_topk_ws_bytes(plan), dtype=torch.uint8, device="cuda")
    scores = torch.empty((w.n_hosts, w.n_kv_heads, L), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.n_hosts, w.n_kv_heads, lp), dtype=torch.int32, device="cuda")
    S.spava_score_topk(plan, q, k, scores, idx, ws)
    torch.cuda.synchronize()
    want = O.block_scores(x["q"], x["k"], w.n_anchor, w.n_hosts, w.host_len, w.n_query)
    got = np64(scores)
    err = np.abs(got - want) / np.maximum(np.abs(want), 1e-30)
    assert err.max() < 1e-5, f"scores rel err {err.max():.2e}"
    check_idx(want, idx.cpu().numpy(), O.select_passing(want, lp), lp)


@pytest.mark.parametrize("L", [1500, 9000, 17000])
def test_selection_with_zero_and_equal_scores(L):
    # Lists the radix passes of the top-lp kernel meet at their extremes:
    # block 0 of KV head 0 scores 70 % of its keys exactly 0 (their logits lie
    # thousands below every query row's maximum, so exp underflows in float32
    # and float64 alike) and keeps more keys than score above 0, so the
    # threshold is 0 and the kept zeros are the lowest-indexed ones, with
    # the full 32-bit range of order keys to split; block 1 of KV head 0
    # holds one key repeated, so every score is equal and the kernel takes
    # the lp lowest indices without a radix pass; the other lists are drawn
    # as usual.  The list lengths take the kernel's 4- and 16-keys-per-thread
    # register paths and the path that re-reads the list per pass.
    w = W.small_workload("bf16", Hq=4, Hkv=2, d=64, la=0, V=3, L=L, n_q=6, lp=int(0.4 * L), seed=41)
    x = W.make_inputs(w)
    G, n0 = w.group, w.n_tokens - w.n_query
    x["q16"][n0:, :G] &= np.uint16(0x7FFF)                   # query rows of group 0: |q|
    x["q"][n0:, :G] = np.abs(x["q"][n0:, :G])
    rng = np.random.default_rng(41)
    bad = rng.choice(L, int(0.7 * L), replace=False)
    x["k"][bad, 0] = -512.0                                 # block 0, KV head 0
    x["k16"][bad, 0] = W.bf16_bits(np.full(w.head_dim, -512.0, np.float32))
    x["k"][L:2 * L, 0] = x["k"][L + 7, 0]                   # block 1, KV head 0: one key
    x["k16"][L:2 * L, 0] = x["k16"][L + 7, 0]
    plan = S.plan_for(w)
    q, k, _ = dev_inputs(x, w)
    ws = torch.empty(S.spava_score_topk_ws_bytes(plan), dtype=torch.uint8, device="cuda")
    scores = torch.empty((w.n_hosts, w.n_kv_heads, L), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.n_hosts, w.n_kv_heads, w.lp), dtype=torch.int32, device="cuda")
    S.spava_score_topk(plan, q, k, scores, idx, ws)
    torch.cuda.synchronize()
    want = O.block_scores(x["q"], x["k"], w.n_anchor, w.n_hosts, w.host_len, w.n_query)
    assert (want[0, 0, bad] == 0).all() and (want[0, 0] > 0).sum() < w.lp
    assert (want[1, 0] == want[1, 0, 0]).all()
    got = np64(scores)
    assert (got[0, 0, bad] == 0).all() and (got[1, 0] == got[1, 0, 0]).all()
    err = np.abs(got - want) / np.maximum(np.abs(want), 1e-30)
    assert err.max() < 1e-5, f"scores rel err {err.max():.2e}"
    sel = O.select_passing(want, w.lp)
    np.testing.assert_array_equal(idx.cpu().numpy()[:2, 0], sel[:2, 0])   # ties: exact
    check_idx(want, idx.cpu().numpy(), sel, w.lp)


@pytest.mark.parametrize("d,L", [(64, 1000), (128, 777)])
def test_column_sums_on_a_large_grid(d, L):
    # V * Hkv * ceil(L / 256) >= 1024 column-sum workgroups: the form with
    # one 4-wave group per workgroup (three to a CU), here with a ragged last
    # group of keys. Every score and index against the oracle, from the
    # one-pass scoring and from the query partials' LSEs.
    w = W.small_workload("bf16", Hq=8, Hkv=8, d=d, la=0, V=32, L=L, n_q=5, lp=100, seed=37)
    assert w.n_hosts * w.n_kv_heads * math.ceil(L / 256) >= 1024
    x = W.make_inputs(w)
    plan = S.plan_for(w)
    q, k, v = dev_inputs(x, w)
    b = S.alloc_buffers(plan, q.device)
    want = O.block_scores(x["q"], x["k"], w.n_anchor, w.n_hosts, w.host_len, w.n_query)
    sel = O.select_passing(want, w.lp)
    S.spava_score_topk(plan, q, k, b.scores, b.idx, b.ws_score)
    torch.cuda.synchronize()
    err = np.abs(np64(b.scores) - want) / np.maximum(np.abs(want), 1e-30)
    assert err.max() < 1e-5, f"one-pass scores rel err {err.max():.2e}"
    check_idx(want, b.idx.cpu().numpy(), sel, w.lp)
    S.spava_attn_fwd_phase(plan, S.SPAVA_PHASE_LOCAL, q, k, v, b.kp, b.vp, b.o, b.lse, b.o_part, b.lse_part)
    scores = torch.zeros_like(b.scores)
    idx = torch.zeros_like(b.idx)
    S.spava_score_topk_from_partials(plan, q, k, b.lse_part, scores, idx)
    torch.cuda.synchronize()
    err = np.abs(np64(scores) - want) / np.maximum(np.abs(want), 1e-30)
    assert err.max() < 1e-5, f"from-partials scores rel err {err.max():.2e}"
    check_idx(want, idx.cpu().numpy(), sel, w.lp)
