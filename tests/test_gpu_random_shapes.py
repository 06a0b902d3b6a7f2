"""Parity on a seeded sweep of random small shapes (workloads.random_small_workloads:
head grouping, width, anchor, hosts, block, query and passing lengths drawn
at random, a few float32), through the C ABI.

Every shape compares every score and index with the oracle and, on the
oracle's selection, every attention output element by element; shapes with
query rows also run the two-phase (Figure 5) order, whose scores come from
the query partials and whose attention must equal the one-call order's bit
for bit; bf16 shapes also run the context-driven selector.  Two shapes in
three also run with q, k, v as views of a packed QKV buffer or of head-major
tensors, which must give bit-identical results.  The copy ranges of the same
shapes and layouts are checked on the CPU by tests/test_copy_bounds.py.
"""
import numpy as np
import pytest
import torch

import oracle as O
import sequence_approximate_attention_amd as S
import workloads as W
from gpu_helpers import TOL, check_close, check_idx, dev_inputs, np64
from test_gpu_strides import heads_major, packed

pytestmark = pytest.mark.gpu

REL_TOL = 1e-5
SHAPES = W.random_small_workloads()
LAYOUTS = (None, packed, heads_major)   # by shape index modulo 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()
    yield


def check_scores(got, want, what):
    err = np.abs(np64(got) - want) / np.maximum(np.abs(want), 1e-30)
    assert err.max() < REL_TOL, f"{what}: scores rel err {err.max():.2e}"


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_random_shape(w):
    print(f"[random] {w.name}", flush=True)
    x = W.make_inputs(w)
    ref = O.approx_prefill(x["q"], x["k"], x["v"], w.n_anchor, w.n_hosts, w.host_len, w.n_query, w.lp)
    plan = S.plan_for(w)
    q, k, v = dev_inputs(x, w)
    tol = TOL[w.dtype]

    b = S.prefill(plan, q, k, v)
    torch.cuda.synchronize()
    check_scores(b.scores, ref["scores"], "one pass")
    check_idx(ref["scores"], b.idx.cpu().numpy(), ref["idx"], w.lp)

    # Attention on the oracle's selection, both orders.
    idx_o = torch.from_numpy(ref["idx"]).cuda()
    b0 = S.prefill(plan, q, k, v, idx=idx_o)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np64(b0.kp), ref["kp"])
    np.testing.assert_array_equal(np64(b0.vp), ref["vp"])
    check_close(np64(b0.o), ref["O"], tol["o_max"], tol["o_mean"], "O")
    check_close(np64(b0.lse), ref["LSE"], tol["lse_max"], None, "LSE")
    if w.n_query:
        check_close(np64(b0.o_part), ref["O_part"], tol["o_max"], tol["o_mean"], "O_part")
        check_close(np64(b0.lse_part), ref["LSE_part"], tol["lse_max"], None, "LSE_part")

        bp = S.prefill(plan, q, k, v, partials_first=True)
        torch.cuda.synchronize()
        check_scores(bp.scores, ref["scores"], "from the query partials")
        check_idx(ref["scores"], bp.idx.cpu().numpy(), ref["idx"], w.lp)
        b1 = S.prefill(plan, q, k, v, idx=idx_o, partials_first=True)
        torch.cuda.synchronize()
        same = (lambda a, c: torch.equal(a.view(torch.int16), c.view(torch.int16))) if w.dtype == W.BF16 \
            else torch.equal
        assert same(b1.o, b0.o) and torch.equal(b1.lse, b0.lse)
        assert torch.equal(b1.o_part, b0.o_part) and torch.equal(b1.lse_part, b0.lse_part)

    def context(p, qq, kk):
        scores = torch.empty((w.n_hosts, w.n_kv_heads, w.host_len), dtype=torch.float32, device="cuda")
        idx = torch.empty((w.n_hosts, w.n_kv_heads, w.lp), dtype=torch.int32, device="cuda")
        ws = torch.empty(max(256, S.spava_score_topk_context_ws_bytes(p)), dtype=torch.uint8, device="cuda")
        S.spava_score_topk_context(p, qq, kk, scores, idx, ws)
        torch.cuda.synchronize()
        return scores, idx

    if w.dtype == W.BF16:
        want = O.context_block_scores(x["q"], x["k"], w.n_anchor, w.n_hosts, w.host_len, w.n_query)
        scores, idx = context(plan, q, k)
        check_scores(scores, want, "context selector")
        check_idx(want, idx.cpu().numpy(), O.select_passing(want, w.lp), w.lp)

    layout = LAYOUTS[SHAPES.index(w) % 3]
    if layout is not None:
        qs, ks, vs = layout(q, k, v)
        ps = plan.with_strides(qs, ks, vs)
        eq = (lambda a, c: torch.equal(a.view(torch.int16), c.view(torch.int16))) if w.dtype == W.BF16 \
            else torch.equal
        bs = S.prefill(ps, qs, ks, vs)
        torch.cuda.synchronize()
        for name in ("scores", "idx", "kp", "vp", "o", "lse", "o_part", "lse_part"):
            assert eq(getattr(bs, name), getattr(b, name)), f"{layout.__name__}: {name}"
        if w.n_query:
            bps = S.prefill(ps, qs, ks, vs, partials_first=True)
            torch.cuda.synchronize()
            for name in ("scores", "idx", "o", "lse", "o_part", "lse_part"):
                assert eq(getattr(bps, name), getattr(bp, name)), f"{layout.__name__} partials-first: {name}"
        if w.dtype == W.BF16:
            s2, i2 = context(ps, qs, ks)
            assert torch.equal(s2, scores) and torch.equal(i2, idx), f"{layout.__name__}: context selector"
