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


def merge_cases(count=40, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        P = int(rng.choice([1, 2, int(rng.integers(3, 12)), int(rng.integers(12, 41))]))
        R = int(rng.choice([1, int(rng.integers(2, 64)), int(rng.integers(64, 300))]))
        H = int(rng.integers(1, 17))
        D = int(rng.choice([4, 8, 60, 64, 128, 132]))
        bf16 = bool(rng.random() < 0.5)
        pad_row = int(rng.choice([0, 0, 4, 36]))     # extra elements per output row
        pad_lse = int(rng.choice([0, 0, 3, 50]))     # extra elements per LSE head row
        out.append((i, P, R, H, D, bf16, pad_row, pad_lse))
    # Grids of at least 512 workgroups (R*H*D/4 >= 131072 threads), which
    # take the shallow load ring (two partials in flight), with partition
    # counts below, at and above the ring's depth, odd and even.
    out += [(count, 1, 1024, 16, 128, True, 0, 0), (count + 1, 2, 1024, 16, 128, False, 4, 3),
            (count + 2, 3, 700, 28, 128, True, 36, 0), (count + 3, 5, 600, 32, 64, False, 0, 50),
            (count + 4, 9, 512, 32, 132, True, 0, 0)]
    return out


@pytest.mark.parametrize("case", merge_cases(), ids=lambda c: "P{1}_R{2}_H{3}_D{4}_{5}_pad{6}_{7}".format(
    *c[:5], "bf16" if c[5] else "f32", c[6], c[7]))
def test_random_merge(case):
    # spava_lse_merge on random partition counts, rows, heads, widths (any
    # multiple of 4), output dtypes and output strides, with whole partials,
    # single (row, head) entries and whole rows at LSE = -inf, and LSE
    # spreads from 0 to 80 (weights far below float32's range).
    i, P, R, H, D, bf16, pad_row, pad_lse = case
    rng = np.random.default_rng(1000 + i)
    o_part = rng.standard_normal((P, R, H, D)).astype(np.float32)
    spread = float(rng.choice([0.0, 1.0, 5.0, 80.0]))
    lse_part = (rng.standard_normal((P, H, R)) * spread + rng.standard_normal()).astype(np.float32)
    lse_part[rng.random((P, H, R)) < 0.1] = -np.inf
    if P > 1:
        lse_part[int(rng.integers(P))] = -np.inf
    lse_part[:, :, int(rng.integers(R))] = -np.inf
    row_stride, head_stride = H * D + pad_row, R + pad_lse
    dt = torch.bfloat16 if bf16 else torch.float32
    o_full = torch.full((R, row_stride), float("nan"), dtype=dt, device="cuda")
    lse_full = torch.full((H, head_stride), float("nan"), dtype=torch.float32, device="cuda")
    S.spava_lse_merge(torch.from_numpy(o_part).cuda(), torch.from_numpy(lse_part).cuda(), o_full, row_stride,
                      lse_full, head_stride)
    torch.cuda.synchronize()
    ro, rl = O.lse_merge(o_part, lse_part.transpose(0, 2, 1))
    o = np64(o_full[:, :H * D].reshape(R, H, D))
    lse = np64(lse_full[:, :R]).T
    # O: the float32 merge, then (bf16 outputs) one round-to-nearest to 8
    # significant bits, at most 2^-8 of the value; LSE: float32 of
    # magnitude up to a few hundred here, so a relative bound.
    rel_o = 2.0 ** -8 if bf16 else 2e-6
    err_o = np.abs(o - ro) - (rel_o * np.abs(ro) + 1e-5)
    assert err_o.max() <= 0, f"merge O off by {err_o.max():.3e} beyond the bound"
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse), fin) and (lse[~fin] == -np.inf).all()
    err_l = np.abs(lse[fin] - rl[fin]) - (2e-5 + 4e-7 * np.abs(rl[fin]))
    assert err_l.size == 0 or err_l.max() <= 0, f"merge LSE off by {err_l.max():.3e} beyond the bound"
    assert (o[~fin] == 0).all()
    # the padding of the strided outputs is left alone
    if pad_row:
        assert torch.isnan(o_full[:, H * D:].float()).all()
    if pad_lse:
        assert torch.isnan(lse_full[:, R:]).all()
