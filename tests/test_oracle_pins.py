"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test checks the oracle against a closed form, a library routine on a
case the method must reduce to, an invariant of the definitions, or brute
force on tiny inputs.  Chosen so that a dropped term, a wrong index, a wrong
visibility rule or a transposed operand fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_qkv(rng, N, Hq, Hkv, d, scale=1.0):
    q = rng.standard_normal((N, Hq, d)) * scale
    k = rng.standard_normal((N, Hkv, d)) * scale
    v = rng.standard_normal((N, Hkv, d))
    return q, k, v


def sdpa(q, k, v, mask=None, causal=False):
    """torch's scaled_dot_product_attention in float64, GQA by repeat_interleave.

    q: [N, Hq, d]; k, v: [N, Hkv, d]; mask: bool [N, N] (True = visible).
    """
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2))).repeat_interleave(G, 0)[None]
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2))).repeat_interleave(G, 0)[None]
    m = None if mask is None else torch.from_numpy(mask)
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=causal)
    return out[0].numpy().transpose(1, 0, 2)


def approx_mask(la, V, L, n_q, idx, g):
    """Visibility over the ORIGINAL token order for KV group g: a second,
    gather-free statement of who sees whom (context tokens see the anchor,
    the selected tokens of earlier blocks and their own block causally;
    anchor and query tokens see every earlier token)."""
    N = la + V * L + n_q
    m = np.tril(np.ones((N, N), dtype=bool))
    for h in range(V):
        b0 = la + h * L
        rows = slice(b0, b0 + L)
        m[rows, la:b0] = False
        for hp in range(h):
            m[rows, la + hp * L + idx[hp, g].astype(np.int64)] = True
    return m


SHAPES = [
    # (la, V, L, n_q, Hq, Hkv, d)
    (3, 2, 5, 3, 2, 1, 8),
    (8, 3, 8, 7, 4, 2, 8),
    (0, 4, 5, 1, 4, 1, 16),
    (5, 1, 16, 0, 2, 2, 8),
    (8, 2, 16, 3, 4, 4, 64),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_dense_causal_matches_torch_sdpa(shape):
    la, V, L, n_q, Hq, Hkv, d = shape
    rng = np.random.default_rng(1)
    N = la + V * L + n_q
    q, k, v = rand_qkv(rng, N, Hq, Hkv, d)
    o, _ = O.dense_causal(q, k, v)
    np.testing.assert_allclose(o, sdpa(q, k, v, causal=True), rtol=0, atol=1e-12)


def test_lse_closed_form_zero_logits():
    # All logits 0: LSE of causal row t is ln(t+1) and O is the mean of v[0..t].
    N, d = 9, 8
    q = np.zeros((N, 2, d))
    k = np.random.default_rng(0).standard_normal((N, 1, d))
    v = np.arange(N, dtype=np.float64)[:, None, None] * np.ones((1, 1, d))
    o, lse = O.dense_causal(q, k, v)
    t = np.arange(N)
    np.testing.assert_allclose(lse[0], np.log(t + 1), atol=1e-14)
    np.testing.assert_allclose(o[:, 1, 0], t / 2.0, atol=1e-12)


def test_lse_shift_invariance():
    # Adding w to every key with q.w = c shifts every logit by c*scale:
    # LSE shifts by exactly that and O does not move.
    rng = np.random.default_rng(3)
    N, d = 12, 16
    q, k, v = rand_qkv(rng, N, 2, 1, d)
    q[:, :, -1] = 0.0
    q[:, :, 0] = 1.0
    w = np.zeros(d)
    w[0] = 2.5                       # q.w = 2.5 for every query row
    o1, l1 = O.dense_causal(q, k, v)
    o2, l2 = O.dense_causal(q, k + w, v)
    np.testing.assert_allclose(l2 - l1, 2.5 / math.sqrt(d), atol=1e-12)
    np.testing.assert_allclose(o2, o1, atol=1e-12)


def test_score_closed_form_golden():
    g = json.load(open(os.path.join(GOLDEN, "score_closed_form.json")))
    s = g["shape"]
    la, V, L, n_q, Hq, Hkv, d = s["la"], s["V"], s["L"], s["n_q"], s["Hq"], s["Hkv"], s["d"]
    N = la + V * L + n_q
    q = np.zeros((N, Hq, d))
    k = np.zeros((N, Hkv, d))
    q[la + V * L:, :, 0] = math.sqrt(d)
    k[:la, 0, 0] = g["anchor_logit"]
    k[la:la + L, 0, 0] = g["block0_logits"]
    k[la + L:la + 2 * L, 0, 0] = g["block1_logits"]
    q[:la + V * L, :, 0] = 100.0     # context-token queries must not vote
    sc = O.block_scores(q, k, la, V, L, n_q)
    np.testing.assert_allclose(sc, np.array(g["expected_scores"]), atol=1e-13)
    np.testing.assert_array_equal(O.select_passing(sc, 2), np.array(g["expected_top2_ascending"]))


@pytest.mark.parametrize("shape", SHAPES)
def test_scores_sum_to_row_count(shape):
    # Every softmax row sums to one: the block's scores sum to n_q * G.
    la, V, L, n_q, Hq, Hkv, d = shape
    rng = np.random.default_rng(5)
    q, k, _ = rand_qkv(rng, la + V * L + n_q, Hq, Hkv, d, scale=2.0)
    sc = O.block_scores(q, k, la, V, L, n_q)
    np.testing.assert_allclose(sc.sum(axis=2), n_q * (Hq // Hkv), rtol=1e-13, atol=1e-13)
    assert (sc >= 0).all()


def test_scores_depend_only_on_block_query_and_group():
    la, V, L, n_q, Hq, Hkv, d = 4, 3, 6, 3, 4, 2, 8
    rng = np.random.default_rng(9)
    N = la + V * L + n_q
    q, k, _ = rand_qkv(rng, N, Hq, Hkv, d)
    base = O.block_scores(q, k, la, V, L, n_q)
    q2 = q.copy()
    q2[:la + V * L] = rng.standard_normal(q2[:la + V * L].shape)       # context/anchor queries
    k2 = k.copy()
    k2[la + L:la + 2 * L] *= 5.0                                        # block 1's keys only
    k2[:la] += 10.0                                                     # anchor keys
    s2 = O.block_scores(q2, k2, la, V, L, n_q)
    np.testing.assert_allclose(s2[0], base[0], atol=1e-13)
    np.testing.assert_allclose(s2[2], base[2], atol=1e-13)
    assert np.abs(s2[1] - base[1]).max() > 1e-3
    # Heads of group 1 change: group 0's scores stay.
    q3 = q.copy()
    q3[la + V * L:, 2:] = rng.standard_normal(q3[la + V * L:, 2:].shape)
    s3 = O.block_scores(q3, k, la, V, L, n_q)
    np.testing.assert_allclose(s3[:, 0], base[:, 0], atol=1e-13)
    assert np.abs(s3[:, 1] - base[:, 1]).max() > 1e-3


def _brute_select(scores, lp):
    """The unique subset S of size lp that beats every outsider in the
    order (score desc, index asc), found by enumerating all subsets."""
    L = len(scores)
    found = []
    for S in itertools.combinations(range(L), lp):
        inside = set(S)
        ok = all((scores[i] > scores[j]) or (scores[i] == scores[j] and i < j)
                 for i in inside for j in range(L) if j not in inside)
        if ok:
            found.append(list(S))
    assert len(found) == 1
    return found[0]


def test_selection_brute_force_with_ties():
    rng = np.random.default_rng(11)
    for trial in range(40):
        L = int(rng.integers(1, 9))
        vals = rng.integers(0, 4, size=L).astype(np.float64)           # many exact ties
        sc = vals[None, None, :]
        for lp in range(L + 1):
            got = O.select_passing(sc, lp)[0, 0].tolist()
            assert got == _brute_select(vals, lp), (vals, lp)


@pytest.mark.parametrize("shape", SHAPES)
def test_full_selection_equals_dense(shape):
    # lp = L: every key passes, so the method is exact causal attention.
    la, V, L, n_q, Hq, Hkv, d = shape
    rng = np.random.default_rng(13)
    N = la + V * L + n_q
    q, k, v = rand_qkv(rng, N, Hq, Hkv, d)
    r = O.approx_prefill(q, k, v, la, V, L, n_q, lp=L)
    od, ld = O.dense_causal(q, k, v)
    np.testing.assert_allclose(r["O"], sdpa(q, k, v, causal=True), atol=1e-12)
    np.testing.assert_allclose(r["LSE"], ld, atol=1e-12)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("lp_frac", [0.0, 0.3, 0.7])
def test_query_anchor_and_first_host_rows_are_exact(shape, lp_frac):
    la, V, L, n_q, Hq, Hkv, d = shape
    lp = int(lp_frac * L)
    rng = np.random.default_rng(17)
    N = la + V * L + n_q
    q, k, v = rand_qkv(rng, N, Hq, Hkv, d)
    r = O.approx_prefill(q, k, v, la, V, L, n_q, lp=lp)
    od = sdpa(q, k, v, causal=True)
    _, ld = O.dense_causal(q, k, v)
    exact = np.r_[0:la + L, la + V * L:N]           # anchor, host 0, query tokens
    np.testing.assert_allclose(r["O"][exact], od[exact], atol=1e-12)
    np.testing.assert_allclose(r["LSE"][:, exact], ld[:, exact], atol=1e-12)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("lp_frac", [0.0, 0.4, 1.0])
def test_context_rows_match_masked_sdpa(shape, lp_frac):
    # Gather-free restatement: attention over the original sequence with a
    # boolean mask built from the selected indices.
    la, V, L, n_q, Hq, Hkv, d = shape
    lp = int(lp_frac * L)
    rng = np.random.default_rng(19)
    N = la + V * L + n_q
    q, k, v = rand_qkv(rng, N, Hq, Hkv, d)
    r = O.approx_prefill(q, k, v, la, V, L, n_q, lp=lp)
    G = Hq // Hkv
    for g in range(Hkv):
        m = approx_mask(la, V, L, n_q, r["idx"], g)
        heads = slice(g * G, (g + 1) * G)
        ref = sdpa(q[:, heads], k[:, g:g + 1], v[:, g:g + 1], mask=m)
        np.testing.assert_allclose(r["O"][:, heads], ref, atol=1e-12)


def test_single_host_is_dense():
    rng = np.random.default_rng(23)
    for la, L, n_q, lp in [(0, 12, 0, 0), (4, 9, 3, 2), (6, 7, 0, 7)]:
        N = la + L + n_q
        q, k, v = rand_qkv(rng, N, 4, 2, 8)
        r = O.approx_prefill(q, k, v, la, 1, L, n_q, lp=lp)
        np.testing.assert_allclose(r["O"], sdpa(q, k, v, causal=True), atol=1e-12)


def test_uniform_keys_golden():
    g = json.load(open(os.path.join(GOLDEN, "uniform_keys_tiny.json")))
    s = g["shape"]
    la, V, L, n_q, lp, Hq, Hkv, d = (s[x] for x in ("la", "V", "L", "n_q", "lp", "Hq", "Hkv", "d"))
    N = la + V * L + n_q
    rng = np.random.default_rng(29)
    q = np.zeros((N, Hq, d))
    k = rng.standard_normal((N, Hkv, d))
    v = np.arange(N, dtype=np.float64)[:, None, None] * np.ones((1, Hkv, d))
    r = O.approx_prefill(q, k, v, la, V, L, n_q, lp)
    np.testing.assert_array_equal(r["idx"], np.broadcast_to(np.arange(lp), (V, Hkv, lp)))
    for row in g["rows"]:
        t = row["token"]
        for a in range(Hq):
            assert abs(r["LSE"][a, t] - math.log(row["n_visible"])) < 1e-12
            np.testing.assert_allclose(r["O"][t, a], row["index_sum"] / row["n_visible"], rtol=1e-13)


def test_merge_of_a_partition_equals_attention_over_the_union():
    rng = np.random.default_rng(31)
    R, nk, d = 5, 23, 8
    qr = rng.standard_normal((R, d))
    keys = rng.standard_normal((nk, d))
    vals = rng.standard_normal((nk, d))
    vis = rng.random((R, nk)) < 0.7
    vis[:, 0] = True
    scale = 0.3
    o_all, l_all = O.attend(qr, keys, vals, vis, scale)
    cuts = [0, 4, 5, 13, 23]
    parts = [O.attend(qr, keys[a:b], vals[a:b], vis[:, a:b], scale) for a, b in zip(cuts, cuts[1:])]
    po = np.stack([p[0] for p in parts])
    pl = np.stack([p[1] for p in parts])
    o_m, l_m = O.lse_merge(po, pl)
    np.testing.assert_allclose(o_m, o_all, atol=1e-13)
    np.testing.assert_allclose(l_m, l_all, atol=1e-13)
    perm = [2, 0, 3, 1]
    o_p, l_p = O.lse_merge(po[perm], pl[perm])
    np.testing.assert_allclose(o_p, o_all, atol=1e-13)
    o_1, l_1 = O.lse_merge(po[:1], pl[:1])
    np.testing.assert_allclose(o_1, po[0], atol=1e-15)
    np.testing.assert_allclose(l_1, pl[0], atol=1e-15)


def test_merge_handles_empty_partials():
    o = np.array([[[1.0, 2.0]], [[5.0, 6.0]]])
    lse = np.array([[-math.inf], [0.25]])
    om, lm = O.lse_merge(o, lse)
    np.testing.assert_allclose(om, [[5.0, 6.0]])
    np.testing.assert_allclose(lm, [0.25])
    om, lm = O.lse_merge(o, np.full((2, 1), -math.inf))
    np.testing.assert_array_equal(om, [[0.0, 0.0]])
    assert lm[0] == -math.inf


def test_passing_row_order_does_not_matter():
    la, V, L, n_q, Hq, Hkv, d = 4, 3, 8, 2, 2, 1, 8
    rng = np.random.default_rng(37)
    N = la + V * L + n_q
    q, k, v = rand_qkv(rng, N, Hq, Hkv, d)
    r = O.approx_prefill(q, k, v, la, V, L, n_q, lp=5)
    perm = rng.permutation(5)
    kp2, vp2 = r["kp"][:, :, perm], r["vp"][:, :, perm]
    for h in range(V):
        o1, l1 = O.context_rows(q, k, v, r["kp"], r["vp"], la, V, L, h, 1 / math.sqrt(d))
        o2, l2 = O.context_rows(q, k, v, kp2, vp2, la, V, L, h, 1 / math.sqrt(d))
        np.testing.assert_allclose(o2, o1, atol=1e-13)
        np.testing.assert_allclose(l2, l1, atol=1e-13)


def test_gather_reads_the_right_rows():
    la, V, L = 3, 3, 5
    N = la + V * L
    k = np.arange(N * 2 * 4, dtype=np.float64).reshape(N, 2, 4)
    v = -k
    idx = np.array([[[0, 4], [1, 2]], [[2, 3], [0, 4]], [[1, 4], [3, 4]]], dtype=np.int32)
    kp, vp = O.gather_passing(k, v, idx, la, L)
    for h in range(V):
        for g in range(2):
            for t in range(2):
                row = la + h * L + idx[h, g, t]
                np.testing.assert_array_equal(kp[g, h, t], k[row, g])
                np.testing.assert_array_equal(vp[g, h, t], v[row, g])


def test_sampled_rows_agree_with_full_oracle():
    la, V, L, n_q, Hq, Hkv, d = 6, 3, 10, 4, 4, 2, 8
    rng = np.random.default_rng(41)
    N = la + V * L + n_q
    q, k, v = rand_qkv(rng, N, Hq, Hkv, d)
    r = O.approx_prefill(q, k, v, la, V, L, n_q, lp=3)
    rows = [(t, a) for t in (0, 5, 6, 15, 16, 35, 36, 39) for a in (0, 3)]
    rows += [(t, a) for t in range(N) for a in range(Hq)]   # every row, grouped per host
    o, l = O.sampled_rows(q, k, v, r["kp"], r["vp"], la, V, L, n_q, rows)
    for n, (t, a) in enumerate(rows):
        np.testing.assert_allclose(o[n], r["O"][t, a], atol=1e-13)
        assert abs(l[n] - r["LSE"][a, t]) < 1e-13


# --- The referee's context-driven selector (APB-V review, Referee Report,
# major comment 1; "What would settle it") --------------------------------

@pytest.mark.parametrize("shape", SHAPES)
def test_context_scores_sum_to_block_rows(shape):
    # Every causal softmax row of the block sums to one: L * G per block.
    la, V, L, n_q, Hq, Hkv, d = shape
    rng = np.random.default_rng(21)
    q, k, _ = rand_qkv(rng, la + V * L + n_q, Hq, Hkv, d, scale=2.0)
    sc = O.context_block_scores(q, k, la, V, L, n_q)
    np.testing.assert_allclose(sc.sum(axis=2), L * (Hq // Hkv), rtol=1e-13, atol=1e-12)
    assert (sc >= 0).all()


def test_context_scores_uniform_keys_harmonic_closed_form():
    # Equal keys within a block: token t spreads 1/(t+1) over keys 0..t, so key
    # j collects G * (H_L - H_j) with H_n the n-th harmonic number.
    la, V, L, n_q, Hq, Hkv, d = 3, 2, 9, 2, 6, 2, 8
    rng = np.random.default_rng(3)
    q, k, _ = rand_qkv(rng, la + V * L + n_q, Hq, Hkv, d)
    for h in range(V):
        b0 = la + h * L
        k[b0:b0 + L] = k[b0]               # one key vector per (block, KV head)
    sc = O.context_block_scores(q, k, la, V, L, n_q)
    harm = [sum(1.0 / i for i in range(1, n + 1)) for n in range(L + 1)]
    G = Hq // Hkv
    want = np.array([G * (harm[L] - harm[j]) for j in range(L)])
    for h in range(V):
        for g in range(Hkv):
            np.testing.assert_allclose(sc[h, g], want, rtol=1e-12)


def test_context_scores_first_token_sees_only_itself():
    # The block's first token attends to key 0 alone (diagonal included):
    # with all later keys dominant for every later token, key 0 keeps G.
    la, V, L, n_q, Hq, Hkv, d = 2, 1, 5, 1, 2, 1, 4
    N = la + V * L + n_q
    q = np.zeros((N, Hq, d))
    k = np.zeros((N, Hkv, d))
    q[:, :, 0] = 1.0
    k[la + 1:la + L, 0, 0] = 60.0          # keys 1.. dominate every row that sees them
    sc = O.context_block_scores(q, k, la, V, L, n_q)
    assert abs(sc[0, 0, 0] - Hq) < 1e-12


def test_context_scores_ignore_other_blocks_anchor_and_query():
    la, V, L, n_q, Hq, Hkv, d = 4, 3, 6, 3, 4, 2, 8
    rng = np.random.default_rng(11)
    N = la + V * L + n_q
    q, k, _ = rand_qkv(rng, N, Hq, Hkv, d)
    base = O.context_block_scores(q, k, la, V, L, n_q)
    q2, k2 = q.copy(), k.copy()
    h = 1
    b0 = la + h * L
    outside = np.r_[0:b0, b0 + L:N]
    q2[outside] = rng.standard_normal(q2[outside].shape) * 5
    k2[outside] = rng.standard_normal(k2[outside].shape) * 5
    np.testing.assert_array_equal(O.context_block_scores(q2, k2, la, V, L, n_q)[h], base[h])


def test_context_scores_brute_force_tiny():
    # Pure-Python causal softmax per (token, head): log-sum-exp by math.fsum.
    la, V, L, n_q, Hq, Hkv, d = 1, 2, 4, 1, 4, 2, 3
    rng = np.random.default_rng(17)
    q, k, _ = rand_qkv(rng, la + V * L + n_q, Hq, Hkv, d, scale=1.5)
    sc = O.context_block_scores(q, k, la, V, L, n_q)
    G = Hq // Hkv
    for h in range(V):
        b0 = la + h * L
        for g in range(Hkv):
            tot = [0.0] * L
            for a in range(g * G, g * G + G):
                for t in range(L):
                    logits = [math.fsum(q[b0 + t, a, c] * k[b0 + j, g, c] for c in range(d)) / math.sqrt(d)
                              for j in range(t + 1)]
                    mx = max(logits)
                    z = math.fsum(math.exp(x - mx) for x in logits)
                    for j in range(t + 1):
                        tot[j] += math.exp(logits[j] - mx) / z
            np.testing.assert_allclose(sc[h, g], tot, rtol=1e-12)


def test_context_selection_can_differ_from_query_selection():
    # A key that every context token of the block attends to but the query
    # does not is kept by the context rule and dropped by the query rule.
    la, V, L, n_q, Hq, Hkv, d = 2, 1, 8, 2, 2, 1, 4
    N = la + V * L + n_q
    q = np.zeros((N, Hq, d))
    k = np.zeros((N, Hkv, d))
    b0 = la
    q[b0:b0 + L, :, 0] = 1.0               # context tokens look along e0
    q[la + L:, :, 1] = 1.0                 # query tokens look along e1
    k[b0 + 0, 0, 0] = 30.0                 # key 0: context-relevant only
    k[b0 + 5, 0, 1] = 30.0                 # key 5: query-relevant only
    ctx = O.select_passing(O.context_block_scores(q, k, la, V, L, n_q), 1)
    qry = O.select_passing(O.block_scores(q, k, la, V, L, n_q), 1)
    assert ctx[0, 0].tolist() == [0] and qry[0, 0].tolist() == [5]
    assert O.kv_overlap(ctx, qry)[0, 0] == 0
    assert O.kv_overlap(ctx, ctx)[0, 0] == 1


@pytest.mark.parametrize("lp", [2, 5, 16, 97])
def test_kv_overlap_closed_forms(lp):
    # The overlap is the size of the intersection of two key sets (APB-V
    # review, "What would settle it"), so it is known without set code on
    # lists whose common members follow from arithmetic:
    #   even keys vs multiples of 3: the common keys are the multiples of 6
    #     up to 2 (lp - 1), floor(2 (lp - 1) / 6) + 1 of them;
    #   0..lp-1 vs 1..lp: all but one key are shared, none at equal positions;
    #   a list against itself reversed in position order (still one set): lp;
    #   disjoint halves (evens vs odds): 0.
    # A position-wise comparison of the two lists fails the first two lines;
    # a merge walk that assumes both lists ascending fails the third.
    evens = np.arange(lp) * 2
    threes = np.arange(lp) * 3
    shifted_a = np.arange(lp)
    shifted_b = np.arange(1, lp + 1)
    odds = np.arange(lp) * 2 + 1
    idx_a = np.stack([evens, shifted_a, evens, evens])[None].astype(np.int32)   # [1, 4, lp]
    idx_b = np.stack([threes, shifted_b, evens[::-1], odds])[None].astype(np.int32)
    got = O.kv_overlap(idx_a, idx_b)
    assert got.shape == (1, 4)
    assert got[0].tolist() == [(2 * (lp - 1)) // 6 + 1, lp - 1, lp, 0]


def test_kv_overlap_small_hand_cases():
    # [1, 2] and [2, 3] share key 2 only (position-wise they share nothing);
    # [0, 5, 9] and [5, 9, 11] share 5 and 9 at shifted positions.
    a = np.array([[[1, 2, 0], [0, 5, 9]]], dtype=np.int32)
    b = np.array([[[2, 3, 7], [5, 9, 11]]], dtype=np.int32)
    assert O.kv_overlap(a, b).tolist() == [[1, 2]]
    # Symmetric in its two arguments.
    assert O.kv_overlap(b, a).tolist() == [[1, 2]]
