"""A seeded sweep of the oracle over small shapes: V in {1..4}, L in
{1, 5, 8, 16}, la in {0, 3, 8}, n_q in {0, 1, 3, 7}, lp in {0, 1, L-1, L},
G in {1, 2, 4}, d in {8, 64}.  Each drawn case checks, against torch's
float64 attention (not the oracle's own routines):

  * lp = L: every row equals dense causal attention;
  * for any lp: query, anchor and host-0 rows equal dense causal attention
    (their key sets are their whole prefixes; the query partials merge
    exactly);
  * context rows equal attention over the original sequence under the
    visibility mask built from the selected indices;
  * the scores of each (block, KV head) sum to n_q * G, and the selection is
    the top lp under (score descending, index ascending).
"""
import numpy as np
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle as O
from test_oracle_pins import approx_mask, rand_qkv, sdpa

shapes = st.fixed_dictionaries({
    "V": st.integers(1, 4),
    "L": st.sampled_from([1, 5, 8, 16]),
    "la": st.sampled_from([0, 3, 8]),
    "n_q": st.sampled_from([0, 1, 3, 7]),
    "lp_kind": st.sampled_from(["0", "1", "L-1", "L"]),
    "G": st.sampled_from([1, 2, 4]),
    "Hkv": st.integers(1, 2),
    "d": st.sampled_from([8, 64]),
    "seed": st.integers(0, 2**16),
})


@settings(max_examples=300, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])
@given(shapes)
def test_oracle_sweep(c):
    V, L, la, n_q, G, Hkv, d = c["V"], c["L"], c["la"], c["n_q"], c["G"], c["Hkv"], c["d"]
    lp = {"0": 0, "1": min(1, L), "L-1": max(L - 1, 0), "L": L}[c["lp_kind"]]
    Hq = G * Hkv
    N = la + V * L + n_q
    rng = np.random.default_rng(c["seed"])
    q, k, v = rand_qkv(rng, N, Hq, Hkv, d, scale=1.5)
    r = O.approx_prefill(q, k, v, la, V, L, n_q, lp)
    dense = sdpa(q, k, v, causal=True)
    # Scores and selection.
    np.testing.assert_allclose(r["scores"].sum(axis=2), n_q * G, rtol=1e-12, atol=1e-12)
    for h in range(V):
        for g in range(Hkv):
            order = sorted(range(L), key=lambda j: (-r["scores"][h, g, j], j))[:lp]
            assert r["idx"][h, g].tolist() == sorted(order)
    # Rows whose key set is their whole prefix.
    exact = np.r_[0:la + L, la + V * L:N]
    np.testing.assert_allclose(r["O"][exact], dense[exact], atol=1e-11)
    if lp == L:
        np.testing.assert_allclose(r["O"], dense, atol=1e-11)
    # Every row under the visibility rule restated as a mask.
    for g in range(Hkv):
        m = approx_mask(la, V, L, n_q, r["idx"], g)
        heads = slice(g * G, (g + 1) * G)
        ref = sdpa(q[:, heads], k[:, g:g + 1], v[:, g:g + 1], mask=m)
        np.testing.assert_allclose(r["O"][:, heads], ref, atol=1e-11)
