"""Shared helpers of the GPU parity tests (inputs to device, tolerances, the
index-parity rule)."""
import numpy as np
import torch

import sequence_approximate_attention_amd as S

# Attention tolerances against the float64 oracle on the same (rounded) inputs.
TOL = {
    "bf16": {"o_max": 2e-2, "o_mean": 2e-3, "lse_max": 1e-3},
    "f32": {"o_max": 1e-4, "o_mean": 1e-5, "lse_max": 1e-4},
}
# Selected sets must agree except for keys whose oracle score lies within
# this relative distance of the oracle's lp-th largest score.
GAP_REL = 1e-6


def to_dev(x: dict, w, name: str) -> torch.Tensor:
    if w.dtype == "bf16":
        bits = x[name + "16"]
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(np.ascontiguousarray(x[name])).to("cuda")


def dev_inputs(x, w):
    return to_dev(x, w, "q"), to_dev(x, w, "k"), to_dev(x, w, "v")


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_idx(scores_oracle, idx_gpu, idx_oracle, lp):
    """Bit-exact index sets except at oracle score gaps below GAP_REL."""
    V, Hkv, L = scores_oracle.shape
    n_diff = 0
    for h in range(V):
        for g in range(Hkv):
            a = set(idx_gpu[h, g].tolist())
            b = set(idx_oracle[h, g].tolist())
            assert len(a) == lp, (h, g, "duplicate or missing indices")
            assert idx_gpu[h, g].tolist() == sorted(a), (h, g, "not ascending")
            diff = a ^ b
            if not diff:
                continue
            sc = scores_oracle[h, g]
            tau = np.sort(sc)[::-1][lp - 1]
            for j in diff:
                assert abs(sc[j] - tau) <= GAP_REL * abs(tau), (
                    f"block {h} head {g}: key {j} score {sc[j]!r} vs threshold {tau!r}")
            n_diff += len(diff)
    return n_diff


def check_close(got, want, tol_max, tol_mean=None, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    both_inf = np.isneginf(got) & np.isneginf(want)
    with np.errstate(invalid="ignore"):
        err = np.abs(np.where(both_inf, 0.0, got - want))
    assert np.isfinite(err).all(), f"{what}: non-finite mismatch"
    mx = float(err.max()) if err.size else 0.0
    assert mx <= tol_max, f"{what}: max-abs {mx:.3e} > {tol_max:.1e}"
    if tol_mean is not None and err.size:
        mean = float(err.mean())
        assert mean <= tol_mean, f"{what}: mean-abs {mean:.3e} > {tol_mean:.1e}"
    return mx


def sample_rows(w, heads, stride=61, query_stride=1, extra=()):
    """(token, head) pairs: every query_stride-th query token (plus the last),
    the first/middle/last tokens of the anchor and of every block, and every
    stride-th token (a prime, so every tile residue is hit)."""
    la, V, L, nq = w.n_anchor, w.n_hosts, w.host_len, w.n_query
    N = la + V * L + nq
    toks = set(range(0, la + V * L, stride))
    toks |= set(range(la + V * L, N, query_stride))
    if nq:
        toks.add(N - 1)
    for b0, n in [(0, la)] + [(la + h * L, L) for h in range(V)]:
        if n:
            toks |= {b0, b0 + 1, b0 + n // 2, b0 + n - 2, b0 + n - 1}
    toks |= set(extra)
    toks = sorted(t for t in toks if 0 <= t < N)
    return [(t, a) for t in toks for a in heads]
