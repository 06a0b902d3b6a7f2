"""spava_score_topk_noalloc (the scoring call for callers that cannot
allocate) against spava_score_topk on the same inputs: scores and indices
bit for bit, on two calls in a row, the second on a smaller plan, so the
second call reuses the static scratch the first one filled."""
import pytest
import torch

import sequence_approximate_attention_amd as S

pytestmark = pytest.mark.gpu


def _inputs(plan, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    N = plan.n_tokens
    q = torch.randn((N, plan.n_q_heads, plan.head_dim), generator=g, device="cuda").to(plan.torch_dtype)
    k = torch.randn((N, plan.n_kv_heads, plan.head_dim), generator=g, device="cuda").to(plan.torch_dtype)
    # A few strong keys per block so that the selection is not decided by noise alone.
    q0 = plan.n_anchor + plan.n_hosts * plan.host_len
    if plan.n_query:
        u = q[q0:].float().mean(dim=(0, 1))
        u = u / u.norm()
        for h in range(plan.n_hosts):
            b0 = plan.n_anchor + h * plan.host_len
            k[b0 + 7: b0 + plan.host_len: 97] = (3.0 * plan.head_dim ** 0.5 * u).to(plan.torch_dtype)
    return q, k


def _reference(plan, q, k):
    scores = torch.empty((plan.n_hosts, plan.n_kv_heads, plan.host_len), dtype=torch.float32, device="cuda")
    idx = torch.empty((plan.n_hosts, plan.n_kv_heads, plan.lp), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(256, S.spava_score_topk_ws_bytes(plan)), dtype=torch.uint8, device="cuda")
    S.spava_score_topk(plan, q, k, scores, idx, ws)
    return scores, idx


def _noalloc(plan, q, k, with_scores):
    scores = (torch.full((plan.n_hosts, plan.n_kv_heads, plan.host_len), float("nan"), device="cuda")
              if with_scores else None)
    idx = torch.full((plan.n_hosts, plan.n_kv_heads, plan.lp), -1, dtype=torch.int32, device="cuda")
    S.spava_score_topk_noalloc(plan, q, k, scores, idx)
    return scores, idx


CASES = [
    # (plan, seed): the first needs 62.9 MB of the 64 MiB scratch when the
    # scores stay there (the 256K frame-shaped layer: 28/4 heads, 32 hosts of
    # 8128, 512 query tokens, lp 4096); the second is the 32K layer; the last
    # a small ragged one in float32.
    (S.Plan(4096, 32, 8128, 512, 28, 4, 128, 4096), 11),
    (S.Plan(2048, 8, 3840, 128, 16, 2, 128, 1024), 12),
    (S.Plan(48, 3, 100, 20, 4, 2, 64, 24, S.SPAVA_F32), 13),
]


def test_noalloc_matches_the_workspace_call_on_consecutive_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    for n, (plan, seed) in enumerate(CASES):
        print(f"[noalloc] case {n}: {plan}", flush=True)
        q, k = _inputs(plan, seed)
        ref_scores, ref_idx = _reference(plan, q, k)
        # Without a scores buffer (the scores live in the static scratch) ...
        _, idx = _noalloc(plan, q, k, with_scores=False)
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx), f"case {n}: indices differ (scores in scratch)"
        # ... and with one: bit-identical scores.
        scores, idx = _noalloc(plan, q, k, with_scores=True)
        torch.cuda.synchronize()
        assert torch.equal(scores.view(torch.int32), ref_scores.view(torch.int32)), f"case {n}: scores differ"
        assert torch.equal(idx, ref_idx), f"case {n}: indices differ"
        del q, k
        torch.cuda.empty_cache()


def test_noalloc_rejects_a_plan_beyond_the_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = S.Plan(4096, 32, 8128, 1024, 28, 4, 128, 4096)
    q = torch.empty((16,), dtype=torch.bfloat16, device="cuda")   # never read: the call fails first
    idx = torch.empty((16,), dtype=torch.int32, device="cuda")
    import ctypes
    rc = S.lib().spava_score_topk_noalloc(ctypes.byref(big.c()), ctypes.c_void_p(q.data_ptr()),
                                          ctypes.c_void_p(q.data_ptr()), None, ctypes.c_void_p(idx.data_ptr()),
                                          None)
    assert rc == S.SPAVA_EWORKSPACE
