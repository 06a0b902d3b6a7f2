"""Strided q, k, v (explicit token and head strides in the plan).

The same values laid out as a packed QKV projection output [N][Hq+2Hkv][d]
or as head-major tensors [H][N][d] give bit-identical scores, indices and
outputs to the dense layout (the kernels do the same arithmetic at other
addresses), and the strided run matches the oracle like the dense one.
"""
import numpy as np
import pytest
import torch

import oracle as O
import sequence_approximate_attention_amd as S
import workloads as W
from gpu_helpers import TOL, check_close, check_idx, dev_inputs, np64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()
    yield


def packed(q, k, v):
    N, Hq, d = q.shape
    Hkv = k.shape[1]
    qkv = torch.empty((N, Hq + 2 * Hkv, d), dtype=q.dtype, device=q.device)
    qkv[:, :Hq] = q
    qkv[:, Hq:Hq + Hkv] = k
    qkv[:, Hq + Hkv:] = v
    return qkv[:, :Hq], qkv[:, Hq:Hq + Hkv], qkv[:, Hq + Hkv:]


def heads_major(q, k, v):
    return tuple(t.transpose(0, 1).contiguous().transpose(0, 1) for t in (q, k, v))


def same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def run(plan, q, k, v, **kw):
    bufs = S.prefill(plan, q, k, v, **kw)
    torch.cuda.synchronize()
    return bufs


CASES = [
    W.small_workload("bf16"),
    W.small_workload("bf16", Hq=8, Hkv=2, d=64, la=0, V=4, L=77, n_q=9, lp=77, seed=8),
    W.small_workload("bf16", Hq=7, Hkv=1, d=128, la=130, V=2, L=200, n_q=33, lp=0, seed=9),
    W.small_workload("f32", Hq=4, Hkv=2, d=128, la=40, V=3, L=90, n_q=12, lp=30, seed=12),
]


@pytest.mark.parametrize("layout", [packed, heads_major], ids=["packed_qkv", "heads_major"])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_strided_layouts_match_dense_and_oracle(w, layout):
    print(f"[strides] {w.name} {layout.__name__}", flush=True)
    x = W.make_inputs(w)
    q, k, v = dev_inputs(x, w)
    plan = S.plan_for(w)
    qs, ks, vs = layout(q, k, v)
    assert not qs.is_contiguous()
    plan_s = plan.with_strides(qs, ks, vs)
    dense = run(plan, q, k, v)
    strided = run(plan_s, qs, ks, vs)
    for name in ("scores", "idx", "o", "lse", "o_part", "lse_part", "kp", "vp"):
        assert same(getattr(strided, name), getattr(dense, name)), name
    # The strided layout against the oracle: the selection, then the
    # attention on the oracle's own selection (inputs flow oracle -> GPU).
    ref = O.approx_prefill(x["q"], x["k"], x["v"], w.n_anchor, w.n_hosts, w.host_len, w.n_query, w.lp)
    check_idx(ref["scores"], strided.idx.cpu().numpy(), ref["idx"], w.lp)
    on_ref = run(plan_s, qs, ks, vs, idx=torch.from_numpy(ref["idx"]).cuda())
    tol = TOL[w.dtype]
    check_close(np64(on_ref.o), ref["O"], tol["o_max"], tol["o_mean"], "O")
    check_close(np64(on_ref.lse), ref["LSE"], tol["lse_max"], None, "LSE")


def test_strided_context_selector_and_partials_first():
    w = CASES[0]
    x = W.make_inputs(w)
    q, k, v = dev_inputs(x, w)
    plan = S.plan_for(w)
    qs, ks, vs = packed(q, k, v)
    plan_s = plan.with_strides(qs, ks, vs)
    # Context selector.
    out = []
    for p, qq, kk in ((plan, q, k), (plan_s, qs, ks)):
        scores = torch.empty((w.n_hosts, w.n_kv_heads, w.host_len), dtype=torch.float32, device="cuda")
        idx = torch.empty((w.n_hosts, w.n_kv_heads, w.lp), dtype=torch.int32, device="cuda")
        ws = torch.empty(max(256, S.spava_score_topk_context_ws_bytes(p)), dtype=torch.uint8, device="cuda")
        S.spava_score_topk_context(p, qq, kk, scores, idx, ws)
        out.append((scores, idx))
    torch.cuda.synchronize()
    assert torch.equal(out[0][0], out[1][0]) and torch.equal(out[0][1], out[1][1])
    # Scores from the query partials.
    a = run(plan, q, k, v, partials_first=True)
    b = run(plan_s, qs, ks, vs, partials_first=True)
    for name in ("scores", "idx", "o", "lse", "o_part", "lse_part"):
        assert same(getattr(a, name), getattr(b, name)), name


def test_strided_32k_packed_qkv():
    w = W.QWEN3B_32K
    print(f"[strides] {w.name} packed", flush=True)
    x = W.make_inputs(w)
    q, k, v = dev_inputs(x, w)
    plan = S.plan_for(w)
    qs, ks, vs = packed(q, k, v)
    dense = run(plan, q, k, v)
    strided = run(plan.with_strides(qs, ks, vs), qs, ks, vs)
    for name in ("scores", "idx", "o", "lse", "o_part", "lse_part"):
        assert same(getattr(strided, name), getattr(dense, name)), name


def test_binding_rejects_mismatched_strides():
    w = CASES[0]
    x = W.make_inputs(w)
    q, k, v = dev_inputs(x, w)
    qs, ks, vs = packed(q, k, v)
    with pytest.raises(ValueError, match="strides"):
        S.prefill(S.plan_for(w), qs, ks, vs)            # dense plan, strided views
    with pytest.raises(ValueError, match="same strides"):
        S.plan_for(w).with_strides(qs, ks, v)         # k and v laid out differently
