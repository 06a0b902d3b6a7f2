"""The Figure 5 ordering: the rows that read no passing block run first
(spava_attn_fwd_phase LOCAL), the selection reuses the query partials'
row LSEs (spava_score_topk_from_partials), then the passing blocks are
gathered and the remaining context rows run (PASSING).

Parity with the oracle as for the one-call order: every score and index and
every output element on small workloads; scores, indices and sampled rows at
full size.  With the same selection the two orders also give bit-identical
attention outputs (they run the same units).
"""
import numpy as np
import pytest
import torch

import oracle as O
import sequence_approximate_attention_amd as S
import workloads as W
from gpu_helpers import TOL, check_close, check_idx, dev_inputs, np64
from test_gpu_fullsize import run_case
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu

REL_TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()
    yield


@pytest.mark.parametrize("w", SMALL + [W.TINY_F32], ids=lambda w: w.name)
def test_small_partials_first(w):
    print(f"[partials-first] {w.name}", flush=True)
    x = W.make_inputs(w)
    ref = O.approx_prefill(x["q"], x["k"], x["v"], w.n_anchor, w.n_hosts, w.host_len, w.n_query, w.lp)
    plan = S.plan_for(w)
    q, k, v = dev_inputs(x, w)
    bufs = S.prefill(plan, q, k, v, partials_first=True)
    torch.cuda.synchronize()
    sc = np64(bufs.scores)
    err = np.abs(sc - ref["scores"]) / np.maximum(np.abs(ref["scores"]), 1e-30)
    assert err.max() < REL_TOL, f"scores rel err {err.max():.2e}"
    check_idx(ref["scores"], bufs.idx.cpu().numpy(), ref["idx"], w.lp)
    # Attention on the oracle's selection, in both orders.
    idx_o = torch.from_numpy(ref["idx"]).cuda()
    b1 = S.prefill(plan, q, k, v, idx=idx_o, partials_first=True)
    b0 = S.prefill(plan, q, k, v, idx=idx_o)
    torch.cuda.synchronize()
    tol = TOL[w.dtype]
    check_close(np64(b1.o), ref["O"], tol["o_max"], tol["o_mean"], "O")
    check_close(np64(b1.lse), ref["LSE"], tol["lse_max"], None, "LSE")
    if w.n_query:
        check_close(np64(b1.o_part), ref["O_part"], tol["o_max"], tol["o_mean"], "O_part")
        check_close(np64(b1.lse_part), ref["LSE_part"], tol["lse_max"], None, "LSE_part")
        assert torch.equal(b1.o_part, b0.o_part) and torch.equal(b1.lse_part, b0.lse_part)
    eq = lambda a, b: torch.equal(a.view(torch.int16), b.view(torch.int16)) if a.dtype == torch.bfloat16 \
        else torch.equal(a, b)
    assert eq(b1.o, b0.o) and torch.equal(b1.lse, b0.lse)


def test_phases_write_disjoint_rows():
    # LOCAL writes the anchor and host 0's rows and the partials; PASSING the
    # context rows of hosts >= 1.  Start from NaN and check each phase's rows.
    w = W.small_workload("bf16", Hq=4, Hkv=2, d=128, la=70, V=3, L=130, n_q=20, lp=40, seed=19)
    x = W.make_inputs(w)
    plan = S.plan_for(w)
    q, k, v = dev_inputs(x, w)
    b = S.alloc_buffers(plan, q.device)
    S.spava_score_topk(plan, q, k, b.scores, b.idx, b.ws_score)
    S.spava_gather_passing(plan, k, v, b.idx, b.kp, b.vp)
    for t in (b.o, b.lse, b.o_part, b.lse_part):
        t.fill_(float("nan"))
    S.spava_attn_fwd_phase(plan, S.SPAVA_PHASE_LOCAL, q, k, v, b.kp, b.vp, b.o, b.lse, b.o_part, b.lse_part)
    torch.cuda.synchronize()
    h1 = w.n_anchor + w.host_len            # first row of host 1
    q0 = w.n_anchor + w.n_hosts * w.host_len
    assert not torch.isnan(b.o[:h1].float()).any() and not torch.isnan(b.lse[:, :h1]).any()
    assert torch.isnan(b.o[h1:q0].float()).all() and torch.isnan(b.lse[:, h1:q0]).all()
    assert not torch.isnan(b.o_part).any() and not torch.isnan(b.lse_part).any()
    S.spava_attn_fwd_phase(plan, S.SPAVA_PHASE_PASSING, q, k, v, b.kp, b.vp, b.o, b.lse, None, None)
    torch.cuda.synchronize()
    assert not torch.isnan(b.o[:q0].float()).any() and not torch.isnan(b.lse[:, :q0]).any()


def test_qwen3b_32k_partials_first():
    run_case(W.QWEN3B_32K, query_stride=3, partials_first=True)


def test_llama8b_128k_text_partials_first():
    w = W.LLAMA8B_128K_TEXT
    run_case(w, query_stride=11, stride=251, heads=[0, w.n_q_heads - 1], partials_first=True)


def test_qwen7b_256k_frames_partials_first():
    # The benchmark's default configuration (the 256K frame shape in this
    # order): every score and index; attention on one query head of every
    # KV group and the last head, every 251st token.
    run_case(W.QWEN7B_256K, query_stride=17, stride=251, partials_first=True)
