"""The C-ABI library: it loads, exports every function include/spava.h
declares, and rejects bad arguments on the host (no GPU needed: every call
here fails validation before anything is enqueued)."""
import ctypes
import os
import re

import pytest

import sequence_approximate_attention_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spava.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spava_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = S.lib()
    names = declared_functions()
    assert set(names) == set(S.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_plan_struct_matches_the_header():
    # 9 int32 fields and a float, then four int64 strides.
    assert ctypes.sizeof(S.spava_plan) == 72
    assert S.spava_plan.q_stride_tok.offset == 40 and S.spava_plan.kv_stride_head.offset == 64


def test_version_and_empty_error():
    assert S.lib().spava_version() == 100
    assert isinstance(S.lib().spava_last_error(), bytes)


def plan(**kw):
    base = dict(n_anchor=32, n_hosts=4, host_len=128, n_query=16, n_q_heads=2, n_kv_heads=1,
                head_dim=64, lp=16, dtype=S.SPAVA_F32, scale=0.0)
    base.update(kw)
    return S.Plan(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(), S.SPAVA_OK),
    (dict(lp=129), S.SPAVA_EINVAL),
    (dict(lp=-1), S.SPAVA_EINVAL),
    (dict(n_q_heads=3, n_kv_heads=2), S.SPAVA_EINVAL),
    (dict(head_dim=96), S.SPAVA_EUNSUPPORTED),
    (dict(dtype=7), S.SPAVA_EUNSUPPORTED),
    (dict(n_hosts=0), S.SPAVA_EINVAL),
    (dict(host_len=0), S.SPAVA_EINVAL),
    (dict(n_query=-1), S.SPAVA_EINVAL),
    (dict(scale=-1.0), S.SPAVA_EINVAL),
    (dict(scale=float("nan")), S.SPAVA_EINVAL),
    (dict(n_hosts=1, host_len=1 << 24, n_q_heads=64, n_kv_heads=8, head_dim=128, lp=0), S.SPAVA_EINVAL),
    (dict(lp=0, n_query=0, n_anchor=0), S.SPAVA_OK),
    # strides (elements): multiples of 16 bytes, non-negative, bounded extents
    (dict(q_stride_tok=4 * 64, q_stride_head=64, kv_stride_tok=3 * 64, kv_stride_head=64), S.SPAVA_OK),
    (dict(q_stride_tok=130), S.SPAVA_EINVAL),
    (dict(dtype=S.SPAVA_BF16, kv_stride_head=68), S.SPAVA_EINVAL),
    (dict(dtype=S.SPAVA_BF16, kv_stride_head=72), S.SPAVA_OK),
    (dict(kv_stride_tok=-64), S.SPAVA_EINVAL),
    (dict(q_stride_head=1 << 26), S.SPAVA_OK),
    (dict(q_stride_head=1 << 31), S.SPAVA_EINVAL),
    (dict(kv_stride_tok=1 << 22), S.SPAVA_EINVAL),
])
def test_plan_check(kw, code):
    assert S.spava_plan_check(plan(**kw)) == code
    if code:
        assert len(S.lib().spava_last_error()) > 0


def test_workspace_sizes():
    p = plan(dtype=S.SPAVA_BF16, head_dim=128)
    r256 = lambda n: (n + 255) // 256 * 256
    sc = lambda L: r256(4 * 1 * L * 4)       # room for float scores [V][Hkv][L] after the statistics
    # bf16 scoring: a (max, sum) float pair per (key chunk of 512, block, KV head, query row)
    assert S.spava_score_topk_ws_bytes(p) == 1 * 4 * 1 * 16 * 2 * 8 + sc(128)
    assert (S.spava_score_topk_ws_bytes(plan(dtype=S.SPAVA_BF16, host_len=1000, lp=16))
            == 2 * 4 * 1 * 16 * 2 * 8 + sc(1000))
    # float32 scoring: one log-sum-exp float per (block, KV head, query row), 256-byte rounded
    assert S.spava_score_topk_ws_bytes(plan(dtype=S.SPAVA_F32)) == 4 * 1 * 16 * 2 * 4 + sc(128)
    assert S.spava_score_topk_ws_bytes(plan(dtype=S.SPAVA_F32, n_query=3)) == 256 + sc(128)
    # context selector: the block's L tokens (times G heads) are the scoring
    # rows, one key chunk; bf16 adds float column sums of each head's row
    # split(s) of >= 1024 tokens
    assert S.spava_score_topk_context_ws_bytes(p) == 1 * 4 * 1 * 128 * 2 * 8 + 2 * 4 * 1 * 128 * 4 + sc(128)
    assert (S.spava_score_topk_context_ws_bytes(plan(dtype=S.SPAVA_BF16, host_len=1000, lp=16))
            == 1 * 4 * 1 * 1000 * 2 * 8 + 2 * 4 * 1 * 1000 * 4 + sc(1000))
    # L = 3000: 3 splits of 1024 tokens per head
    assert (S.spava_score_topk_context_ws_bytes(plan(dtype=S.SPAVA_BF16, host_len=3000, lp=16))
            == 1 * 4 * 1 * 3000 * 2 * 8 + 3 * 2 * 4 * 1 * 3000 * 4 + sc(3000))
    assert S.spava_score_topk_context_ws_bytes(plan(dtype=S.SPAVA_F32)) == 4 * 1 * 128 * 2 * 4 + sc(128)
    assert S.spava_score_topk_context_ws_bytes(plan(dtype=S.SPAVA_F32, n_query=0)) == 4 * 1 * 128 * 2 * 4 + sc(128)
    assert S.spava_score_topk_context_ws_bytes(plan(lp=999)) == 0
    # key-contiguous V: Hkv * d * (pad(la) + V*pad(L) + pad(n_q)) + passing, bf16
    main = 1 * 128 * (64 + 4 * 128 + 64) * 2
    pas = 1 * 128 * 64 * 2
    assert S.spava_attn_fwd_ws_bytes(p) == main + pas
    assert S.spava_attn_fwd_ws_bytes(plan(lp=999)) == 0


def test_null_and_misaligned_pointers_rejected_on_host():
    # Every call here must fail its host checks: the pointers are fake and
    # nothing may be launched with them.  Where a GPU is present a check that
    # let a call through would launch on those addresses, so the test only
    # runs without one.
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake-pointer host checks run on machines without a GPU")
    lib = S.lib()
    p = plan().c()
    fake = ctypes.c_void_p(0x10000)          # never dereferenced: validation fails first
    odd = ctypes.c_void_p(0x10004)
    assert lib.spava_score_topk(ctypes.byref(p), None, fake, fake, fake, fake, 1 << 20, None) == S.SPAVA_EINVAL
    assert lib.spava_score_topk(ctypes.byref(p), odd, fake, fake, fake, fake, 1 << 20, None) == S.SPAVA_EINVAL
    assert lib.spava_score_topk(ctypes.byref(p), fake, fake, fake, fake, fake, 4, None) == S.SPAVA_EWORKSPACE
    # scores may be NULL (they then live in the workspace, which must hold them)
    need = lib.spava_score_topk_ws_bytes(ctypes.byref(p))
    assert lib.spava_score_topk(ctypes.byref(p), fake, fake, None, fake, fake, need - 1, None) == S.SPAVA_EWORKSPACE
    assert lib.spava_gather_passing(ctypes.byref(p), fake, None, fake, fake, fake, None) == S.SPAVA_EINVAL
    assert lib.spava_attn_fwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, None, fake,
                              fake, 1 << 20, None) == S.SPAVA_EINVAL
    pb = plan(dtype=S.SPAVA_BF16).c()
    assert lib.spava_attn_fwd(ctypes.byref(pb), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                              fake, 16, None) == S.SPAVA_EWORKSPACE
    assert b"workspace" in lib.spava_last_error()
    assert lib.spava_lse_merge(0, 4, 2, 64, fake, fake, fake, 128, fake, 4, S.SPAVA_F32, None) == S.SPAVA_EINVAL
    assert lib.spava_lse_merge(2, 4, 2, 62, fake, fake, fake, 128, fake, 4, S.SPAVA_F32, None) == S.SPAVA_EINVAL
    assert lib.spava_lse_merge(2, 4, 2, 64, fake, fake, fake, 64, fake, 4, S.SPAVA_F32, None) == S.SPAVA_EINVAL
    assert lib.spava_lse_merge(2, 4, 2, 64, fake, fake, fake, 128, fake, 4, 9, None) == S.SPAVA_EUNSUPPORTED
    # Nothing to do: succeeds without touching memory.
    assert lib.spava_lse_merge(2, 0, 2, 64, None, None, None, 128, None, 0, S.SPAVA_F32, None) == S.SPAVA_OK
    p0 = plan(lp=0).c()
    assert lib.spava_gather_passing(ctypes.byref(p0), None, None, None, None, None, None) == S.SPAVA_OK
    # Context selector: same checks as the query selector, its own workspace size.
    assert lib.spava_score_topk_context(ctypes.byref(p), None, fake, fake, fake, fake, 1 << 20, None) == S.SPAVA_EINVAL
    assert lib.spava_score_topk_context(ctypes.byref(p), odd, fake, fake, fake, fake, 1 << 20, None) == S.SPAVA_EINVAL
    # (scores = NULL: the workspace must also hold the scores, so need - 1
    # fails the check before anything is launched)
    need = lib.spava_score_topk_context_ws_bytes(ctypes.byref(p))
    assert lib.spava_score_topk_context(ctypes.byref(p), fake, fake, None, fake, fake, need - 1, None) == S.SPAVA_EWORKSPACE
    assert lib.spava_score_topk_context(ctypes.byref(p), fake, fake, fake, fake, fake, 16, None) == S.SPAVA_EWORKSPACE
    assert b"spava_score_topk_context" in lib.spava_last_error()
    # Overlap: bad sizes, NULL or misaligned pointers; nothing to do succeeds.
    assert lib.spava_kv_overlap(-1, 4, fake, fake, fake, None) == S.SPAVA_EINVAL
    assert lib.spava_kv_overlap(2, -4, fake, fake, fake, None) == S.SPAVA_EINVAL
    assert lib.spava_kv_overlap(2, 4, None, fake, fake, None) == S.SPAVA_EINVAL
    assert lib.spava_kv_overlap(2, 4, fake, fake, None, None) == S.SPAVA_EINVAL
    assert lib.spava_kv_overlap(2, 4, fake, ctypes.c_void_p(0x10002), fake, None) == S.SPAVA_EINVAL
    assert lib.spava_kv_overlap(0, 4, None, None, None, None) == S.SPAVA_OK
    # Attention in phases: unknown phase; the LOCAL phase needs no passing
    # blocks but its partials, the PASSING phase the reverse.
    assert lib.spava_attn_fwd_phase(ctypes.byref(p), 7, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                    fake, 1 << 20, None) == S.SPAVA_EINVAL
    assert b"phase" in lib.spava_last_error()
    assert lib.spava_attn_fwd_phase(ctypes.byref(p), S.SPAVA_PHASE_LOCAL, fake, fake, fake, None, None, fake, fake,
                                    None, fake, fake, 1 << 20, None) == S.SPAVA_EINVAL
    assert lib.spava_attn_fwd_phase(ctypes.byref(p), S.SPAVA_PHASE_PASSING, fake, fake, fake, None, fake, fake,
                                    fake, None, None, fake, 1 << 20, None) == S.SPAVA_EINVAL
    assert lib.spava_attn_fwd_phase(ctypes.byref(pb), S.SPAVA_PHASE_PASSING, fake, fake, fake, fake, fake, fake,
                                    fake, None, None, fake, 16, None) == S.SPAVA_EWORKSPACE
    # Scores from the query partials: lse_part is required when n_query > 0.
    assert lib.spava_score_topk_from_partials(ctypes.byref(p), fake, fake, None, fake, fake, None) == S.SPAVA_EINVAL
    assert lib.spava_score_topk_from_partials(ctypes.byref(p), fake, odd, fake, fake, fake, None) == S.SPAVA_EINVAL
