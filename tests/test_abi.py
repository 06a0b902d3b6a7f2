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
    assert S.lib().spava_version() == 200
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
    # strides near the int64 range are rejected without overflowing
    (dict(kv_stride_tok=1 << 62), S.SPAVA_EINVAL),
    (dict(q_stride_head=(1 << 63) - 1), S.SPAVA_EINVAL),
    (dict(dtype=S.SPAVA_BF16, q_stride_tok=(1 << 62) + 8), S.SPAVA_EINVAL),
    # sizes at the int32 limit are rejected without overflowing
    (dict(n_hosts=(1 << 31) - 1, host_len=(1 << 31) - 1, lp=0), S.SPAVA_EINVAL),
    (dict(n_anchor=(1 << 31) - 1), S.SPAVA_EINVAL),
    (dict(n_query=(1 << 31) - 1), S.SPAVA_EINVAL),
    (dict(n_q_heads=(1 << 31) - 1, n_kv_heads=1), S.SPAVA_EINVAL),
    (dict(host_len=(1 << 31) - 1, lp=(1 << 31) - 1, n_hosts=1), S.SPAVA_EINVAL),
    # a token stride shorter than a row would overlap the next token's row
    (dict(kv_stride_tok=32, kv_stride_head=64), S.SPAVA_EINVAL),
    (dict(q_stride_tok=48), S.SPAVA_EINVAL),
    (dict(kv_stride_tok=64, kv_stride_head=2 * 64), S.SPAVA_OK),
    # token strides stay below 2^24 bytes (tiny plans, so that no extent
    # check is what rejects them)
    (dict(n_anchor=0, n_hosts=1, host_len=2, n_query=1, lp=0, dtype=S.SPAVA_BF16,
          kv_stride_tok=(1 << 23) - 8), S.SPAVA_OK),
    (dict(n_anchor=0, n_hosts=1, host_len=2, n_query=1, lp=0, dtype=S.SPAVA_BF16,
          kv_stride_tok=1 << 23), S.SPAVA_EINVAL),
    (dict(n_anchor=0, n_hosts=1, host_len=2, n_query=1, lp=0, dtype=S.SPAVA_F32,
          q_stride_tok=1 << 22), S.SPAVA_EINVAL),
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
    # plans at the int32 limits: no size, no overflow
    for kw in (dict(n_hosts=(1 << 31) - 1, host_len=(1 << 31) - 1, lp=0), dict(n_query=(1 << 31) - 1),
               dict(n_q_heads=(1 << 31) - 1, n_kv_heads=1)):
        assert S.spava_score_topk_ws_bytes(plan(**kw)) == 0
        assert S.spava_score_topk_context_ws_bytes(plan(**kw)) == 0


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
                              None) == S.SPAVA_EINVAL
    pb = plan(dtype=S.SPAVA_BF16).c()
    assert lib.spava_attn_fwd(ctypes.byref(pb), fake, odd, fake, fake, fake, fake, fake, fake, fake,
                              None) == S.SPAVA_EINVAL
    assert b"aligned" in lib.spava_last_error()
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
                                    None) == S.SPAVA_EINVAL
    assert b"phase" in lib.spava_last_error()
    assert lib.spava_attn_fwd_phase(ctypes.byref(p), S.SPAVA_PHASE_LOCAL, fake, fake, fake, None, None, fake, fake,
                                    None, fake, None) == S.SPAVA_EINVAL
    assert lib.spava_attn_fwd_phase(ctypes.byref(p), S.SPAVA_PHASE_PASSING, fake, fake, fake, None, fake, fake,
                                    fake, None, None, None) == S.SPAVA_EINVAL
    # Scores from the query partials: lse_part is required when n_query > 0.
    assert lib.spava_score_topk_from_partials(ctypes.byref(p), fake, fake, None, fake, fake, None) == S.SPAVA_EINVAL
    assert lib.spava_score_topk_from_partials(ctypes.byref(p), fake, odd, fake, fake, fake, None) == S.SPAVA_EINVAL


def test_noalloc_scoring_rejects_plans_beyond_its_scratch_on_the_host():
    # The 256K frame-shaped layer fits the static scratch even with the
    # scores kept there; twice its query rows do not.  The rejection happens
    # before the device is touched, so this runs without a GPU.
    fits = S.Plan(4096, 32, 8128, 512, 28, 4, 128, 4096)
    assert S.spava_score_topk_ws_bytes(fits) <= S.SPAVA_NOALLOC_SCRATCH_BYTES
    big = S.Plan(4096, 32, 8128, 1024, 28, 4, 128, 4096)
    assert S.spava_score_topk_ws_bytes(big) > S.SPAVA_NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced: the call fails validation first
    rc = S.lib().spava_score_topk_noalloc(ctypes.byref(big.c()), fake, fake, fake, fake, None)
    assert rc == S.SPAVA_EWORKSPACE
    assert b"static scratch" in S.lib().spava_last_error()
    # Argument checks as spava_score_topk: NULL idx with lp > 0.
    rc = S.lib().spava_score_topk_noalloc(ctypes.byref(fits.c()), fake, fake, fake, None, None)
    assert rc == S.SPAVA_EINVAL


def _int32s():
    from hypothesis import strategies as st
    edge = st.sampled_from([-(1 << 31), -1, 0, 1, 2, 7, 64, 128, 1000, (1 << 15), (1 << 24), (1 << 31) - 1])
    return st.one_of(edge, st.integers(-(1 << 31), (1 << 31) - 1), st.integers(0, 5000))


def _int64s():
    from hypothesis import strategies as st
    edge = st.sampled_from([0, 8, 64, 128, 136, 1 << 22, 1 << 31, 1 << 62, (1 << 63) - 1, -8, -(1 << 63)])
    return st.one_of(edge, st.integers(-(1 << 63), (1 << 63) - 1), st.integers(0, 1 << 20))


def test_plan_arithmetic_never_misbehaves():
    # Random plans, extreme values included: the check returns one of its
    # codes, the workspace sizes are 0 exactly for rejected plans, and both
    # are repeatable.  (The host-sanitizer run of this file turns any
    # overflow or out-of-bounds access on the way into an abort.)
    from hypothesis import given, settings, HealthCheck
    from hypothesis import strategies as st

    fields = st.fixed_dictionaries(dict(
        n_anchor=_int32s(), n_hosts=_int32s(), host_len=_int32s(), n_query=_int32s(),
        n_q_heads=_int32s(), n_kv_heads=_int32s(), head_dim=st.sampled_from([64, 128, 0, 96, -64]),
        lp=_int32s(), dtype=st.sampled_from([S.SPAVA_BF16, S.SPAVA_F32, 2, -1]),
        scale=st.sampled_from([0.0, 0.125, -1.0, float("inf"), float("nan"), 1e30]),
        q_stride_tok=_int64s(), q_stride_head=_int64s(), kv_stride_tok=_int64s(), kv_stride_head=_int64s()))

    @settings(max_examples=400, deadline=None, suppress_health_check=list(HealthCheck), derandomize=True)
    @given(fields)
    def run(kw):
        p = S.Plan(**kw)
        rc = S.spava_plan_check(p)
        assert rc in (S.SPAVA_OK, S.SPAVA_EINVAL, S.SPAVA_EUNSUPPORTED)
        assert S.spava_plan_check(p) == rc
        for f in (S.spava_score_topk_ws_bytes, S.spava_score_topk_context_ws_bytes):
            n = f(p)
            assert (n == 0) == (rc != S.SPAVA_OK)
            assert n % 256 == 0 and n == f(p)

    run()


@pytest.mark.parametrize("kw", [
    None,   # every workload of the recipe
    dict(n_anchor=0, n_hosts=1, host_len=(1 << 23) - 64, n_query=64, n_q_heads=1, n_kv_heads=1,
         head_dim=128, lp=1024, dtype=S.SPAVA_BF16),
    dict(n_anchor=100, n_hosts=65536, host_len=128, n_query=16, n_q_heads=2, n_kv_heads=1,
         head_dim=64, lp=64, dtype=S.SPAVA_BF16),
    dict(n_anchor=3, n_hosts=3, host_len=1, n_query=0, n_q_heads=8, n_kv_heads=8,
         head_dim=128, lp=1, dtype=S.SPAVA_F32),
], ids=["workloads", "one_long_block", "many_hosts", "tiny_f32_no_query"])
def test_launch_setup_runs_to_the_launch_without_a_device(kw):
    # Valid plans pass every host check and reach the kernel launches, which
    # fail cleanly (SPAVA_ELAUNCH) where there is no GPU: the launch set-up
    # (unit counts, splits, grids, workspace carving) runs on the host, and
    # under the host-sanitizer build of this file any overflow in it aborts.
    # The pointers are fake, so this runs only without a GPU.
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake-pointer launch set-up runs on machines without a GPU")
    import workloads as W
    plans = [S.plan_for(w) for w in W.WORKLOADS + W.PAGE_DEFAULT_WORKLOADS] if kw is None else [plan(**kw)]
    lib = S.lib()
    fake = ctypes.c_void_p(1 << 20)
    for pl in plans:
        assert S.spava_plan_check(pl) == S.SPAVA_OK
        p = pl.c()
        need = lib.spava_score_topk_ws_bytes(ctypes.byref(p))
        need_ctx = lib.spava_score_topk_context_ws_bytes(ctypes.byref(p))
        rcs = [lib.spava_score_topk(ctypes.byref(p), fake, fake, fake, fake, fake, need, None),
               lib.spava_score_topk(ctypes.byref(p), fake, fake, None, fake, fake, need, None),
               lib.spava_score_topk_context(ctypes.byref(p), fake, fake, fake, fake, fake, need_ctx, None),
               lib.spava_gather_passing(ctypes.byref(p), fake, fake, fake, fake, fake, None),
               lib.spava_attn_fwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, fake, None)]
        if pl.n_query > 0:
            rcs.append(lib.spava_score_topk_from_partials(ctypes.byref(p), fake, fake, fake, fake, fake, None))
        if need <= S.SPAVA_NOALLOC_SCRATCH_BYTES:
            rcs.append(lib.spava_score_topk_noalloc(ctypes.byref(p), fake, fake, fake, fake, None))
        expect = [S.SPAVA_ELAUNCH] * len(rcs)
        if pl.lp == 0:
            expect[3] = S.SPAVA_OK   # nothing to gather
        for ph in (S.SPAVA_PHASE_ALL, S.SPAVA_PHASE_LOCAL, S.SPAVA_PHASE_PASSING):
            rcs.append(lib.spava_attn_fwd_phase(ctypes.byref(p), ph, fake, fake, fake, fake, fake, fake, fake,
                                                fake, fake, None))
            # one host: the PASSING phase has no rows to run
            expect.append(S.SPAVA_OK if ph == S.SPAVA_PHASE_PASSING and pl.n_hosts == 1 else S.SPAVA_ELAUNCH)
        assert rcs == expect, (pl, rcs, lib.spava_last_error())
    assert lib.spava_lse_merge(33, 512, 28, 128, fake, fake, fake, 28 * 128, fake, 512, S.SPAVA_BF16,
                               None) == S.SPAVA_ELAUNCH
    assert lib.spava_kv_overlap(128, 4096, fake, fake, fake, None) == S.SPAVA_ELAUNCH


def test_last_error_is_per_thread():
    # The error text is thread-local: threads that fail different checks at
    # the same time each read back their own message (ctypes releases the
    # GIL during the calls, so the threads do overlap in the library).
    import threading
    lib = S.lib()
    cases = {"lp": (plan(lp=129), b"lp (129)"), "dtype": (plan(dtype=7), b"dtype 7"),
             "heads": (plan(n_q_heads=3, n_kv_heads=2), b"n_q_heads (3)"), "ok": (plan(), b"")}
    bad = []

    def worker(name):
        p, want = cases[name]
        pc = p.c()
        for _ in range(2000):
            lib.spava_plan_check(ctypes.byref(pc))
            got = lib.spava_last_error()
            if (want and want not in got) or (not want and got):
                bad.append((name, got))
                return

    threads = [threading.Thread(target=worker, args=(n,)) for n in cases for _ in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not bad, bad[:4]


def test_binding_rejects_strided_outputs_past_their_storage():
    # spava_lse_merge writes o and lse through plain pointers with the given
    # strides; the binding checks that the last element written lies inside
    # each tensor's storage (an output of the wrong dtype or too few rows is
    # rejected before the call).
    import torch
    o = torch.empty(4 * 64 + 10, dtype=torch.bfloat16)
    S._reach(o, 4 * 64 + 10, "o")
    S._reach(o[10:], 4 * 64, "o")
    S._reach(o, 0, "o")
    with pytest.raises(ValueError, match="past the end"):
        S._reach(o[10:], 4 * 64 + 1, "o")
    # Element counts are in the tensor's own dtype: float32 needs twice the bytes.
    f32 = torch.empty(4 * 64 + 10, dtype=torch.bfloat16).view(torch.float32)
    S._reach(f32, (4 * 64 + 10) // 2, "o")
    with pytest.raises(ValueError, match="past the end"):
        S._reach(f32, (4 * 64 + 10) // 2 + 1, "o")
    lse = torch.empty(3, 100)
    S._reach(lse[:, 40:], 2 * 100 + 60, "lse")
    with pytest.raises(ValueError, match="past the end"):
        S._reach(lse[:, 40:], 2 * 100 + 61, "lse")
