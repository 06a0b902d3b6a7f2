"""The seeded input generator: shapes, determinism, planted structure, bf16 cast."""
import numpy as np
import torch

import workloads as W


def test_shapes_and_token_counts():
    assert W.TINY_F32.n_tokens == 560
    assert W.QWEN3B_32K.n_tokens == 32896
    assert W.QWEN7B_64K.n_tokens == 65792
    assert W.QWEN3B_128K.n_tokens == 131200
    assert W.QWEN7B_256K.n_tokens == 264704
    for w in W.WORKLOADS + W.PAGE_DEFAULT_WORKLOADS:
        assert w.n_q_heads % w.n_kv_heads == 0
        assert 0 <= w.lp <= w.host_len


def test_page_default_ratios():
    # la = n/64 and lp = n/128 of the whole input length, 8 hosts.
    for w in W.PAGE_DEFAULT_WORKLOADS:
        n = w.n_tokens
        assert n % 128 == 0
        assert w.n_anchor * 64 == n and w.lp * 128 == n and w.n_hosts == 8
    assert W.LLAMA8B_128K_TEXT.n_tokens == 131072
    assert (W.LLAMA8B_128K_TEXT.n_q_heads, W.LLAMA8B_128K_TEXT.n_kv_heads) == (32, 8)


def test_determinism_and_seed_dependence():
    w = W.small_workload()
    a = W.make_inputs(w)
    b = W.make_inputs(w)
    c = W.make_inputs(w, seed=w.seed + 1)
    for n in ("q", "k", "v"):
        np.testing.assert_array_equal(a[n], b[n])
        assert not np.array_equal(a[n], c[n])


def test_bf16_round_matches_torch_and_is_idempotent():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]   # exact ties
    r = W.bf16_round(x)
    t = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(r, t)
    np.testing.assert_array_equal(W.bf16_round(r), r)
    bits = W.bf16_bits(r)
    np.testing.assert_array_equal((bits.astype(np.uint32) << 16).view(np.float32), r)


def test_planted_keys_present():
    w = W.TINY_F32
    x = W.make_inputs(w)
    k = x["k"]
    d = w.head_dim
    for h in range(w.n_hosts):
        blk = k[w.n_anchor + h * w.host_len: w.n_anchor + (h + 1) * w.host_len, 0]
        norms = np.linalg.norm(blk, axis=1)
        planted = np.isclose(norms, 3 * np.sqrt(d), rtol=1e-5)
        assert planted.sum() == 4
        rows = blk[planted]
        assert np.allclose(rows, rows[0])


def test_needle_and_frames_structure():
    w = W.QWEN3B_128K.with_(n_hosts=3, host_len=256, n_anchor=64, n_query=16, lp=32)
    k = W.make_inputs(w)["k"]
    same = np.all(k[1:] == k[:-1], axis=(1, 2))
    assert same.sum() == 63                                     # one span of 64 equal keys
    w = W.QWEN7B_256K.with_(n_hosts=2, host_len=2048, n_anchor=1024, n_query=8, lp=64,
                            n_q_heads=4, n_kv_heads=2)
    k = W.make_inputs(w)["k"].astype(np.float64)
    nctx = w.n_anchor + w.n_hosts * w.host_len
    fr = k[:nctx].reshape(-1, 1024, 2, w.head_dim).mean(axis=1)   # frame means ~ offsets
    assert 0.35 < fr.var() < 0.65                                # variance 0.5 offsets
