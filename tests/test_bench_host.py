"""bench.py's host-side accounting (CPU only): the algorithmic flops its
roofline divides by, the committed traffic summaries it reads, the order it
picks, and its one-GPU guard."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads as W
from test_oracle_pins import approx_mask

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("la,V,L,n_q,lp", [(3, 2, 5, 3, 2), (8, 3, 8, 7, 8), (0, 4, 5, 1, 0), (5, 1, 16, 0, 3),
                                           (0, 1, 9, 4, 9), (7, 5, 6, 0, 1), (2, 3, 11, 5, 4)])
def test_attention_pairs_are_the_visible_pairs(la, V, L, n_q, lp):
    # The roofline's flop count (4·d per visible (query, key) pair per query
    # head) counts exactly the pairs a second, gather-free statement of the
    # visibility rule marks visible, whichever lp keys each block keeps.
    rng = np.random.default_rng(la + 10 * V + 100 * L)
    idx = np.stack([np.stack([np.sort(rng.choice(L, lp, replace=False)) for _ in range(1)]) for _ in range(V)])
    m = approx_mask(la, V, L, n_q, idx, 0)
    w = W.small_workload("bf16", Hq=2, Hkv=1, d=64, la=la, V=V, L=L, n_q=n_q, lp=lp)
    assert bench.attn_pairs_per_head(w) == int(m.sum())
    assert bench.attn_flops(w) == 4.0 * 64 * 2 * int(m.sum())


def test_score_flops_count_the_scoring_rows_keys():
    w = W.small_workload("bf16", Hq=4, Hkv=2, d=64, la=3, V=3, L=10, n_q=5, lp=4)
    # query selector: every query row and head against every block key
    assert bench.score_flops(w) == 2.0 * 64 * (5 * 4) * (3 * 10)
    # context selector: each block's tokens causally over the block's own keys
    assert bench.score_flops(w, "context") == 2.0 * 64 * 4 * 3 * (10 * 11 // 2)


def write_summary(path, workload, sha, traffic):
    path.write_text("# summary\n\n```\nkernel = attn_bf16_kernel<128>\n"
                    f"workload = {workload}\nkernel_source_sha256 = {sha}\n"
                    f"fetch_bytes_per_launch = 1\nwrite_bytes_per_launch = 2\n"
                    f"traffic_bytes_per_launch = {traffic}\n```\n")


def test_traffic_is_read_only_for_the_built_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_DIR", str(tmp_path))
    sha = bench.attn_source_sha256()
    write_summary(tmp_path / "attn_fwd_a_traffic.md", "wl_a", sha, 1.5e9)
    write_summary(tmp_path / "attn_fwd_b_traffic.md", "wl_b", "0" * 64, 2.5e9)
    assert bench.measured_traffic("wl_a") == 1.5e9
    assert bench.measured_traffic("wl_b") is None       # taken on other kernel sources
    assert bench.measured_traffic("wl_c") is None       # no summary


def test_committed_traffic_summaries_are_consistent():
    # Each committed summary names a workload bench.py knows, and its total
    # is its fetched plus written bytes.
    import glob
    names = {w.name for w in W.WORKLOADS + W.PAGE_DEFAULT_WORKLOADS + [W.QWEN3B_32K_PAGE_DEFAULTS_Q128]}
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "attn_fwd_*_traffic.md")))
    assert paths
    for p in paths:
        f = dict(line.strip().split(" = ", 1) for line in open(p) if " = " in line)
        assert f["workload"] in names, p
        assert len(f["kernel_source_sha256"]) == 64
        total = float(f["fetch_bytes_per_launch"]) + float(f["write_bytes_per_launch"])
        assert abs(total - float(f["traffic_bytes_per_launch"])) <= 1e-4 * total, p


def test_order_choice():
    by = {w.name: w for w in W.WORKLOADS + W.PAGE_DEFAULT_WORKLOADS}
    assert bench.pick_order(by["qwen2.5vl7b_256k_frames"]) == "partials-first"
    assert bench.pick_order(by["llama3.1-8b_128k_text"]) == "partials-first"
    assert bench.pick_order(by["qwen2.5vl3b_32k"]) == "one-pass"
    assert bench.pick_order(by["qwen2.5vl7b_256k_frames"], "context") == "one-pass"
    assert bench.pick_order(by["qwen2.5vl7b_256k_frames"].with_(n_query=0)) == "one-pass"


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
