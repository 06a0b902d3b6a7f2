"""A whole layer captured in a HIP graph and replayed.

The library allocates, frees and synchronises nothing and enqueues every
kernel on the caller's stream, so one layer (scores and top-lp, gather,
attention, merge; both call orders) can be captured once and replayed as a
fixed executor over its buffers.  Every replay, with every output reset
between replays (so a replay must write all of it) and with new inputs
copied into the captured input buffers, must equal eager execution on the
same inputs bit for bit: the calls are deterministic.
"""
import pytest
import torch

import sequence_approximate_attention_amd as S
import workloads as W
from gpu_helpers import dev_inputs

pytestmark = pytest.mark.gpu

OUTPUTS = ("scores", "idx", "kp", "vp", "o", "lse", "o_part", "lse_part")

CASES = [
    W.small_workload("bf16", Hq=4, Hkv=2, d=128, la=100, V=3, L=300, n_q=20, lp=50, seed=40),
    W.small_workload("bf16", Hq=8, Hkv=2, d=64, la=0, V=4, L=200, n_q=9, lp=64, seed=41),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()
    yield


def snapshot(bufs):
    return {n: getattr(bufs, n).clone() for n in OUTPUTS}


def same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


@pytest.mark.parametrize("partials_first", [False, True], ids=["one_pass", "partials_first"])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_layer_graph_replays_match_eager(w, partials_first):
    print(f"[graph] {w.name} partials_first={partials_first}", flush=True)
    plan = S.plan_for(w)
    inputs = []
    for t in range(3):
        wt = w.with_(seed=w.seed + 100 * t)
        inputs.append(dev_inputs(W.make_inputs(wt), wt))
    q, k, v = (x.clone() for x in inputs[0])   # the buffers the graph reads
    bufs = S.alloc_buffers(plan, q.device)

    def load(i):
        q.copy_(inputs[i][0])
        k.copy_(inputs[i][1])
        v.copy_(inputs[i][2])

    refs = []
    for i in range(len(inputs)):
        load(i)
        S.prefill(plan, q, k, v, bufs=bufs, partials_first=partials_first)
        torch.cuda.synchronize()
        refs.append(snapshot(bufs))
    assert not same(refs[0]["o"], refs[1]["o"]), "the input sets must give different layers"

    # One eager call on a side stream first, as torch's capture expects.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        S.prefill(plan, q, k, v, bufs=bufs, partials_first=partials_first)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        S.prefill(plan, q, k, v, bufs=bufs, partials_first=partials_first)
    torch.cuda.synchronize()

    for rep in range(6):
        i = (rep * 2) % len(inputs)
        load(i)
        for n in OUTPUTS:
            getattr(bufs, n).zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in OUTPUTS:
            assert same(getattr(bufs, n), refs[i][n]), f"replay {rep} (inputs {i}): {n} differs from eager"
