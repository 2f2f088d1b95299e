"""crisp_prefill, crisp_attend_dense, crisp_prefill_batch (single-launch
path) and crisp_prefill_noalloc inside a captured HIP graph (needs an
MI355X).

Every call is asynchronous on the caller's stream and the library never
allocates, synchronises or fills memory with a memset node, so a caller can
capture a whole prefill.  Each graph is replayed several times, with eager
calls (on other inputs) and synchronisations between the replays, and every
replay must equal the eager call on the same inputs bit for bit.
"""
import pytest
import torch

import _parity as P
from dynamic_sparse_attention_map_amd import crisp, synth

pytestmark = pytest.mark.gpu

HQ, HKV = 4, 2
KINDS = [synth.VS, synth.DIFFUSE, synth.VS, synth.VS]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    crisp.lib()


def dev(n, seed_id):
    inp = synth.generate(synth.custom_spec(n, HQ, HKV, KINDS, seed_id=seed_id))
    return inp.q.cuda(), inp.k.cuda(), inp.v.cuda()


def bits(t):
    return t.contiguous().view(torch.int16)


@pytest.mark.parametrize("n", [4096, 8192 + 300, 20000])
def test_prefill_graph_replays_equal_eager(n):
    P.log(f"graph prefill n={n}")
    q, k, v = dev(n, 400 + n % 13)
    q2, k2, v2 = dev(n, 500 + n % 13)                 # other inputs for the eager calls between
    ws = crisp.alloc_workspace(n, HQ, HKV)
    ws2 = crisp.alloc_workspace(n, HQ, HKV)
    want = torch.empty_like(q)
    crisp.crisp_prefill(q, k, v, 1.0, ws, want)
    torch.cuda.synchronize()

    out = torch.zeros_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            crisp.crisp_prefill(q, k, v, 1.0, ws, out)
    torch.cuda.synchronize()
    other = torch.empty_like(q2)
    for rep in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(want)), f"replay {rep} differs from the eager call"
        crisp.crisp_prefill(q2, k2, v2, 1.0, ws2, other)  # eager work between the replays
        crisp.crisp_prefill(q, k, v, 2.0, ws, other)      # the graph's own workspace, other alpha
        torch.cuda.synchronize()


def test_dense_graph_replays_equal_eager():
    n = 8192 + 300
    q, k, v = dev(n, 600)
    ws = crisp.alloc_workspace(n, HQ, HKV)
    want = torch.empty_like(q)
    crisp.crisp_attend_dense(q, k, v, ws, want)
    torch.cuda.synchronize()
    out = torch.zeros_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            crisp.crisp_attend_dense(q, k, v, ws, out)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(want)), f"replay {rep} differs from the eager call"
        crisp.crisp_prefill(q, k, v, 1.0, ws, torch.empty_like(q))
        torch.cuda.synchronize()


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            fn()
    torch.cuda.synchronize()
    return g


def test_batch_graph_replays_equal_eager():
    """The single-launch batch path (sequences of one length routed and
    selected as one layer, one attention launch, its tables written from
    kernel arguments) captured and replayed."""
    lens = [3000, 2048, 2048, 640]
    devs = [dev(n, 700 + i) for i, n in enumerate(lens)]
    others = [dev(n, 720 + i) for i, n in enumerate(lens)]
    ws = crisp.alloc_batch_workspace(lens, HQ, HKV)
    ws2 = crisp.alloc_batch_workspace(lens, HQ, HKV)
    cols = lambda ds, j: [d[j] for d in ds]
    want = [torch.empty_like(d[0]) for d in devs]
    crisp.crisp_prefill_batch(cols(devs, 0), cols(devs, 1), cols(devs, 2), want, 1.0, ws)
    torch.cuda.synchronize()
    outs = [torch.zeros_like(d[0]) for d in devs]
    g = capture(lambda: crisp.crisp_prefill_batch(cols(devs, 0), cols(devs, 1), cols(devs, 2),
                                                  outs, 1.0, ws))
    scratch = [torch.empty_like(d[0]) for d in devs]
    for rep in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for b in range(len(lens)):
            assert torch.equal(bits(outs[b]), bits(want[b])), f"replay {rep}, sequence {b}"
        crisp.crisp_prefill_batch(cols(others, 0), cols(others, 1), cols(others, 2), scratch, 1.0, ws2)
        crisp.crisp_prefill_batch(cols(others, 0), cols(others, 1), cols(others, 2), scratch, 1.0, ws)
        torch.cuda.synchronize()


def test_noalloc_graph_replays_equal_eager():
    """crisp_prefill_noalloc, meant for callers under graph capture: replays
    equal the eager call, with eager calls on other inputs in between that
    use the same static scratch array."""
    n = 8192 + 300
    q, k, v = dev(n, 740)
    q2, k2, v2 = dev(n, 741)
    want = torch.empty_like(q)
    crisp.crisp_prefill_noalloc(q, k, v, 1.0, want)      # also resolves the scratch address
    torch.cuda.synchronize()
    out = torch.zeros_like(q)
    g = capture(lambda: crisp.crisp_prefill_noalloc(q, k, v, 1.0, out))
    other = torch.empty_like(q2)
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(want)), f"replay {rep} differs from the eager call"
        crisp.crisp_prefill_noalloc(q2, k2, v2, 2.0, other)
        torch.cuda.synchronize()
