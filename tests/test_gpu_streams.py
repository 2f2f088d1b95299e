"""Concurrent calls on two streams (needs an MI355X).

The library keeps no state between calls (the caller owns every buffer,
including the workspace), so prefills of different inputs on two streams
with their own workspaces may overlap in time; each output must equal the
same call made alone, bit for bit.  Both streams keep the default priority.
"""
import pytest
import torch

import _parity as P
from dynamic_sparse_attention_map_amd import crisp, synth

pytestmark = pytest.mark.gpu

HQ, HKV = 4, 2
KINDS = [synth.VS, synth.DIFFUSE, synth.VS, synth.DIFFUSE]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    crisp.lib()


def dev(n, seed_id):
    inp = synth.generate(synth.custom_spec(n, HQ, HKV, KINDS, seed_id=seed_id))
    return inp.q.cuda(), inp.k.cuda(), inp.v.cuda()


def bits(t):
    return t.contiguous().view(torch.int16)


@pytest.mark.parametrize("lens", [(20000, 6000), (8192, 8192 + 300)])
def test_two_streams_equal_alone(lens):
    P.log(f"two streams lens={lens}")
    ins = [dev(n, 800 + i + n % 7) for i, n in enumerate(lens)]
    wss = [crisp.alloc_workspace(n, HQ, HKV) for n in lens]
    alone = []
    for (q, k, v), ws in zip(ins, wss):
        o = torch.empty_like(q)
        crisp.crisp_prefill(q, k, v, 1.0, ws, o)
        torch.cuda.synchronize()
        alone.append(o)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = [torch.zeros_like(q) for q, _, _ in ins]
    torch.cuda.synchronize()
    for rep in range(3):
        for (q, k, v), ws, o, s in zip(ins, wss, outs, streams):
            with torch.cuda.stream(s):
                for _ in range(2):              # keep both streams busy for a while
                    crisp.crisp_prefill(q, k, v, 1.0, ws, o, stream=s)
        torch.cuda.synchronize()
        for b in range(2):
            assert torch.equal(bits(outs[b]), bits(alone[b])), f"rep {rep}, stream {b}"
