"""crisp_prefill_noalloc (the entry point for callers that cannot allocate)
against crisp_prefill with a caller workspace (needs an MI355X).

Both run the same kernels, so the outputs must be bit-identical.  Two calls
in a row on one device share the library's static scratch; the second is
smaller than the first, so it runs over what the first left behind.
"""
import ctypes as C

import pytest
import torch

from dynamic_sparse_attention_map_amd import crisp, synth

pytestmark = pytest.mark.gpu

WORKSPACE = 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    crisp.lib()


def _inputs(n, hq, hkv, seed_id):
    kinds = [synth.VS if h % 4 != 3 else synth.DIFFUSE for h in range(hq)]
    inp = synth.generate(synth.custom_spec(n, hq, hkv, kinds, seed_id=seed_id))
    return inp.q.cuda(), inp.k.cuda(), inp.v.cuda()


def _noalloc(q, k, v, out, alpha=1.0, opts=None):
    """The raw C call (ctypes), as a caller without torch would make it."""
    hq, n, d = q.shape
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    return crisp.lib().crisp_prefill_noalloc(
        C.c_void_p(q.data_ptr()), C.c_void_p(k.data_ptr()), C.c_void_p(v.data_ptr()), n, hq,
        k.shape[0], d, 128, float(alpha), None if opts is None else C.byref(opts),
        C.c_void_p(out.data_ptr()), stream)


def _reference(q, k, v, alpha=1.0, opts=None):
    hq, n, _ = q.shape
    out = torch.empty_like(q)
    crisp.crisp_prefill(q, k, v, alpha, crisp.alloc_workspace(n, hq, k.shape[0]), out, opts=opts)
    return out


def _same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_noalloc_two_calls_match_prefill():
    # 20000 tokens, 32/8 heads: the multi-launch selection path (N_b = 157),
    # then 3057 tokens, 4/2 heads: the one-work-group paths and a partial
    # last block, over the first call's leftovers
    for n, hq, hkv, seed in ((20000, 32, 8, 301), (3057, 4, 2, 302)):
        print(f"noalloc n={n} hq={hq} hkv={hkv}", flush=True)
        q, k, v = _inputs(n, hq, hkv, seed)
        want = _reference(q, k, v)
        got = torch.full_like(q, float("nan"))
        assert _noalloc(q, k, v, got) == 0
        torch.cuda.synchronize()
        assert _same_bits(got, want), (n, hq, hkv)


def test_noalloc_options_and_refusal():
    """Options pass through (the FlexPrefill baseline, the dense gate); a layer
    over the scratch limit is refused before anything runs and leaves the
    output untouched."""
    q, k, v = _inputs(4096 + 64, 8, 2, 303)
    for opts in (crisp.flexprefill_opts(), crisp.default_opts(dense_below_tokens=8192)):
        want = _reference(q, k, v, opts=opts)
        got = torch.empty_like(q)
        crisp.crisp_prefill_noalloc(q, k, v, 1.0, got, opts=opts)
        torch.cuda.synchronize()
        assert _same_bits(got, want)
    big_n = 40000
    assert crisp.crisp_workspace_size(big_n, 32, 8)[0] > crisp.NOALLOC_SCRATCH_BYTES
    qb = torch.zeros(32, big_n, 128, dtype=torch.bfloat16, device="cuda")
    kb = torch.zeros(8, big_n, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(qb, 7.0)
    assert _noalloc(qb, kb, kb, out) == WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
