"""Several sequences per call, strided layouts and the context-length gate
(needs an MI355X).

crisp_prefill_batch runs Alg. 1 on each sequence in turn, or, with a
workspace of crisp_workspace_size_batch, routes and selects every sequence
and attends the whole batch in one launch ("fused").  Each output is checked
bit for bit against crisp_prefill on a contiguous copy of that sequence: the
same kernels see the same values. crisp_prefill itself is
checked against the oracle (routing, selection and attention) on the same
sequences.  The gate (Section 5.3, "Short contexts") must reproduce
crisp_attend_dense bit for bit and the oracle's dense causal attention.
"""
import ctypes as C

import numpy as np
import pytest
import torch

import _parity as P
from dynamic_sparse_attention_map_amd import crisp, synth
from oracle import oracle as O

pytestmark = pytest.mark.gpu

B = 128
HQ, HKV = 4, 2
KINDS = [synth.VS, synth.DIFFUSE, synth.VS, synth.VS]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    crisp.lib()


def gen(n, seed_id):
    """A seeded sequence of n >= 1 tokens (None for n == 0)."""
    return synth.generate(synth.custom_spec(n, HQ, HKV, KINDS, seed_id=seed_id)) if n else None


def batch_ws(lens, kind, hq=HQ, hkv=HKV):
    """The workspace that selects crisp_prefill_batch's path: the longest
    sequence's (one sequence after another) or the batch's (one launch)."""
    if kind == "serial":
        return crisp.alloc_workspace(max(lens), hq, hkv)
    return crisp.alloc_batch_workspace(lens, hq, hkv)


PATHS = ["serial", "fused"]


def single(q, k, v, alpha=1.0, opts=None):
    """crisp_prefill on contiguous [heads, n, 128] device tensors."""
    n = q.shape[1]
    out = torch.empty_like(q)
    crisp.crisp_prefill(q, k, v, alpha, crisp.alloc_workspace(n, HQ, HKV), out, opts=opts)
    return out


def same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))


def oracle_check(inp, got, alpha=1.0, tag=""):
    """The oracle's routing and selection against the GPU stages on the same
    sequence, and the oracle's attention on the GPU's own lists against
    `got`."""
    n = inp.spec.n
    qd, kd = inp.q.cuda(), inp.k.cuda()
    ws = crisp.alloc_workspace(n, HQ, HKV)
    gr = P.gpu_route(qd, kd, ws)
    grh = P.host(gr)
    orc_r = O.route(inp.q, inp.k, n, HQ, HKV)
    P.check_route(grh, orc_r)
    gs = P.host(P.gpu_select(qd, kd, gr, alpha, ws))
    P.check_select(inp, grh, gs, alpha, orc_r)
    nb = -(-n // B)
    rows = np.arange(HQ * nb, dtype=np.int32)
    want = O.attend(inp.q, inp.k, inp.v, n, HQ, HKV, 128, gs["row_ptr"].reshape(-1), gs["col_idx"],
                    rows)
    full = torch.zeros(HQ, nb * B, 128)
    full[:, :n] = got.float().cpu()
    P.check_outputs(full.numpy().reshape(HQ * nb, B, 128), want, f"batch {tag}")


@pytest.mark.parametrize("path", PATHS)
def test_varlen_packed_tokens_major(path):
    """[total, heads, d] packed sequences with cumulative offsets (ragged,
    one of length 1, one empty), one call, one workspace."""
    lens = [300, 1, 0, 1000, 129, 2048]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    total = cu[-1]
    P.log(f"varlen lens={lens}")
    inps = [gen(n, 300 + i) for i, n in enumerate(lens)]
    q = torch.zeros(total, HQ, 128, dtype=torch.bfloat16)
    k = torch.zeros(total, HKV, 128, dtype=torch.bfloat16)
    v = torch.zeros(total, HKV, 128, dtype=torch.bfloat16)
    for b, n in enumerate(lens):
        if n:
            q[cu[b]:cu[b + 1]] = inps[b].q.transpose(0, 1)
            k[cu[b]:cu[b + 1]] = inps[b].k.transpose(0, 1)
            v[cu[b]:cu[b + 1]] = inps[b].v.transpose(0, 1)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = torch.full_like(qd, float("nan"))
    crisp.prefill_varlen(qd, kd, vd, cu, out, 1.0, batch_ws(lens, path))
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        if n == 0:
            continue
        ref = single(inps[b].q.cuda(), inps[b].k.cuda(), inps[b].v.cuda())
        got = out[cu[b]:cu[b + 1]].transpose(0, 1)
        assert same_bits(got, ref), f"sequence {b} (n={n}) differs from crisp_prefill"
        oracle_check(inps[b], got, tag=f"varlen {path} seq {b} n={n}")


@pytest.mark.parametrize("path", PATHS)
def test_batch_seq_heads_layout(path):
    """Equal lengths in a [batch, seq, heads, d] tensor."""
    n, batch = 1024, 2
    inps = [gen(n, 320 + b) for b in range(batch)]
    q = torch.stack([i.q.transpose(0, 1) for i in inps]).cuda()     # [B, n, H, d]
    k = torch.stack([i.k.transpose(0, 1) for i in inps]).cuda()
    v = torch.stack([i.v.transpose(0, 1) for i in inps]).cuda()
    out = torch.empty_like(q)
    crisp.crisp_prefill_batch([q[b].transpose(0, 1) for b in range(batch)],
                              [k[b].transpose(0, 1) for b in range(batch)],
                              [v[b].transpose(0, 1) for b in range(batch)],
                              [out[b].transpose(0, 1) for b in range(batch)],
                              1.0, batch_ws([n] * batch, path))
    for b in range(batch):
        ref = single(inps[b].q.cuda(), inps[b].k.cuda(), inps[b].v.cuda())
        assert same_bits(out[b].transpose(0, 1), ref), f"batch element {b}"


@pytest.mark.parametrize("path", PATHS)
def test_batch_contiguous_default_strides(path):
    """strides == NULL: each sequence contiguous [heads, n, d], separate
    allocations, called through the C ABI directly."""
    lens = [640, 77, 1500]
    inps = [gen(n, 340 + i) for i, n in enumerate(lens)]
    dev = [(i.q.cuda(), i.k.cuda(), i.v.cuda()) for i in inps]
    outs = [torch.empty_like(d[0]) for d in dev]
    arr = (crisp.crisp_seq * len(lens))()
    for b, ((q, k, v), o) in enumerate(zip(dev, outs)):
        arr[b] = crisp.crisp_seq(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lens[b])
    ws = batch_ws(lens, path)
    rc = crisp.lib().crisp_prefill_batch(arr, len(lens), None, HQ, HKV, 128, 128, 1.0, None,
                                         C.c_void_p(ws.data_ptr()), ws.numel(),
                                         C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == crisp.CRISP_OK, crisp.status_string(rc)
    for b, (q, k, v) in enumerate(dev):
        assert same_bits(outs[b], single(q, k, v)), f"sequence {b}"


def test_gate_runs_dense_below_threshold():
    n = 3000                      # N_b = 24: the sparse path keeps a strict subset
    inp = gen(n, 360)
    q, k, v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
    ws = crisp.alloc_workspace(n, HQ, HKV)
    gated = single(q, k, v, opts=crisp.default_opts(dense_below_tokens=n + 1))
    dense = torch.empty_like(q)
    crisp.crisp_attend_dense(q, k, v, ws, dense)
    assert same_bits(gated, dense)
    nb = -(-n // B)
    rp, ci = O.full_causal_lists(HQ, nb)
    want = O.attend(inp.q, inp.k, inp.v, n, HQ, HKV, 128, rp, ci, np.arange(HQ * nb, dtype=np.int32))
    full = torch.zeros(HQ, nb * B, 128)
    full[:, :n] = gated.float().cpu()
    P.check_outputs(full.numpy().reshape(HQ * nb, B, 128), want, "gated dense")
    # at the threshold itself the sparse path runs
    ungated = single(q, k, v)
    assert same_bits(single(q, k, v, opts=crisp.default_opts(dense_below_tokens=n)), ungated)
    assert not same_bits(gated, ungated)


@pytest.mark.parametrize("path", PATHS)
def test_gate_inside_a_batch(path):
    """A gate between the lengths: short sequences dense, long ones sparse."""
    lens = [3000, 5000]
    inps = [gen(n, 380 + i) for i, n in enumerate(lens)]
    opts = crisp.default_opts(dense_below_tokens=4096)
    dev = [(i.q.cuda(), i.k.cuda(), i.v.cuda()) for i in inps]
    outs = [torch.empty_like(d[0]) for d in dev]
    crisp.crisp_prefill_batch([d[0] for d in dev], [d[1] for d in dev], [d[2] for d in dev], outs,
                              1.0, batch_ws(lens, path), opts=opts)
    q, k, v = dev[0]
    dense = torch.empty_like(q)
    crisp.crisp_attend_dense(q, k, v, crisp.alloc_workspace(lens[0], HQ, HKV), dense)
    assert same_bits(outs[0], dense)
    assert not same_bits(outs[0], single(*dev[0]))
    assert same_bits(outs[1], single(*dev[1]))


def test_fused_batch_llama_heads():
    """The single-launch path at the Llama-3.1-8B head shape (32 query / 8 KV
    heads): twelve sequences of mixed lengths (short, ragged, one of 20000
    tokens), each bit-identical to crisp_prefill on it alone; the serial path
    on the same call agrees too."""
    hq, hkv = 32, 8
    lens = [20000, 2048, 2048, 77, 4096 + 5, 1, 2048, 640, 8192, 129, 3000, 2048]
    kinds = [synth.VS if h % 4 != 3 else synth.DIFFUSE for h in range(hq)]
    inps = [synth.generate(synth.custom_spec(n, hq, hkv, kinds, seed_id=400 + i))
            for i, n in enumerate(lens)]
    P.log(f"fused batch lens={lens}")
    dev = [(i.q.cuda(), i.k.cuda(), i.v.cuda()) for i in inps]
    for path in PATHS:
        outs = [torch.full_like(d[0], float("nan")) for d in dev]
        crisp.crisp_prefill_batch([d[0] for d in dev], [d[1] for d in dev], [d[2] for d in dev], outs,
                                  1.0, batch_ws(lens, path, hq, hkv))
        torch.cuda.synchronize()
        for b, (q, k, v) in enumerate(dev):
            ref = torch.empty_like(q)
            crisp.crisp_prefill(q, k, v, 1.0, crisp.alloc_workspace(lens[b], hq, hkv), ref)
            assert same_bits(outs[b], ref), f"{path}: sequence {b} (n={lens[b]})"


def test_fused_equal_lengths_group():
    """Six packed [total, heads, d] sequences of one ragged length (1500
    tokens): the single-launch path routes and selects them as one group of
    6 x 4 query heads; each output equals crisp_prefill on that sequence."""
    n, count = 1500, 6
    inps = [gen(n, 500 + i) for i in range(count)]
    cu = [i * n for i in range(count + 1)]
    q = torch.cat([i.q.transpose(0, 1) for i in inps]).cuda()     # [total, H, d]
    k = torch.cat([i.k.transpose(0, 1) for i in inps]).cuda()
    v = torch.cat([i.v.transpose(0, 1) for i in inps]).cuda()
    out = torch.full_like(q, float("nan"))
    crisp.prefill_varlen(q, k, v, cu, out, 1.0, batch_ws([n] * count, "fused"))
    torch.cuda.synchronize()
    for b in range(count):
        ref = single(inps[b].q.cuda(), inps[b].k.cuda(), inps[b].v.cuda())
        assert same_bits(out[cu[b]:cu[b + 1]].transpose(0, 1), ref), f"sequence {b}"
    oracle_check(inps[3], out[cu[3]:cu[4]].transpose(0, 1), tag="equal-length group seq 3")
