"""Parity at the full workload sizes (needs an MI355X; each case runs the
oracle on the host for routing and selection of every head, and for attention
on seeded samples of query blocks and queries).

Sizes: Qwen2.5-7B shape at 131072 tokens (c3), the Llama-3.1-8B shape at
131072 tokens (h128, the benchmark's workload, in the benchmark's launch
configuration), Llama shape at 524288 tokens (c4), and the mass-cliff sweep
(c5) at 8192 .. 262144 tokens with alpha in {0.5, 1, 2}.
"""
import json
import os

import numpy as np
import pytest
import torch

import _parity as P
from dynamic_sparse_attention_map_amd import crisp, synth
from oracle import oracle as O

pytestmark = pytest.mark.gpu

B = 128
# where the mass-cliff block counts are written (one JSON file per length)
OUT_DIR = P.OUT_DIR


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    crisp.lib()


def sample_queries(nb, hq, blocks_per_head, queries_per_block, seed):
    """(head, position) pairs: stratified query blocks (0, Nb-1, uniform) and
    uniform queries inside each, always including the block's last query."""
    rng = np.random.default_rng(seed)
    sel = []
    for h in range(hq):
        qbs = {0, nb - 1}
        while len(qbs) < min(blocks_per_head, nb):
            qbs.add(int(rng.integers(nb)))
        for qb in sorted(qbs):
            offs = {B - 1} | set(rng.integers(0, B, size=queries_per_block - 1).tolist())
            sel += [(h, qb * B + o) for o in sorted(offs)]
    return np.array(sel, dtype=np.int32)


def full_case(name, n=None, blocks_per_head=64, queries_per_block=2, whole_blocks_per_head=16,
              prefill_check=True):
    """Routing and sets of every head against the oracle; attention on the
    oracle's lists compared on `whole_blocks_per_head` stratified query blocks
    per head (all 128 rows each: qb = 0, N_b - 1 and uniform others) and on
    `queries_per_block` queries in each of `blocks_per_head` stratified
    blocks per head."""
    spec = synth.config_spec(name, n)
    n, hq, hkv = spec.n, spec.hq, spec.hkv
    nb = -(-n // B)
    P.log(f"case {name}: n={n} hq={hq} hkv={hkv}; generating")
    inp = synth.generate(spec, threads=16)
    q, k, v = P.to_dev(inp)
    ws = crisp.alloc_workspace(n, hq, hkv)
    gr = P.gpu_route(q, k, ws)
    gs_dev = P.gpu_select(q, k, gr, 1.0, ws)
    grh, gs = P.host(gr), P.host(gs_dev)
    P.log(f"case {name}: oracle routing + selection")
    orc_r = O.route(inp.q, inp.k, n, hq, hkv)
    P.check_route(grh, orc_r, margin=0.05)
    P.record(name, "routing", {"heads": hq, "mismatches": 0,
                               "min_margin": float(np.min(np.abs(orc_r.c_struct - O.TAU_PROXY)))})
    rep = P.check_select(inp, grh, gs, 1.0, orc_r)
    P.log(rep.line())
    P.record(name, "selection", rep.as_dict())
    plan = O.plan(inp.q, inp.k, n, hq, hkv, alpha=1.0, routed=orc_r)
    P.log(f"case {name}: attention on the oracle's lists")
    out = P.gpu_attend(q, k, v, plan.row_ptr, plan.col_idx, ws)
    # whole query blocks: every row of the diagonal (masked) block and of
    # the blocks before it
    rows = P.sample_rows(nb, hq, whole_blocks_per_head, seed=7 * n + hq)
    want_b = O.attend(inp.q, inp.k, inp.v, n, hq, hkv, 128, plan.row_ptr, plan.col_idx, rows)
    full = out.view(hq * nb, B, 128) if n % B == 0 else None
    assert full is not None, "whole-block sampling assumes n is a multiple of the block size"
    got_b = full[torch.as_tensor(rows, dtype=torch.long, device=out.device)].float().cpu().numpy()
    P.check_outputs(got_b, want_b, f"{name} attend ({len(rows)} whole blocks)")
    for h in range(hq):
        m = rows // nb == h
        P.check_outputs(got_b[m], want_b[m], f"{name} blocks head {h}")
    rec = P.attention_record(got_b, want_b, rows // nb)
    rec["blocks_per_head"] = int(len(rows) // hq)
    P.record(name, "attention_whole_blocks", rec)
    # single queries in many more blocks
    sel = sample_queries(nb, hq, blocks_per_head, queries_per_block, seed=n + hq)
    want = O.attend_queries(inp.q, inp.k, inp.v, n, hq, hkv, 128, plan.row_ptr, plan.col_idx, sel)
    hs = torch.as_tensor(sel[:, 0], dtype=torch.long, device=out.device)
    ps = torch.as_tensor(sel[:, 1], dtype=torch.long, device=out.device)
    got = out[hs, ps].float().cpu().numpy()
    P.check_outputs(got[:, None, :], want[:, None, :], f"{name} attend ({len(sel)} queries)")
    for h in range(hq):
        m = sel[:, 0] == h
        P.check_outputs(got[m][:, None, :], want[m][:, None, :], f"{name} head {h}")
    rec = P.attention_record(got[:, None, :], want[:, None, :], sel[:, 0])
    rec["blocks_per_head"] = blocks_per_head
    P.record(name, "attention_sampled_queries", rec)
    if prefill_check:
        # the end-to-end prefill on the GPU's own lists equals the staged calls
        out2 = torch.empty_like(q)
        crisp.crisp_prefill(q, k, v, 1.0, ws, out2)
        staged = P.gpu_attend(q, k, v, gs["row_ptr"], gs["col_idx"], crisp.alloc_workspace(n, hq, hkv))
        assert torch.equal(out2.view(torch.int16), staged.view(torch.int16))
        # where the GPU's lists equal the oracle's, outputs match the oracle
        same = [h for h in range(hq)
                if np.array_equal(gs["row_ptr"][h], plan.row_ptr[h])
                and np.array_equal(gs["col_idx"][gs["row_ptr"][h][0]:gs["row_ptr"][h][-1]],
                                   plan.col_idx[plan.row_ptr[h][0]:plan.row_ptr[h][-1]])]
        P.log(f"case {name}: heads with identical lists: {len(same)}/{hq}")
        P.record(name, "heads_with_identical_lists", len(same))
        m = np.isin(sel[:, 0], same)
        got2 = out2[hs[torch.as_tensor(m, device=out.device)], ps[torch.as_tensor(m, device=out.device)]].float().cpu().numpy()
        P.check_outputs(got2[:, None, :], want[m][:, None, :], f"{name} prefill")
    return rep


def test_c3_qwen_131072():
    full_case("c3")


def test_h128_llama_131072():
    full_case("h128")


def test_c4_llama_524288():
    full_case("c4", blocks_per_head=64, queries_per_block=2, whole_blocks_per_head=8)


@pytest.mark.parametrize("n", synth.MASS_CLIFF_NS)
def test_c5_mass_cliff_sweep(n):
    """Route + select on the GPU and the oracle for alpha in {0.5, 1, 2};
    block counts of CRISP against the cumulative gamma = 0.95 selector."""
    spec = synth.config_spec("c5", n)
    hq, hkv = spec.hq, spec.hkv
    nb = -(-n // B)
    P.log(f"case c5: n={n}; generating")
    inp = synth.generate(spec, threads=16)
    q, k, _ = P.to_dev(inp)
    ws = crisp.alloc_workspace(n, hq, hkv)
    gr = P.gpu_route(q, k, ws)
    grh = P.host(gr)
    orc_r = O.route(inp.q, inp.k, n, hq, hkv)
    P.check_route(grh, orc_r)
    assert grh["pattern"].all()
    record = {"n": n, "alpha": {}}
    for alpha in (0.5, 1.0, 2.0):
        gs = P.host(P.gpu_select(q, k, gr, alpha, ws))
        rep = P.check_select(inp, grh, gs, alpha, orc_r)
        P.log(rep.line() + f" alpha={alpha}")
        P.record(f"c5_n{n}", f"selection_alpha{alpha}", rep.as_dict())
        pairs = int((gs["row_ptr"][:, nb] - gs["row_ptr"][:, 0]).sum())
        crisp_sel = [int(gs["counts"][h][0] + gs["counts"][h][1]) for h in range(hq)]
        record["alpha"][str(alpha)] = {"crisp_blocks_per_head": crisp_sel, "pairs": pairs}
    gamma_pure = [len(O.gamma_select(orc_r.p_v[h])) + len(O.gamma_select(orc_r.p_s[h])) for h in range(hq)]
    gamma_clip = [len(O.gamma_select(orc_r.p_v[h], kmin_blocks=8)) + len(O.gamma_select(orc_r.p_s[h], kmin_blocks=8))
                  for h in range(hq)]
    record["gamma_pure_blocks_per_head"] = gamma_pure
    record["gamma_kmin_blocks_per_head"] = gamma_clip
    # sink-only collapse on the concentrated heads (token-0 mass 0.96 >= gamma)
    assert all(g == 2 for g in gamma_pure[:16]), gamma_pure[:16]
    c1 = record["alpha"]["1.0"]["crisp_blocks_per_head"]
    assert all(c >= 16 for c in c1[:16])          # at least k_min per direction
    os.makedirs(OUT_DIR, exist_ok=True)
    with open(os.path.join(OUT_DIR, f"c5_counts_{n}.json"), "w") as f:
        json.dump(record, f)
    P.log(f"c5 n={n}: gamma pure (distributed heads) mean "
          f"{np.mean(gamma_pure[16:]):.1f}, crisp alpha=1 mean {np.mean(c1[16:]):.1f}, "
          f"alpha=2 mean {np.mean(record['alpha']['2.0']['crisp_blocks_per_head'][16:]):.1f}")
