"""HIP path vs the CPU oracle on the same seeded inputs (needs an MI355X).

Every call goes through the C ABI (ctypes binding of libcrisp.so).
"""
import numpy as np
import pytest
import torch

import _parity as P
from dynamic_sparse_attention_map_amd import crisp, synth
from oracle import oracle as O

pytestmark = pytest.mark.gpu

B = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    crisp.lib()


def case(inp, alpha=1.0, rows=None, tag=""):
    """Route, select and attend on the GPU; check all three against the oracle
    (attention on the oracle's lists, on the query blocks `rows`: all of
    them by default, none for an empty array).  The counts and errors are
    also written to the parity record of the case."""
    sp = inp.spec
    n, hq, hkv = sp.n, sp.hq, sp.hkv
    nb = -(-n // B)
    name = f"{sp.name}{tag}".replace(" ", "_").replace("=", "")
    P.log(f"case {sp.name}{tag}: n={n} hq={hq} hkv={hkv} alpha={alpha}")
    q, k, v = P.to_dev(inp)
    ws = crisp.alloc_workspace(n, hq, hkv)
    gr = P.gpu_route(q, k, ws)
    orc_r = O.route(inp.q, inp.k, n, hq, hkv)
    grh = P.host(gr)
    P.check_route(grh, orc_r)
    gs = P.host(P.gpu_select(q, k, gr, alpha, ws))
    rep = P.check_select(inp, grh, gs, alpha, orc_r)
    P.log(rep.line())
    P.record(name, "selection", rep.as_dict())
    plan = O.plan(inp.q, inp.k, n, hq, hkv, alpha=alpha)
    out = P.gpu_attend(q, k, v, plan.row_ptr, plan.col_idx, ws)
    if rows is None:
        rows = np.arange(hq * nb, dtype=np.int32)
    if len(rows):
        want = O.attend(inp.q, inp.k, inp.v, n, hq, hkv, 128, plan.row_ptr, plan.col_idx, rows)
        full = torch.zeros(hq, nb * B, 128)          # rows past n (a partial last block) are 0
        full[:, :n] = out.float().cpu()
        got = full.numpy().reshape(hq * nb, B, 128)[rows]
        P.check_outputs(got, want, f"{sp.name}{tag} attend")
        for h in range(hq):
            sel = rows // nb == h
            if sel.any():
                P.check_outputs(got[sel], want[sel], f"{sp.name}{tag} head {h}")
        P.record(name, "attention_whole_blocks", P.attention_record(got, want, rows // nb))
    return dict(q=q, k=k, v=v, ws=ws, gr=gr, gs=gs, plan=plan, out=out, inp=inp)


def test_c1_full_parity():
    case(synth.generate(synth.config_spec("c1")))


def test_c1_dense_matches_oracle():
    inp = synth.generate(synth.config_spec("c1"))
    n, hq, hkv = 4096, 4, 1
    nb = -(-n // B)
    q, k, v = P.to_dev(inp)
    ws = crisp.alloc_workspace(n, hq, hkv)
    out = torch.empty_like(q)
    crisp.crisp_attend_dense(q, k, v, ws, out)
    rp, ci = O.full_causal_lists(hq, nb)
    rows = np.arange(hq * nb, dtype=np.int32)
    want = O.attend(inp.q, inp.k, inp.v, n, hq, hkv, 128, rp, ci, rows)
    got = out.float().cpu().numpy().reshape(hq * nb, B, 128)
    P.check_outputs(got, want, "c1 dense")
    # the same lists given explicitly give the same bits
    out2 = P.gpu_attend(q, k, v, rp, ci, ws)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("beta", [1.2, 0.5])
def test_running_max_rescale(beta):
    """Scores that grow along the keys: q_i . k_j is close to f_i * beta * j,
    with f_i from 0.6 to 1.4 by the row's position i % 32 within its
    wavefront's 32 queries.  The running max of a row then grows by about
    f_i * beta * 64 raw units per 64-key sub-tile: with beta = 1.2 that is
    46-108 units around the 2^8 lazy-rescale gap (about 63), with beta = 0.5
    19-45 units, so rows are rescaled on every sub-tile, every other one or
    less often, with probabilities up to 2^8 in between, and the rescale
    factors differ between the rows q and q + 16 whose row sums one lane
    holds.  Dense attention against the oracle on every row."""
    n, hq, hkv = 2048, 4, 1
    nb = n // B
    qt, kt, vt = synth.growing_scores(n, hq, hkv, beta, seed=1234 + int(beta * 10))
    dq, dk, dv = qt.cuda(), kt.cuda(), vt.cuda()
    ws = crisp.alloc_workspace(n, hq, hkv)
    out = torch.empty_like(dq)
    crisp.crisp_attend_dense(dq, dk, dv, ws, out)
    rp, ci = O.full_causal_lists(hq, nb)
    rows = np.arange(hq * nb, dtype=np.int32)
    want = O.attend(qt, kt, vt, n, hq, hkv, 128, rp, ci, rows)
    got = out.float().cpu().numpy().reshape(hq * nb, B, 128)
    P.check_outputs(got, want, f"rescale beta={beta}")


def test_c1_prefill_equals_stages():
    inp = synth.generate(synth.config_spec("c1"))
    r = case(inp)
    q, k, v, ws = r["q"], r["k"], r["v"], r["ws"]
    out = torch.empty_like(q)
    crisp.crisp_prefill(q, k, v, 1.0, ws, out)
    gs = r["gs"]
    ws2 = crisp.alloc_workspace(4096, 4, 1)
    staged = P.gpu_attend(q, k, v, gs["row_ptr"], gs["col_idx"], ws2)
    assert torch.equal(out.view(torch.int16), staged.view(torch.int16))


@pytest.mark.parametrize("n,hq,hkv", [(3 * B - 5, 3, 3), (101 * B + 77, 4, 2),
                                       (128 * B, 8, 2), (128 * B + 1, 4, 2)])
def test_prefill_equals_stages_across_vt_switch(n, hq, hkv):
    """Up to N_b = 128 crisp_prefill lays V^T out inside the selection launch
    (four images per extra work-group; 3 KV heads x 6 images leave the last
    one partial), beyond it in a launch of its own, as crisp_attend always
    does: the same lists give the same output bits either way."""
    pat = [synth.VS, synth.DIFFUSE] * (hq // 2) + [synth.VS] * (hq % 2)
    inp = synth.generate(synth.custom_spec(n, hq, hkv, pat, seed_id=400 + n % 97))
    P.log(f"prefill vs stages n={n} hq={hq} hkv={hkv}")
    q, k, v = P.to_dev(inp)
    ws = crisp.alloc_workspace(n, hq, hkv)
    out = torch.empty_like(q)
    crisp.crisp_prefill(q, k, v, 1.0, ws, out)
    gs = P.gpu_select(q, k, P.gpu_route(q, k, ws), 1.0, ws)
    staged = P.gpu_attend(q, k, v, gs["row_ptr"], gs["col_idx"], crisp.alloc_workspace(n, hq, hkv))
    assert torch.equal(out.view(torch.int16), staged.view(torch.int16))


@pytest.mark.parametrize("n", [128, 256, 384, 640])
def test_tiny_sequences(n):
    """N_b = 1, 2 (every block kept), 3 and 5 (ragged proxy tiles)."""
    sp = synth.custom_spec(n, 2, 1, [synth.VS, synth.DIFFUSE], seed_id=60 + n // 128)
    case(synth.generate(sp), tag=f"-n{n}")


@pytest.mark.parametrize("n", [1, 77, 129, 300, 1000, 3000 + 57])
def test_ragged_sequences(n):
    """n not a multiple of B: N_b = ceil(n/B), a partial last block in the
    proxy rows, the slash split, the PE means and the attention tiles."""
    kinds = [synth.VS, synth.DIFFUSE, synth.VS, synth.VS]
    sp = synth.custom_spec(n, 4, 2, kinds, seed_id=100 + n % 97)
    r = case(synth.generate(sp), tag=f"-n{n}")
    # the end-to-end call on the GPU's own lists equals the staged calls
    q, k, v = r["q"], r["k"], r["v"]
    out = torch.empty_like(q)
    crisp.crisp_prefill(q, k, v, 1.0, crisp.alloc_workspace(n, 4, 2), out)
    gs = r["gs"]
    staged = P.gpu_attend(q, k, v, gs["row_ptr"], gs["col_idx"], crisp.alloc_workspace(n, 4, 2))
    assert torch.equal(out.view(torch.int16), staged.view(torch.int16))


def test_ragged_dense_matches_oracle():
    n, hq, hkv = 2048 + 100, 4, 1
    sp = synth.custom_spec(n, hq, hkv, [synth.VS, synth.DIFFUSE, synth.VS, synth.VS], seed_id=111)
    inp = synth.generate(sp)
    nb = -(-n // B)
    q, k, v = P.to_dev(inp)
    out = torch.empty_like(q)
    crisp.crisp_attend_dense(q, k, v, crisp.alloc_workspace(n, hq, hkv), out)
    rp, ci = O.full_causal_lists(hq, nb)
    want = O.attend(inp.q, inp.k, inp.v, n, hq, hkv, 128, rp, ci, np.arange(hq * nb, dtype=np.int32))
    got = torch.zeros(hq, nb * B, 128)
    got[:, :n] = out.float().cpu()
    P.check_outputs(got.numpy().reshape(hq * nb, B, 128), want, "ragged dense")


def test_empty_sequence():
    q = torch.empty(4, 0, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(1, 0, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    crisp.crisp_prefill(q, k, k, 1.0, crisp.alloc_workspace(0, 4, 1), out)
    torch.cuda.synchronize()


@pytest.mark.parametrize("hq,hkv", [(2, 2), (7, 1), (8, 2)])
def test_group_sizes(hq, hkv):
    kinds = [synth.VS if h % 3 else synth.DIFFUSE for h in range(hq)]
    sp = synth.custom_spec(2048 + 384, hq, hkv, kinds, seed_id=70 + hq)
    case(synth.generate(sp), tag=f"-g{hq // hkv}")


@pytest.mark.parametrize("alpha", [0.0, 0.5, 2.0, 1e6])
def test_alpha_extremes(alpha):
    sp = synth.custom_spec(4096, 4, 2, [synth.VS, synth.VS, synth.DIFFUSE, synth.VS], seed_id=80)
    r = case(synth.generate(sp), alpha=alpha, tag=f"-a{alpha}")
    if alpha == 0.0:
        # every block above a zero floor: VS rows are the full causal rows
        gs = r["gs"]
        for h in (0, 1, 3):
            assert gs["counts"][h][0] == 32 and gs["counts"][h][1] == 32
            for qb in range(32):
                assert gs["row_ptr"][h][qb + 1] - gs["row_ptr"][h][qb] == qb + 1


@pytest.mark.parametrize("n", [32 * B, 129 * B])
@pytest.mark.parametrize("gamma", [1.0, 0.05])
def test_gamma_extremes(n, gamma):
    """The PE cut-off at gamma = 1 (the fixed-point mass of the whole map may
    fall just short of it: then every causal entry is kept) and at a small
    gamma (a handful kept), on the one-work-group path (N_b = 32) and the
    multi-launch path (N_b = 129): routing bits, sets and K* against the
    oracle (Alg. 4)."""
    sp = synth.custom_spec(n, 4, 2, [synth.VS, synth.DIFFUSE, synth.DIFFUSE, synth.VS],
                           seed_id=80 + n // B)
    inp = synth.generate(sp)
    q, k, _ = P.to_dev(inp)
    ws = crisp.alloc_workspace(n, 4, 2)
    opts = crisp.default_opts(gamma=gamma)
    gr = P.gpu_route(q, k, ws, opts=opts)
    orc = O.route(inp.q, inp.k, n, 4, 2)
    grh = P.host(gr)
    P.check_route(grh, orc)
    gs = P.host(P.gpu_select(q, k, gr, 1.0, ws, opts=opts))
    rep = P.check_select(inp, grh, gs, 1.0, orc, gamma=gamma)
    P.log(rep.line() + f" gamma={gamma} K*={gs['counts'][:, 2].tolist()}")
    if gamma == 1.0:
        nb = n // B
        for h in range(4):
            if not orc.pattern[h]:
                assert gs["counts"][h][2] >= nb * (nb + 1) // 2 - 2, (h, gs["counts"][h])


@pytest.mark.parametrize("alpha", [0.75, 1.25, 1.5])
def test_alpha_sweep_values(alpha):
    """The other alpha settings the paper evaluates (Sec. 5 setup, App. E)."""
    inp = synth.generate(synth.config_spec("c2"))
    rows = P.sample_rows(32768 // B, 32, 3, seed=int(alpha * 100))
    case(inp, alpha=alpha, rows=rows, tag=f"-a{alpha}")


@pytest.mark.parametrize("tau", [0.15, 0.25])
def test_tau_sweep_values(tau):
    """Routing thresholds of the paper's robustness check (App. E): bits exact,
    then selection on the routes they give."""
    inp = synth.generate(synth.config_spec("c2"))
    n, hq, hkv = 32768, 32, 8
    q, k, _ = P.to_dev(inp)
    ws = crisp.alloc_workspace(n, hq, hkv)
    opts = crisp.default_opts(tau_proxy=tau)
    gr = P.gpu_route(q, k, ws, opts=opts)
    orc = O.route(inp.q, inp.k, n, hq, hkv, tau=tau)
    grh = P.host(gr)
    P.check_route(grh, orc)
    gs = P.host(P.gpu_select(q, k, gr, 1.0, ws, opts=opts))
    P.log(P.check_select(inp, grh, gs, 1.0, orc).line() + f" tau={tau}")


@pytest.mark.parametrize("n", [64 * B, 64 * B + 1, 128 * B, 128 * B + 1])
def test_one_workgroup_path_boundaries(n):
    """Either side of the lengths where the route reductions (N_b <= 64),
    the list expansion and the PE cut-off (N_b <= 128) switch from one
    work-group per head to several launches: routing, sets and CSR against
    the oracle, outputs on sampled rows."""
    sp = synth.custom_spec(n, 4, 2, [synth.VS, synth.DIFFUSE, synth.VS, synth.DIFFUSE],
                           seed_id=140 + n % 7)
    nb = -(-n // B)
    case(synth.generate(sp), rows=P.sample_rows(nb, 4, 8, seed=n % 11), tag=f" n={n}")


@pytest.mark.parametrize("n,gamma", [(16 * B, 0.95), (64 * B, 0.95), (64 * B, 0.5),
                                     (128 * B, 0.95), (129 * B, 0.95), (129 * B, 0.5)])
def test_pe_cutoff_exact_ties(n, gamma):
    """Pooled maps made of exact ties: constant queries, and keys constant
    inside each key block with two values alternating by block, so every row
    of the map holds two groups of equal values.  All heads are sent down the
    PE path (pattern 0).  The gamma cut-off lands inside a group of equal
    values and the flat-order tie rule decides which of them are kept, so K*
    and the kept entries must equal the oracle's exactly: the threshold
    exemption of the other tests would hide a wrong tie rule.  N_b = 16, 64
    and 128 take the one-work-group cut-off, 129 the multi-launch passes."""
    hq, hkv = 2, 1
    nb = n // B
    q = torch.full((hq, n, 128), 1.0, dtype=torch.bfloat16)
    q[1] = 0.5
    k = torch.zeros((hkv, n, 128), dtype=torch.bfloat16)
    k.view(hkv, nb, B, 128)[:, 0::2] = 0.25
    qd, kd = q.cuda(), k.cuda()
    ws = crisp.alloc_workspace(n, hq, hkv)
    z = torch.zeros(hq, nb, dtype=torch.float32, device="cuda")
    r = dict(pattern=torch.zeros(hq, dtype=torch.uint8, device="cuda"), p_v=z, p_s=z)
    gs = P.host(P.gpu_select(qd, kd, r, 1.0, ws, opts=crisp.default_opts(gamma=gamma)))
    tri = nb * (nb + 1) // 2
    keep = np.tril(np.eye(nb, dtype=bool))
    keep[:, 0] = True
    ties_cut = 0
    for h in range(hq):
        ab = O.pe_map(q, k, n, hq, hkv, 128, h)
        s = O.pe_select(ab, gamma)
        kv, ks, kp = gs["counts"][h]
        assert (kv, ks) == (0, 0)
        assert int(kp) == s.kstar, (h, int(kp), s.kstar)
        M = P.rows_matrix(gs["row_ptr"][h], gs["col_idx"], nb)
        assert gs["row_ptr"][h][0] == h * tri
        want = s.mask.astype(bool) | keep
        assert np.array_equal(M, want), (h, np.argwhere(M ^ want)[:10].tolist())
        # heads whose cut-off value is shared by entries the cut keeps and
        # entries it drops
        cut = s.mask.astype(bool)
        eq = (ab.astype(np.float32) == np.float32(s.vstar)) & np.tril(np.ones((nb, nb), dtype=bool))
        ties_cut += int((eq & cut).any() and (eq & ~cut).any())
    assert ties_cut >= 1, "the inputs no longer cut inside a tie group"
    P.log(f"pe ties n={n} gamma={gamma}: K* {gs['counts'][:, 2].tolist()}, cut inside a tie group on {ties_cut} heads")


_C2 = {}


def c2_state():
    """c2 (32768 tokens, 32/8 heads) routed, selected and attended once per
    module: routing and sets checked against the oracle for every head."""
    if not _C2:
        _C2.update(case(synth.generate(synth.config_spec("c2")), rows=np.zeros(0, np.int32)))
    return _C2


@pytest.mark.parametrize("part", range(4))
def test_c2_full_parity(part):
    """Every query block of every head of c2 (all 256 per head, in four
    groups of 8 heads): attention on the oracle's lists against the oracle."""
    st = c2_state()
    nb, hq = 32768 // B, 32
    heads = np.arange(8 * part, 8 * part + 8)
    rows = (heads[:, None] * nb + np.arange(nb)[None, :]).reshape(-1).astype(np.int32)
    inp, plan, out = st["inp"], st["plan"], st["out"]
    want = O.attend(inp.q, inp.k, inp.v, 32768, hq, 8, 128, plan.row_ptr, plan.col_idx, rows)
    got = out.view(hq * nb, B, 128)[torch.as_tensor(rows, dtype=torch.long, device=out.device)]
    got = got.float().cpu().numpy()
    P.check_outputs(got, want, f"c2 heads {heads[0]}-{heads[-1]} attend")
    for h in heads:
        m = rows // nb == h
        P.check_outputs(got[m], want[m], f"c2 head {h}")
    P.record("c2", f"attention_heads_{heads[0]}_{heads[-1]}", P.attention_record(got, want, rows // nb))


def test_select_is_deterministic():
    inp = synth.generate(synth.config_spec("c2"))
    q, k, v = P.to_dev(inp)
    ws = crisp.alloc_workspace(32768, 32, 8)
    gr = P.gpu_route(q, k, ws)
    a = P.host(P.gpu_select(q, k, gr, 1.0, ws))
    for _ in range(3):
        b = P.host(P.gpu_select(q, k, gr, 1.0, ws))
        for key in a:
            assert np.array_equal(a[key], b[key]), key


# -------------------------------------- selection rules and the baseline
@pytest.mark.parametrize("alpha", [1.0, 2.0])
def test_median_noise_floor(alpha):
    """Appendix H's median floor: sets against the oracle, outputs on the
    oracle's lists, and the prefill equal to the staged calls."""
    sp = synth.custom_spec(8192 + 300, 8, 2, [synth.VS, synth.VS, synth.VS, synth.DIFFUSE,
                                              synth.VS, synth.CONC, synth.DIST, synth.DIFFUSE],
                           seed_id=120)
    inp = synth.generate(sp)
    n, hq, hkv = sp.n, sp.hq, sp.hkv
    opts = crisp.default_opts(vs_rule=crisp.VS_NOISE_MEDIAN)
    q, k, v = P.to_dev(inp)
    ws = crisp.alloc_workspace(n, hq, hkv)
    gr = P.gpu_route(q, k, ws, opts=opts)
    grh = P.host(gr)
    orc_r = O.route(inp.q, inp.k, n, hq, hkv)
    P.check_route(grh, orc_r)
    gs = P.host(P.gpu_select(q, k, gr, alpha, ws, opts=opts))
    rep = P.check_select(inp, grh, gs, alpha, orc_r, vs_rule="median")
    P.log(rep.line() + f" median alpha={alpha}")
    plan = O.plan(inp.q, inp.k, n, hq, hkv, alpha=alpha, routed=orc_r, vs_rule="median")
    nb = -(-n // B)
    rows = P.sample_rows(nb, hq, 12, seed=7)
    out = P.gpu_attend(q, k, v, plan.row_ptr, plan.col_idx, ws)
    want = O.attend(inp.q, inp.k, inp.v, n, hq, hkv, 128, plan.row_ptr, plan.col_idx, rows)
    full = torch.zeros(hq, nb * B, 128)
    full[:, :n] = out.float().cpu()
    P.check_outputs(full.numpy().reshape(hq * nb, B, 128)[rows], want, f"median alpha={alpha}")
    out2 = torch.empty_like(q)
    crisp.crisp_prefill(q, k, v, alpha, crisp.alloc_workspace(n, hq, hkv), out2, opts=opts)
    staged = P.gpu_attend(q, k, v, gs["row_ptr"], gs["col_idx"], crisp.alloc_workspace(n, hq, hkv))
    assert torch.equal(out2.view(torch.int16), staged.view(torch.int16))


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_flexprefill_baseline(name):
    """Appendix A: JSD routing (Alg. 5) and the cumulative gamma rule with
    the k_min clip (Alg. 6) against the oracle, then attention parity."""
    inp = synth.generate(synth.config_spec(name))
    sp = inp.spec
    n, hq, hkv = sp.n, sp.hq, sp.hkv
    opts = crisp.flexprefill_opts()
    q, k, v = P.to_dev(inp)
    ws = crisp.alloc_workspace(n, hq, hkv)
    gr = P.gpu_route(q, k, ws, opts=opts)
    grh = P.host(gr)
    orc_r = O.route_jsd(inp.q, inp.k, n, hq, hkv)
    P.check_route_jsd(grh, orc_r)
    P.log(f"{name} D_JS: {np.round(orc_r.c_struct, 3).tolist()} VS heads {int(orc_r.pattern.sum())}/{hq}")
    gs = P.host(P.gpu_select(q, k, gr, 1.0, ws, opts=opts))
    # heads whose bits agree are compared set by set
    same = [h for h in range(hq) if grh["pattern"][h] == orc_r.pattern[h]]
    rep = P.check_select(inp, grh, gs, 1.0, orc_r, heads=same, vs_rule="gamma")
    P.log(rep.line() + " flexprefill")
    plan = O.plan(inp.q, inp.k, n, hq, hkv, routed=orc_r, vs_rule="gamma")
    nb = -(-n // B)
    rows = P.sample_rows(nb, hq, 8, seed=11)
    out = P.gpu_attend(q, k, v, plan.row_ptr, plan.col_idx, ws)
    want = O.attend(inp.q, inp.k, inp.v, n, hq, hkv, 128, plan.row_ptr, plan.col_idx, rows)
    got = out.float().cpu().numpy().reshape(hq * nb, B, 128)[rows]
    P.check_outputs(got, want, f"{name} flexprefill attend")
    out2 = torch.empty_like(q)
    crisp.crisp_prefill(q, k, v, 1.0, crisp.alloc_workspace(n, hq, hkv), out2, opts=opts)
    staged = P.gpu_attend(q, k, v, gs["row_ptr"], gs["col_idx"], crisp.alloc_workspace(n, hq, hkv))
    assert torch.equal(out2.view(torch.int16), staged.view(torch.int16))


def test_flexprefill_ragged():
    """The baseline's router and rule on a ragged length (partial last block
    in the key means, the pooled estimate and the gamma rule)."""
    n, hq, hkv = 3000 + 57, 4, 2
    sp = synth.custom_spec(n, hq, hkv, [synth.VS, synth.DIFFUSE, synth.VS, synth.VS], seed_id=130)
    inp = synth.generate(sp)
    nb = -(-n // B)
    opts = crisp.flexprefill_opts()
    q, k, v = P.to_dev(inp)
    ws = crisp.alloc_workspace(n, hq, hkv)
    gr = P.gpu_route(q, k, ws, opts=opts)
    grh = P.host(gr)
    orc_r = O.route_jsd(inp.q, inp.k, n, hq, hkv)
    P.check_route_jsd(grh, orc_r)
    gs = P.host(P.gpu_select(q, k, gr, 1.0, ws, opts=opts))
    same = [h for h in range(hq) if grh["pattern"][h] == orc_r.pattern[h]]
    P.log(P.check_select(inp, grh, gs, 1.0, orc_r, heads=same, vs_rule="gamma").line() + " ragged fp")
    out = torch.empty_like(q)
    crisp.crisp_prefill(q, k, v, 1.0, crisp.alloc_workspace(n, hq, hkv), out, opts=opts)
    rows = np.arange(hq * nb, dtype=np.int32)
    want = O.attend(inp.q, inp.k, inp.v, n, hq, hkv, 128, gs["row_ptr"].reshape(-1), gs["col_idx"],
                    rows)
    full = torch.zeros(hq, nb * B, 128)
    full[:, :n] = out.float().cpu()
    P.check_outputs(full.numpy().reshape(hq * nb, B, 128), want, "ragged flexprefill prefill")
