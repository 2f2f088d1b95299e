"""Pins of the CPU oracle against what the paper and the mathematics fix.

None of these re-types the oracle's own loops: proxy maps and attention are
checked against numpy / torch softmax with explicit masks, diagonal scores
against numpy.trace, selections against exhaustive search over subsets, and
several quantities against closed forms (uniform logits; the two-level model
of Appendix C of the CRISP paper).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def rand_qkv(n, hq, hkv, d, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(hq, n, d, generator=g) * scale).to(torch.bfloat16)
    k = (torch.randn(hkv, n, d, generator=g) * scale).to(torch.bfloat16)
    v = torch.randn(hkv, n, d, generator=g).to(torch.bfloat16)
    return q, k, v


def brute_proxy(q, k, h, G, B):
    """A^ by numpy: masked logits, softmax along keys (float64)."""
    n, d = q.shape[1], q.shape[2]
    qh = q[h, n - B:].double().numpy()
    kg = k[h // G].double().numpy()
    s = qh @ kg.T / math.sqrt(d)
    pos = np.arange(n)
    qi = n - B + np.arange(B)
    s[pos[None, :] > qi[:, None]] = -np.inf
    s -= s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=1, keepdims=True)


def brute_scores(ahat, B):
    """colmean / diagmean via numpy.trace / blockpool by reshape."""
    Bq, n = ahat.shape
    nb = n // B
    a_v = ahat.mean(axis=0)
    a_s = np.array([np.trace(ahat, offset=sig - (Bq - 1)) for sig in range(n)]) / Bq
    return a_v.reshape(nb, B).sum(1), a_s.reshape(nb, B).sum(1)


# ------------------------------------------------------------------ golden
def test_paper_defaults_match_golden():
    gd = json.load(open(os.path.join(GOLDEN, "paper_defaults.json")))
    assert O.TAU_PROXY == gd["tau_proxy"]["value"]
    assert O.GAMMA == gd["gamma_pe"]["value"]
    assert O.K_MIN_TOKENS == gd["k_min_tokens"]["value"]
    assert O.K_MIN_TOKENS // gd["block_size"]["value"] == gd["k_min_blocks"]["value"]
    assert O.W_SINK == gd["w_sink"]["value"] == gd["block_size"]["value"]
    assert O.W_LOCAL == gd["w_local"]["value"] == gd["block_size"]["value"]


# ------------------------------------------------------------ proxy + scores
@pytest.mark.parametrize("n,d,B", [(256, 16, 32), (384, 128, 128), (512, 128, 128), (512, 16, 64)])
def test_proxy_and_scores_bruteforce(n, d, B):
    hq, hkv = 4, 2
    q, k, _ = rand_qkv(n, hq, hkv, d, seed=n + d + B, scale=1.5)
    for h in range(hq):
        a_or = O.proxy_map(q, k, n, hq, hkv, d, h, B)
        a_bf = brute_proxy(q, k, h, hq // hkv, B)
        np.testing.assert_allclose(a_or, a_bf, rtol=1e-12, atol=1e-15)
        pv, ps, cs = O.block_scores(a_or, B, B, B)
        pv_bf, ps_bf = brute_scores(a_bf, B)
        np.testing.assert_allclose(pv, pv_bf, rtol=1e-11, atol=1e-15)
        np.testing.assert_allclose(ps, ps_bf, rtol=1e-11, atol=1e-15)
        # Eq. 2 with w_sink = w_local = B is the first plus the last block
        anchor = np.zeros(n, bool)
        anchor[:B] = True
        anchor[n - B:] = True
        assert cs == pytest.approx(a_bf[:, anchor].sum(1).mean(), rel=1e-12)
        if n // B > 1:
            assert cs == pytest.approx(pv[0] + pv[-1], rel=1e-12)


def test_slash_tile_split_identity():
    """(i, k) in key tile t lands in slash block t if c <= i, else t+1."""
    n, d, B = 512, 16, 64
    q, k, _ = rand_qkv(n, 1, 1, d, seed=5)
    a = brute_proxy(q, k, 0, 1, B)
    nb = n // B
    ps = np.zeros(nb + 1)
    for t in range(nb):
        tile = a[:, t * B:(t + 1) * B]
        lo = np.tril(tile).sum()        # c <= i
        up = np.triu(tile, 1).sum()     # c > i
        ps[t] += lo / B
        ps[t + 1] += up / B
    _, ps_bf = brute_scores(a, B)
    assert ps[nb] == pytest.approx(0.0, abs=1e-15)
    np.testing.assert_allclose(ps[:nb], ps_bf, rtol=1e-11, atol=1e-15)


@pytest.mark.parametrize("n,B", [(1024, 128), (256, 32)])
def test_score_invariants(n, B):
    d = 64
    q, k, _ = rand_qkv(n, 2, 1, d, seed=11, scale=2.0)
    r = O.route(q, k, n, 2, 1, d, B, 0.2, B, B)
    for h in range(2):
        a = O.proxy_map(q, k, n, 2, 1, d, h, B)
        np.testing.assert_allclose(a.sum(1), 1.0, atol=1e-12)
        assert r.p_v[h].sum() == pytest.approx(1.0, abs=1e-12)
        assert r.p_s[h].sum() == pytest.approx(1.0, abs=1e-12)
        assert r.p_s[h][0] <= r.p_v[h][0] + 1e-15
        assert np.all(r.p_v[h] >= 0) and np.all(r.p_s[h] >= 0)


def test_uniform_logits_closed_form():
    """Q = 0: row i is uniform over its q_i + 1 visible keys."""
    n, B = 4096, 128
    q = torch.zeros(1, n, 128, dtype=torch.bfloat16)
    _, k, _ = rand_qkv(n, 1, 1, 128, seed=3)
    r = O.route(q, k, n, 1, 1)
    qi = n - B + np.arange(B)
    pv0 = np.mean(B / (qi + 1.0))
    pvl = np.mean((np.arange(B) + 1.0) / (qi + 1.0))
    assert r.p_v[0][0] == pytest.approx(pv0, rel=1e-12)
    assert r.p_v[0][-1] == pytest.approx(pvl, rel=1e-12)
    assert r.c_struct[0] == pytest.approx(pv0 + pvl, rel=1e-12)
    assert r.c_struct[0] == pytest.approx(0.047, abs=0.001)
    assert r.pattern[0] == 0                  # diffuse: PE (Alg. 2)


def test_one_hot_sink_routes_vs():
    n, d = 4096, 16
    q = torch.zeros(1, n, d)
    k = torch.zeros(1, n, d)
    q[0, :, 0] = 8.0
    k[0, 0, 0] = 15.0                          # logit 8*15/4 = 30 on token 0
    r = O.route(q.to(torch.bfloat16), k.to(torch.bfloat16), n, 1, 1, d)
    assert r.c_struct[0] > 0.999999
    assert r.pattern[0] == 1


def two_level(n, d, B, k_sig, a=4.0, b_sig=3.0, b_bg=1.0, sig_pos=None):
    """Appendix C model: identical query rows; k_sig keys at logit z, the rest at z - Delta."""
    q = torch.zeros(1, n, d)
    q[0, :, 0] = a
    k = torch.zeros(1, n, d)
    k[0, :, 0] = b_bg
    pos = np.arange(k_sig) if sig_pos is None else np.asarray(sig_pos)
    k[0, pos, 0] = b_sig
    s = 1.0 / math.sqrt(d)
    z, zb = a * b_sig * s, a * b_bg * s
    return q.to(torch.bfloat16), k.to(torch.bfloat16), z, z - zb, pos


def test_two_level_model_appendix_c():
    n, d, B, ks = 2048, 16, 128, 4
    q, k, z, delta, pos = two_level(n, d, B, ks)
    a = O.proxy_map(q, k, n, 1, 1, d, 0, B)
    # last row sees all n keys: background mass eps of Appendix C
    eps = math.exp(-delta) / (ks + (n - ks) * math.exp(-delta))
    assert a[B - 1, n - 1] == pytest.approx(eps, rel=1e-12)
    assert a[B - 1, 0] == pytest.approx(1.0 / (ks + (n - ks) * math.exp(-delta)), rel=1e-12)
    # every row: m = q_i + 1 visible keys
    pv, ps, cs = O.block_scores(a, B, B, B)
    qi = n - B + np.arange(B)
    zrow = ks + (qi + 1 - ks) * math.exp(-delta)
    pv_exact = np.zeros(n // B)
    pv_exact[0] = np.mean((ks + (B - ks) * math.exp(-delta)) / zrow)
    pv_exact[1:-1] = np.mean(B * math.exp(-delta) / zrow)
    pv_exact[-1] = np.mean((np.arange(B) + 1) * math.exp(-delta) / zrow)
    np.testing.assert_allclose(pv, pv_exact, rtol=1e-11)


def test_gamma_noise_count_appendix_c():
    """gamma-cumsum takes ceil(gamma_res / eps_blk) background blocks (App. C),
    a count that grows with n while the sink mass a_sink falls."""
    d, B, ks = 16, 128, 8
    counts = []
    for n in (4096, 8192, 16384):
        q, k, z, delta, pos = two_level(n, d, B, ks, b_sig=9.0, b_bg=1.0)
        assert delta == pytest.approx(8.0)
        r = O.route(q, k, n, 1, 1, d, B)
        pv = r.p_v[0]
        qi = n - B + np.arange(B)
        zrow = ks + (qi + 1 - ks) * math.exp(-delta)
        a_sink = np.mean((ks + (B - ks) * math.exp(-delta)) / zrow)
        eps_blk = np.mean(B * math.exp(-delta) / zrow)
        assert pv[0] == pytest.approx(a_sink, rel=1e-12)
        gres = 0.95 - a_sink
        assert 0 < gres < (n // B - 2) * eps_blk
        sel = O.gamma_select(pv, 0.95)
        n_garbage = len([j for j in sel if j != 0])
        assert n_garbage == math.ceil(gres / eps_blk)
        counts.append(n_garbage)
    assert counts[0] < counts[1] < counts[2]


# -------------------------------------------------------------- VS select
def brute_vs(p, alpha, kmin):
    pf = p.astype(np.float32)
    nb = len(pf)
    r = max(np.float32(1.0) - pf[0] - pf[-1], np.float32(0.0))
    mu = np.float32(r) / np.float32(nb - 2)
    th = np.float32(alpha) * mu
    cnt = int((pf > th).sum())
    kk = min(max(cnt, kmin), nb)
    best, best_key = None, None
    for sub in itertools.combinations(range(nb), kk):
        key = (float(np.sum(pf[list(sub)], dtype=np.float64)), [-j for j in sub])
        if best is None or key > best_key:
            best, best_key = sub, key
    return sorted(best)


@pytest.mark.parametrize("seed", range(12))
def test_vs_select_bruteforce_subsets(seed):
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(5, 12))
    p = rng.random(nb) ** 3
    p[0] += rng.random() * 3
    p /= p.sum()
    for alpha in (0.5, 1.0, 1.5, 3.0):
        for kmin in (1, 2, 4):
            got = O.vs_select(p, alpha, kmin).sel.tolist()
            assert got == brute_vs(p, alpha, kmin), (alpha, kmin)


def test_vs_select_handbuilt():
    # floor case: r = 1 - 0.5 - 0.1 = 0.4, mu = 0.4 / 8 = 0.05
    p = np.array([0.5, 0.2, 0.01, 0.06, 0.01, 0.04, 0.01, 0.05, 0.02, 0.1])
    s = O.vs_select(p, 1.0, 2)
    assert s.sel.tolist() == [0, 1, 3, 9]     # 0.05 is not > 0.05
    assert s.theta == pytest.approx(0.05, rel=1e-6) and not s.clipped
    # clipped case: top-k_min with ties to the lower index
    p2 = np.array([0.9, 0.01, 0.02, 0.02, 0.01, 0.02, 0.01, 0.01])
    s2 = O.vs_select(p2 / p2.sum(), 100.0, 4)
    assert s2.clipped and s2.sel.tolist() == [0, 2, 3, 5]
    # r clamped at 0: every positive block passes
    p3 = np.array([0.7, 0.05, 0.02, 0.01, 0.4])
    s3 = O.vs_select(p3, 1.0, 1)
    assert s3.theta == 0.0 and s3.sel.tolist() == [0, 1, 2, 3, 4]


def test_vs_select_alpha_extremes():
    rng = np.random.default_rng(7)
    p = rng.random(64)
    p /= p.sum()
    assert O.vs_select(p, 0.0, 8).sel.tolist() == list(range(64))   # all p > 0
    top8 = sorted(np.argsort(-p, kind="stable")[:8].tolist())
    assert O.vs_select(p, 1e30, 8).sel.tolist() == top8


def test_vs_select_tiny_nb_selects_all():
    for nb in (1, 2):
        assert O.vs_select(np.ones(nb) / nb, 1.0, 8).sel.tolist() == list(range(nb))


# ----------------------------------------------------------- gamma select
@pytest.mark.parametrize("seed", range(8))
def test_gamma_select_minimal_cardinality(seed):
    rng = np.random.default_rng(100 + seed)
    nb = 10
    p = rng.random(nb) ** 2
    p /= p.sum()
    sel = O.gamma_select(p, 0.95)
    pf = p.astype(np.float32).astype(np.float64)
    assert pf[sel].sum() >= np.float64(np.float32(0.95))
    for kk in range(1, len(sel)):
        for sub in itertools.combinations(range(nb), kk):
            assert pf[list(sub)].sum() < np.float64(np.float32(0.95))
    clipped = O.gamma_select(p, 0.95, kmin_blocks=nb)
    assert clipped.tolist() == list(range(nb))


# ---------------------------------------------------------------- PE path
def brute_pe_map(q, k, h, G, B):
    n, d = q.shape[1], q.shape[2]
    nb = n // B
    qb = q[h].double().numpy().reshape(nb, B, d).mean(1)
    kb = k[h // G].double().numpy().reshape(nb, B, d).mean(1)
    s = qb @ kb.T / math.sqrt(d)
    s[np.triu(np.ones((nb, nb), bool), 1)] = -np.inf
    s -= s.max(1, keepdims=True)
    e = np.exp(s)
    a = e / e.sum(1, keepdims=True)
    return a / a.sum()


@pytest.mark.parametrize("n,d,B", [(512, 16, 32), (1024, 128, 128)])
def test_pe_map_bruteforce(n, d, B):
    q, k, _ = rand_qkv(n, 4, 2, d, seed=21, scale=3.0)
    for h in range(4):
        np.testing.assert_allclose(O.pe_map(q, k, n, 4, 2, d, h, B), brute_pe_map(q, k, h, 2, B),
                                   rtol=1e-11, atol=1e-16)


@pytest.mark.parametrize("seed", range(10))
def test_pe_select_exhaustive(seed):
    rng = np.random.default_rng(200 + seed)
    nb = 4
    a = np.tril(rng.random((nb, nb)) ** 3)
    a /= a.sum()
    gamma = float(rng.choice([0.5, 0.8, 0.95]))
    s = O.pe_select(a, gamma)
    vals = a.astype(np.float32).astype(np.float64)
    causal = [(i, j) for i in range(nb) for j in range(i + 1)]
    g32 = np.float64(np.float32(gamma))
    best = min(kk for kk in range(1, len(causal) + 1)
               for sub in itertools.combinations(causal, kk)
               if sum(vals[e] for e in sub) >= g32)
    assert s.kstar == best
    assert s.mask.sum() == best
    assert sum(vals[e] for e in causal if s.mask[e]) >= g32
    assert np.all(np.triu(s.mask, 1) == 0)


def test_pe_uniform_closed_form():
    """Q = 0: entry (qb, kb) = 1 / ((qb+1) Nb); K* follows by counting."""
    n, B, d = 2048, 128, 128
    nb = n // B
    q = torch.zeros(1, n, d, dtype=torch.bfloat16)
    _, k, _ = rand_qkv(n, 1, 1, d, seed=4)
    a = O.pe_map(q, k, n, 1, 1, d, 0, B)
    exact = np.tril(1.0 / ((np.arange(nb)[:, None] + 1.0) * nb) * np.ones((nb, nb)))
    np.testing.assert_allclose(a, exact, rtol=1e-13)
    gamma = 0.3
    s = O.pe_select(a, gamma)
    # rows 0..r-1 hold r/Nb; row r's entries hold 1/((r+1)Nb) each
    g = float(np.float32(gamma))
    r = int(math.floor(g * nb))
    need = math.ceil((g * nb - r) * (r + 1) - 1e-9)
    assert s.kstar == r * (r + 1) // 2 + need
    # ties in row r resolve to the lowest flat index: its first `need` entries
    assert s.mask[r, :need].all() and not s.mask[r, need:].any()


# ------------------------------------------------------------------ expand
@pytest.mark.parametrize("seed", range(6))
def test_expand_bruteforce(seed):
    rng = np.random.default_rng(300 + seed)
    nb = int(rng.integers(3, 40))
    sv = np.sort(rng.choice(nb, size=int(rng.integers(1, nb)), replace=False))
    ss = np.sort(rng.choice(nb, size=int(rng.integers(1, nb)), replace=False))
    row_ptr, col, cnt = O.expand(nb, True, sv, ss)
    ref = np.zeros((nb, nb), bool)
    for qb in range(nb):
        for kb in range(qb + 1):
            off = qb - kb                       # diagonal offset block
            ref[qb, kb] = (kb == 0 or kb == qb or kb in set(sv.tolist())
                           or (nb - 1 - off) in set(ss.tolist()))
    for qb in range(nb):
        row = col[row_ptr[qb]:row_ptr[qb + 1]]
        assert row.tolist() == np.nonzero(ref[qb])[0].tolist()
        assert row[0] == 0 and row[-1] == qb and np.all(np.diff(row) > 0)
    assert cnt == ref.sum()
    # PE rows: selected pairs plus {0, qb}
    pm = np.tril(rng.random((nb, nb)) < 0.3).astype(np.uint8)
    rp2, col2, _ = O.expand(nb, False, pe_mask=pm)
    for qb in range(nb):
        want = set(np.nonzero(pm[qb, :qb + 1])[0].tolist()) | {0, qb}
        assert col2[rp2[qb]:rp2[qb + 1]].tolist() == sorted(want)


# ------------------------------------------------------------------ attend
def sdpa64(q, k, v, G, mask):
    """torch float64 softmax attention with an explicit boolean mask."""
    qd = q.double()
    kd = k.double().repeat_interleave(G, 0)
    vd = v.double().repeat_interleave(G, 0)
    return torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, attn_mask=mask)


@pytest.mark.parametrize("n,d,B", [(256, 16, 32), (512, 128, 128)])
def test_attend_dense_is_textbook(n, d, B):
    hq, hkv = 4, 2
    nb = n // B
    q, k, v = rand_qkv(n, hq, hkv, d, seed=31, scale=1.2)
    rp, ci = O.full_causal_lists(hq, nb)
    rows = np.arange(hq * nb)
    out = O.attend(q, k, v, n, hq, hkv, d, rp, ci, rows, B).reshape(hq, n, d)
    causal = torch.ones(n, n, dtype=torch.bool).tril()
    ref = sdpa64(q, k, v, hq // hkv, causal).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    # row 0 attends to key 0 only
    np.testing.assert_array_equal(out[:, 0], v.double().numpy().repeat(hq // hkv, 0)[:, 0])


def test_attend_sparse_matches_explicit_mask():
    n, d, B = 512, 16, 32
    hq, hkv = 2, 1
    nb = n // B
    q, k, v = rand_qkv(n, hq, hkv, d, seed=41, scale=1.5)
    rng = np.random.default_rng(9)
    per = nb * (nb + 1) // 2
    row_ptr = np.zeros((hq, nb + 1), np.int32)
    col = np.zeros(hq * per, np.int32)
    mask = torch.zeros(hq, n, n, dtype=torch.bool)
    for h in range(hq):
        sv = np.sort(rng.choice(nb, 3, replace=False))
        ss = np.sort(rng.choice(nb, 3, replace=False))
        rp, _, _ = O.expand(nb, True, sv, ss, base=h * per, col_idx=col)
        row_ptr[h] = rp
        for qb in range(nb):
            for kb in col[rp[qb]:rp[qb + 1]]:
                mask[h, qb * B:(qb + 1) * B, kb * B:(kb + 1) * B] = True
    mask &= torch.ones(n, n, dtype=torch.bool).tril()
    out = O.attend(q, k, v, n, hq, hkv, d, row_ptr, col, np.arange(hq * nb), B).reshape(hq, n, d)
    ref = sdpa64(q, k, v, 2, mask).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    # a subset of rows in any order gives the same values
    rows = np.array([5, 0, nb + 3])
    sub = O.attend(q, k, v, n, hq, hkv, d, row_ptr, col, rows, B)
    for t, r in enumerate(rows):
        h, qb = divmod(int(r), nb)
        np.testing.assert_allclose(sub[t], out[h, qb * B:(qb + 1) * B], rtol=1e-12)


def test_attend_queries_is_textbook():
    n, d, B = 384, 16, 32
    hq, hkv = 2, 1
    nb = n // B
    q, k, v = rand_qkv(n, hq, hkv, d, seed=51, scale=1.3)
    rp, ci = O.full_causal_lists(hq, nb)
    sel = np.array([[0, 0], [1, n - 1], [0, 77], [1, 200]], dtype=np.int32)
    got = O.attend_queries(q, k, v, n, hq, hkv, d, rp, ci, sel, B)
    ref = sdpa64(q, k, v, 2, torch.ones(n, n, dtype=torch.bool).tril()).numpy()
    for i, (h, t) in enumerate(sel):
        np.testing.assert_allclose(got[i], ref[h, t], rtol=1e-10, atol=1e-12)


# ------------------------------------------------- ragged n (N_b = ceil(n/B))
def brute_proxy_any(q, k, h, G, B):
    """A^ for any n: the last R = min(B, n) query rows, causal."""
    n, d = q.shape[1], q.shape[2]
    R = min(B, n)
    qh = q[h, n - R:].double().numpy()
    kg = k[h // G].double().numpy()
    s = qh @ kg.T / math.sqrt(d)
    qi = n - R + np.arange(R)
    s[np.arange(n)[None, :] > qi[:, None]] = -np.inf
    s -= s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=1, keepdims=True)


def brute_scores_any(a, B):
    """p_v by block column sums (partial last block); p_s by the offset of
    every entry from its query's diagonal: slash block Nb-1-floor(o/B)."""
    R, n = a.shape
    nb = -(-n // B)
    starts = np.arange(0, n, B)
    pv = np.add.reduceat(a.sum(0), starts) / R
    qi = (n - R + np.arange(R))[:, None]
    kk = np.arange(n)[None, :]
    valid = kk <= qi
    j = nb - 1 - (qi - kk) // B
    ps = np.zeros(nb)
    np.add.at(ps, j[valid], a[valid])
    return pv, ps / R


@pytest.mark.parametrize("n,B", [(1, 128), (100, 128), (129, 128), (300, 128), (200, 64),
                                 (1000, 128), (1111, 32)])
def test_ragged_proxy_and_scores_bruteforce(n, B):
    d, hq, hkv = 32, 2, 1
    q, k, _ = rand_qkv(n, hq, hkv, d, seed=n + B, scale=1.5)
    nb = -(-n // B)
    r = O.route(q, k, n, hq, hkv, d, B, 0.2, B, B)
    for h in range(hq):
        a = O.proxy_map(q, k, n, hq, hkv, d, h, B)
        a_bf = brute_proxy_any(q, k, h, hq // hkv, B)
        assert a.shape == (min(B, n), n)
        np.testing.assert_allclose(a, a_bf, rtol=1e-12, atol=1e-15)
        pv_bf, ps_bf = brute_scores_any(a_bf, B)
        np.testing.assert_allclose(r.p_v[h], pv_bf, rtol=1e-11, atol=1e-15)
        np.testing.assert_allclose(r.p_s[h], ps_bf, rtol=1e-11, atol=1e-15)
        assert r.p_v[h].sum() == pytest.approx(1.0, abs=1e-12)
        assert r.p_s[h].sum() == pytest.approx(1.0, abs=1e-12)
        # C_struct: mass of the first and the last block (one block if Nb = 1)
        anchor = np.zeros(n, bool)
        anchor[:B] = True
        anchor[(nb - 1) * B:] = True
        assert r.c_struct[h] == pytest.approx(a_bf[:, anchor].sum(1).mean(), rel=1e-12)
        want = pv_bf[0] + (pv_bf[-1] if nb > 1 else 0.0)
        assert r.c_struct[h] == pytest.approx(want, rel=1e-12)


def test_ragged_offset_reading_equals_trace_reading_when_aligned():
    """For n a multiple of B the offset-indexed slash blocks equal the
    diagonal-trace definition (sigma = k + B-1-i) used for aligned n."""
    n, B, d = 512, 64, 16
    q, k, _ = rand_qkv(n, 1, 1, d, seed=77)
    a = brute_proxy_any(q, k, 0, 1, B)
    pv1, ps1 = brute_scores_any(a, B)
    pv2, ps2 = brute_scores(a, B)
    np.testing.assert_allclose(pv1, pv2, rtol=1e-12)
    np.testing.assert_allclose(ps1, ps2, rtol=1e-12)


def test_ragged_uniform_closed_form():
    """Q = 0, n = 1000: row i is uniform over q_i + 1 keys; the last block
    holds 1000 - 7*128 = 104 keys."""
    n, B = 1000, 128
    q = torch.zeros(1, n, 128, dtype=torch.bfloat16)
    _, k, _ = rand_qkv(n, 1, 1, 128, seed=6)
    r = O.route(q, k, n, 1, 1)
    qi = n - B + np.arange(B)
    pv0 = np.mean(B / (qi + 1.0))
    last0 = 7 * B
    pvl = np.mean(np.maximum(qi - last0 + 1, 0) / (qi + 1.0))
    assert r.p_v[0][0] == pytest.approx(pv0, rel=1e-12)
    assert r.p_v[0][-1] == pytest.approx(pvl, rel=1e-12)
    # slash recency block: offsets 0..127 of every row
    assert r.p_s[0][-1] == pytest.approx(np.mean(B / (qi + 1.0)), rel=1e-12)


def brute_pe_map_any(q, k, h, G, B):
    n, d = q.shape[1], q.shape[2]
    nb = -(-n // B)
    qd, kd = q[h].double().numpy(), k[h // G].double().numpy()
    qb = np.stack([qd[b * B:(b + 1) * B].mean(0) for b in range(nb)])
    kb = np.stack([kd[b * B:(b + 1) * B].mean(0) for b in range(nb)])
    s = qb @ kb.T / math.sqrt(d)
    s[np.triu(np.ones((nb, nb), bool), 1)] = -np.inf
    s -= s.max(1, keepdims=True)
    e = np.exp(s)
    a = e / e.sum(1, keepdims=True)
    return a / a.sum()


@pytest.mark.parametrize("n,B", [(300, 128), (1000, 128), (77, 32), (5, 128)])
def test_ragged_pe_map_bruteforce(n, B):
    d = 32
    q, k, _ = rand_qkv(n, 2, 1, d, seed=500 + n, scale=3.0)
    for h in range(2):
        np.testing.assert_allclose(O.pe_map(q, k, n, 2, 1, d, h, B), brute_pe_map_any(q, k, h, 2, B),
                                   rtol=1e-11, atol=1e-16)


@pytest.mark.parametrize("n,B", [(1, 32), (37, 32), (300, 128), (1000, 128)])
def test_ragged_attend_is_textbook(n, B):
    d, hq, hkv = 16, 4, 2
    nb = -(-n // B)
    q, k, v = rand_qkv(n, hq, hkv, d, seed=700 + n, scale=1.2)
    rp, ci = O.full_causal_lists(hq, nb)
    out = O.attend(q, k, v, n, hq, hkv, d, rp, ci, np.arange(hq * nb), B).reshape(hq, nb * B, d)
    causal = torch.ones(n, n, dtype=torch.bool).tril()
    ref = sdpa64(q, k, v, hq // hkv, causal).numpy()
    np.testing.assert_allclose(out[:, :n], ref, rtol=1e-10, atol=1e-12)
    assert np.all(out[:, n:] == 0)
    sel = np.array([[h, p] for h in range(hq) for p in (0, n - 1, n // 2)], dtype=np.int32)
    one = O.attend_queries(q, k, v, n, hq, hkv, d, rp, ci, sel, B)
    np.testing.assert_allclose(one, ref[sel[:, 0], sel[:, 1]], rtol=1e-10, atol=1e-12)


def test_ragged_plan_small_nb_is_dense():
    """N_b <= 2 (mu = r / (N_b - 2) undefined) selects every causal block."""
    for n in (50, 200, 256):
        q, k, _ = rand_qkv(n, 2, 1, 128, seed=n)
        p = O.plan(q, k, n, 2, 1)
        rp, ci = O.full_causal_lists(2, -(-n // 128))
        for h in range(2):
            lens = np.diff(p.row_ptr[h])
            assert lens.tolist() == np.diff(rp[h]).tolist()


# ------------------------------------------- FlexPrefill baseline (App. A)
def brute_abar(q, k, h, G, B):
    """Alg. 5 by numpy: softmax over blocks of the pooled query and
    the per-block key means."""
    n, d = q.shape[1], q.shape[2]
    R = min(B, n)
    nb = -(-n // B)
    qbar = q[h, n - R:].double().numpy().mean(0)
    kd = k[h // G].double().numpy()
    kbar = np.stack([kd[b * B:(b + 1) * B].mean(0) for b in range(nb)])
    z = kbar @ qbar / math.sqrt(d)
    e = np.exp(z - z.max())
    return e / e.sum()


@pytest.mark.parametrize("n,B", [(1024, 128), (1000, 128), (640, 64)])
def test_jsd_matches_scipy(n, B):
    from scipy.spatial.distance import jensenshannon
    d, hq, hkv = 32, 4, 2
    q, k, _ = rand_qkv(n, hq, hkv, d, seed=900 + n, scale=2.0)
    r = O.route(q, k, n, hq, hkv, d, B, 0.2, B, B)
    rj = O.route_jsd(q, k, n, hq, hkv, d, B, 0.1, routed=r)
    for h in range(hq):
        pv_bf, _ = brute_scores_any(brute_proxy_any(q, k, h, hq // hkv, B), B)
        want = jensenshannon(pv_bf, brute_abar(q, k, h, hq // hkv, B))   # natural log
        assert rj.c_struct[h] == pytest.approx(want, rel=1e-9, abs=1e-12)
        assert rj.pattern[h] == (np.float32(want) >= np.float32(0.1))
    np.testing.assert_array_equal(rj.p_v, r.p_v)


def test_jsd_closed_forms():
    """Identical distributions give 0; disjoint supports give sqrt(ln 2)."""
    n, d, B = 512, 16, 128
    # Q = 0: A^ rows uniform over their visible keys; abar uniform over blocks
    q = torch.zeros(1, n, d, dtype=torch.bfloat16)
    _, k, _ = rand_qkv(n, 1, 1, d, seed=12)
    r = O.route(q, k, n, 1, 1, d, B)
    uni = np.full(n // B, 1.0 / (n // B))
    from scipy.spatial.distance import jensenshannon
    assert O.jsd(q, k, n, 1, 1, d, 0, r.p_v[0], B) == pytest.approx(jensenshannon(r.p_v[0], uni), rel=1e-12)
    # p_v all on block 0 while abar is (numerically) all on the last block
    pv = np.zeros(n // B)
    pv[0] = 1.0
    q2 = torch.zeros(1, n, d)
    q2[0, :, 0] = 30.0
    k2 = torch.zeros(1, n, d)
    k2[0, n - B:, 0] = 30.0
    got = O.jsd(q2.to(torch.bfloat16), k2.to(torch.bfloat16), n, 1, 1, d, 0, pv, B)
    assert got == pytest.approx(math.sqrt(math.log(2.0)), rel=1e-9)


def brute_vs_median(p, alpha, kmin):
    pf = p.astype(np.float32)
    nb = len(pf)
    mid = np.sort(pf[1:nb - 1])
    m = len(mid)
    med = mid[m // 2] if m % 2 else np.float32((mid[m // 2 - 1] + mid[m // 2]) * np.float32(0.5))
    assert med == np.float32(np.median(pf[1:nb - 1]))      # numpy's median, in float
    th = np.float32(alpha) * np.float32(med)
    cnt = int((pf > th).sum())
    kk = min(max(cnt, kmin), nb)
    order = sorted(range(nb), key=lambda j: (-pf[j], j))
    return sorted(order[:kk]), th


@pytest.mark.parametrize("seed", range(10))
def test_vs_select_median_floor(seed):
    rng = np.random.default_rng(1000 + seed)
    nb = int(rng.integers(4, 40))
    p = rng.random(nb) ** 3
    p[0] += 2.0
    p /= p.sum()
    for alpha in (0.5, 1.0, 2.0):
        for kmin in (1, 3, 8):
            s = O.vs_select(p, alpha, kmin, floor="median")
            want, th = brute_vs_median(p, alpha, kmin)
            assert s.sel.tolist() == want
            assert s.theta == th


def test_median_floor_resists_one_dominant_block():
    """Appendix H's clumpy-noise case: one large interior block lifts the
    mean floor above weaker signal blocks but not the median floor."""
    nb = 40
    p = np.full(nb, 0.005)
    p[0], p[-1] = 0.3, 0.1
    p[5] = 0.8                     # dominant interior block
    p[10:13] = 0.02                # weaker genuine signal
    p /= p.sum()
    mean_sel = set(O.vs_select(p, 1.0, 1).sel.tolist())
    med_sel = set(O.vs_select(p, 1.0, 1, floor="median").sel.tolist())
    assert mean_sel == {0, 5, 39}              # mu = 0.72 / 38 > 0.014
    assert med_sel == {0, 5, 10, 11, 12, 39}   # median = 0.0035


def test_gamma_rule_with_kmin_clip():
    rng = np.random.default_rng(5)
    p = rng.random(30) ** 4
    p[0] = 200.0                   # the sink alone reaches gamma: the cliff's collapse
    p /= p.sum()
    pure = O.gamma_select(p, 0.95)
    assert pure.tolist() == [0]
    clipped = O.gamma_select(p, 0.95, kmin_blocks=8)
    assert len(pure) < 8 and len(clipped) == 8
    order = sorted(range(30), key=lambda j: (-np.float32(p[j]), j))
    assert clipped.tolist() == sorted(order[:8])
    assert set(pure.tolist()) <= set(clipped.tolist())
