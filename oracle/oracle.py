"""ctypes wrapper of the CRISP CPU oracle (crisp_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test-suite, the smoke check and the
benchmark's CPU-baseline leg, never by the HIP library or its binding.

The wrapper only marshals arguments; every step of the method is computed in
the C file, in double precision, following the CRISP paper (arXiv 2609.01925).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "crisp_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# Paper defaults (Section 5, "Setup"; Section 3.2 for the anchor windows).
TAU_PROXY = 0.2
# FlexPrefill's JSD threshold (Alg. 5) is not given by the CRISP paper; 0.1
# is this implementation's default for the baseline router.
TAU_JSD = 0.1
GAMMA = 0.95
K_MIN_TOKENS = 1024
W_SINK = 128
W_LOCAL = 128


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP, no BLAS)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                        "-o", tmp, SRC, "-lm"], check=True)
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = C.CDLL(LIB)
        P = C.c_void_p
        i, f, i64 = C.c_int, C.c_float, C.c_int64
        L.orc_proxy_map.argtypes = [P, P, i, i, i, i, i, i, P]
        L.orc_block_scores.argtypes = [P, i, i, i, i, P, P, P]
        L.orc_route.argtypes = [P, P, i, i, i, i, i, f, i, i, P, P, P, P]
        L.orc_vs_select.argtypes = [P, i, f, i, P, P, P, P]
        L.orc_vs_select_median.argtypes = [P, i, f, i, P, P, P, P]
        L.orc_jsd.argtypes = [P, P, i, i, i, i, i, i, P, P]
        L.orc_gamma_select.argtypes = [P, i, f, i, P]
        L.orc_pe_map.argtypes = [P, P, i, i, i, i, i, i, P]
        L.orc_pe_select.argtypes = [P, i, f, P, P, P]
        L.orc_pe_select.restype = i64
        L.orc_expand.argtypes = [i, i, P, i, P, i, P, i64, P, P]
        L.orc_expand.restype = i64
        L.orc_attend.argtypes = [P, P, P, i, i, i, i, i, P, P, P, i, P]
        L.orc_threads.restype = i
        L.orc_attend_queries.argtypes = [P, P, P, i, i, i, i, i, P, P, P, i, P]
        _lib = L
    return _lib


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().orc_threads())


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _u16(x) -> np.ndarray:
    """Accept a uint16 array of bf16 bits or a CPU torch.bfloat16 tensor."""
    if isinstance(x, np.ndarray):
        assert x.dtype == np.uint16
        return np.ascontiguousarray(x)
    import torch
    assert x.dtype == torch.bfloat16 and x.device.type == "cpu"
    return x.contiguous().view(torch.int16).numpy().view(np.uint16)


def nblocks(n: int, B: int = 128) -> int:
    """N_b = ceil(n / B): the last block may be partial (Section 4.3)."""
    return (n + B - 1) // B


def proxy_map(q, k, n, hq, hkv, d, h, B=128) -> np.ndarray:
    """A^ of one query head, [min(B, n), n] float64 (Alg. 2)."""
    out = np.zeros((min(B, n), n), dtype=np.float64)
    rc = lib().orc_proxy_map(_p(_u16(q)), _p(_u16(k)), n, hq, hkv, d, B, h, _p(out))
    assert rc == 0, rc
    return out


def block_scores(ahat: np.ndarray, B=128, w_sink=W_SINK, w_local=W_LOCAL):
    """(p_v, p_s, C_struct) of one head from its A^ (Alg. 3, Eq. 2)."""
    ahat = np.ascontiguousarray(ahat, dtype=np.float64)
    n = ahat.shape[1]
    assert ahat.shape[0] == min(B, n)
    nb = nblocks(n, B)
    pv = np.zeros(nb)
    ps = np.zeros(nb)
    cs = np.zeros(1)
    rc = lib().orc_block_scores(_p(ahat), n, B, w_sink, w_local, _p(pv), _p(ps), _p(cs))
    assert rc == 0
    return pv, ps, float(cs[0])


@dataclass
class Route:
    p_v: np.ndarray        # [hq, Nb] float64
    p_s: np.ndarray        # [hq, Nb] float64
    c_struct: np.ndarray   # [hq] float64
    pattern: np.ndarray    # [hq] uint8, 1 = VS, 0 = PE


def route(q, k, n, hq, hkv, d=128, B=128, tau=TAU_PROXY, w_sink=W_SINK, w_local=W_LOCAL) -> Route:
    """PatSearch (Alg. 2) for every query head."""
    nb = nblocks(n, B)
    pv = np.zeros((hq, nb))
    ps = np.zeros((hq, nb))
    cs = np.zeros(hq)
    pat = np.zeros(hq, dtype=np.uint8)
    rc = lib().orc_route(_p(_u16(q)), _p(_u16(k)), n, hq, hkv, d, B, float(tau), w_sink, w_local,
                         _p(pv), _p(ps), _p(cs), _p(pat))
    assert rc == 0, rc
    return Route(pv, ps, cs, pat)


def jsd(q, k, n, hq, hkv, d, h, p_v, B=128) -> float:
    """FlexPrefill's D_JS of one head (Alg. 5) against its p_v."""
    pv = np.ascontiguousarray(p_v, dtype=np.float64)
    out = np.zeros(1)
    rc = lib().orc_jsd(_p(_u16(q)), _p(_u16(k)), n, hq, hkv, d, B, h, _p(pv), _p(out))
    assert rc == 0, rc
    return float(out[0])


def route_jsd(q, k, n, hq, hkv, d=128, B=128, tau_jsd=TAU_JSD, routed: Route | None = None) -> Route:
    """Alg. 5 for every head: p_v / p_s as route(); c_struct holds D_JS and
    the pattern is "VS iff D_JS >= tau_jsd" (in float)."""
    r = routed if routed is not None else route(q, k, n, hq, hkv, d, B)
    djs = np.array([jsd(q, k, n, hq, hkv, d, h, r.p_v[h], B) for h in range(hq)])
    pat = (djs.astype(np.float32) >= np.float32(tau_jsd)).astype(np.uint8)
    return Route(r.p_v, r.p_s, djs, pat)


@dataclass
class VSSel:
    sel: np.ndarray        # ascending int32 block indices
    theta: float           # alpha * mu, float
    kth: float             # k-th largest value (decisive when clipped)
    clipped: bool          # k_min clip was active


def vs_select(p: np.ndarray, alpha: float, kmin_blocks: int = K_MIN_TOKENS // 128,
              floor: str = "mean") -> VSSel:
    """Noise-floor selection in one direction: the sink-aware mean floor of
    Alg. 3 / Eq. 3-4, or the median floor of Appendix H (floor="median")."""
    p = np.ascontiguousarray(p, dtype=np.float64)
    nb = p.shape[0]
    sel = np.zeros(nb, dtype=np.int32)
    th = np.zeros(1, dtype=np.float32)
    kth = np.zeros(1, dtype=np.float32)
    cl = np.zeros(1, dtype=np.int32)
    fn = {"mean": lib().orc_vs_select, "median": lib().orc_vs_select_median}[floor]
    cnt = fn(_p(p), nb, float(alpha), kmin_blocks, _p(sel), _p(th), _p(kth), _p(cl))
    return VSSel(sel[:cnt].copy(), float(th[0]), float(kth[0]), bool(cl[0]))


def gamma_select(p: np.ndarray, gamma: float = GAMMA, kmin_blocks: int = 0) -> np.ndarray:
    """Cumulative-gamma selection in one direction (Alg. 6)."""
    p = np.ascontiguousarray(p, dtype=np.float64)
    nb = p.shape[0]
    sel = np.zeros(nb, dtype=np.int32)
    cnt = lib().orc_gamma_select(_p(p), nb, float(gamma), kmin_blocks, _p(sel))
    return sel[:cnt].copy()


def pe_map(q, k, n, hq, hkv, d, h, B=128) -> np.ndarray:
    """Normalised pooled map A-bar of one query head, [Nb, Nb] (Alg. 4)."""
    nb = nblocks(n, B)
    out = np.zeros((nb, nb), dtype=np.float64)
    rc = lib().orc_pe_map(_p(_u16(q)), _p(_u16(k)), n, hq, hkv, d, B, h, _p(out))
    assert rc == 0, rc
    return out


@dataclass
class PESel:
    mask: np.ndarray       # [Nb, Nb] uint8
    kstar: int
    vstar: float           # K*-th value (float)
    cum_before: float      # running sum of the first K*-1 entries


def pe_select(abar: np.ndarray, gamma: float = GAMMA) -> PESel:
    """gamma-cumsum over the flattened pooled map (Alg. 4)."""
    abar = np.ascontiguousarray(abar, dtype=np.float64)
    nb = abar.shape[0]
    mask = np.zeros((nb, nb), dtype=np.uint8)
    vs = np.zeros(1, dtype=np.float32)
    cb = np.zeros(1, dtype=np.float64)
    ks = lib().orc_pe_select(_p(abar), nb, float(gamma), _p(mask), _p(vs), _p(cb))
    return PESel(mask, int(ks), float(vs[0]), float(cb[0]))


def expand(nb: int, vs: bool, sv=None, ss=None, pe_mask=None, base: int = 0,
           col_idx: np.ndarray | None = None):
    """Block index lists of one head (Alg. 3 / Alg. 4 + {0, qb}).

    Returns (row_ptr[Nb+1] int32 absolute offsets, col_idx, count)."""
    sv = np.ascontiguousarray(sv if sv is not None else np.zeros(0), dtype=np.int32)
    ss = np.ascontiguousarray(ss if ss is not None else np.zeros(0), dtype=np.int32)
    pm = np.ascontiguousarray(pe_mask if pe_mask is not None else np.zeros((nb, nb)), dtype=np.uint8)
    row_ptr = np.zeros(nb + 1, dtype=np.int32)
    if col_idx is None:
        col_idx = np.zeros(base + nb * (nb + 1) // 2, dtype=np.int32)
    cnt = lib().orc_expand(nb, 1 if vs else 0, _p(sv), len(sv), _p(ss), len(ss), _p(pm), base,
                           _p(row_ptr), _p(col_idx))
    return row_ptr, col_idx, int(cnt)


def attend(q, k, v, n, hq, hkv, d, row_ptr, col_idx, rows, B=128) -> np.ndarray:
    """Eq. 1 on the given block lists for the listed (h*Nb+qb) query blocks.

    row_ptr: [hq, Nb+1] int32 absolute offsets; returns [len(rows), B, d] float64."""
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col_idx = np.ascontiguousarray(col_idx, dtype=np.int32)
    assert d <= 1024
    out = np.zeros((len(rows), B, d), dtype=np.float64)
    rc = lib().orc_attend(_p(_u16(q)), _p(_u16(k)), _p(_u16(v)), n, hq, hkv, d, B, _p(row_ptr),
                          _p(col_idx), _p(rows), len(rows), _p(out))
    assert rc == 0, rc
    return out


def attend_queries(q, k, v, n, hq, hkv, d, row_ptr, col_idx, qsel, B=128) -> np.ndarray:
    """Eq. 1 for individual queries; qsel is [m, 2] (head, position); returns [m, d]."""
    qsel = np.ascontiguousarray(qsel, dtype=np.int32).reshape(-1, 2)
    out = np.zeros((len(qsel), d), dtype=np.float64)
    rc = lib().orc_attend_queries(_p(_u16(q)), _p(_u16(k)), _p(_u16(v)), n, hq, hkv, d, B,
                                  _p(np.ascontiguousarray(row_ptr, dtype=np.int32)),
                                  _p(np.ascontiguousarray(col_idx, dtype=np.int32)), _p(qsel),
                                  len(qsel), _p(out))
    assert rc == 0, rc
    return out


# --------------------------------------------------------------------------
# Whole-path composition (Alg. 1): route -> select -> expand, every head.
# --------------------------------------------------------------------------
@dataclass
class Plan:
    route: Route
    vs_v: list             # per head VSSel or None
    vs_s: list
    pe: list               # per head PESel or None
    row_ptr: np.ndarray    # [hq, Nb+1] int32, absolute offsets
    col_idx: np.ndarray    # int32
    nb: int


def full_causal_lists(hq: int, nb: int):
    """row_ptr / col_idx with every causal block listed (dense)."""
    per = nb * (nb + 1) // 2
    row_ptr = np.zeros((hq, nb + 1), dtype=np.int32)
    col_idx = np.zeros(hq * per, dtype=np.int32)
    for h in range(hq):
        base = h * per
        pos = base
        for qb in range(nb):
            row_ptr[h, qb] = pos
            col_idx[pos:pos + qb + 1] = np.arange(qb + 1, dtype=np.int32)
            pos += qb + 1
        row_ptr[h, nb] = pos
    return row_ptr, col_idx


def plan(q, k, n, hq, hkv, d=128, B=128, alpha=1.0, tau=TAU_PROXY, gamma=GAMMA,
         kmin_tokens=K_MIN_TOKENS, heads=None, routed: Route | None = None,
         vs_rule: str = "mean", gamma_vs: float = GAMMA) -> Plan:
    """Alg. 1 up to the index set: routing, per-head selection and expansion.

    vs_rule picks the VS budget: "mean" (Alg. 3), "median" (Appendix H) or
    "gamma" (FlexPrefill's cumulative rule, Alg. 6, with the k_min clip).
    Head h's lists start at offset h*Nb*(Nb+1)/2 of col_idx (its worst case).
    `routed` reuses an earlier route() / route_jsd() result for the same inputs."""
    nb = nblocks(n, B)
    r = routed if routed is not None else route(q, k, n, hq, hkv, d, B, tau, B, B)
    per = nb * (nb + 1) // 2
    row_ptr = np.zeros((hq, nb + 1), dtype=np.int32)
    col_idx = np.zeros(hq * per, dtype=np.int32)
    vs_v, vs_s, pe = [None] * hq, [None] * hq, [None] * hq
    kmin = kmin_tokens // B
    for h in (range(hq) if heads is None else heads):
        if r.pattern[h]:
            if vs_rule == "gamma":
                sv = VSSel(gamma_select(r.p_v[h], gamma_vs, kmin), 0.0, 0.0, False)
                sls = VSSel(gamma_select(r.p_s[h], gamma_vs, kmin), 0.0, 0.0, False)
            else:
                sv = vs_select(r.p_v[h], alpha, kmin, vs_rule)
                sls = vs_select(r.p_s[h], alpha, kmin, vs_rule)
            vs_v[h], vs_s[h] = sv, sls
            rp, _, _ = expand(nb, True, sv.sel, sls.sel, base=h * per, col_idx=col_idx)
        else:
            ab = pe_map(q, k, n, hq, hkv, d, h, B)
            ps = pe_select(ab, gamma)
            pe[h] = ps
            rp, _, _ = expand(nb, False, pe_mask=ps.mask, base=h * per, col_idx=col_idx)
        row_ptr[h] = rp
    return Plan(r, vs_v, vs_s, pe, row_ptr, col_idx, nb)
