"""Seeded synthetic Q/K/V for the CRISP sparse-prefill hot path.

This module only draws inputs. It holds none of the method's arithmetic
(no proxy map, no routing, no selection, no attention): both the HIP path
and the CPU oracle consume what it returns, and neither is imported here.

What the inputs stand in for
----------------------------
The CRISP paper (arXiv 2609.01925) measures accuracy on long-context suites
and latency as attention-only time from 64k to 512k tokens on Llama-3.1-8B
(32 query / 8 KV heads, head_dim 128) and Qwen2.5-7B (28 / 4) (Section 5,
"Setup").  None of that data or any weights exist here, so the generator plants
the attention structure the paper describes instead: a three-class hierarchy
of architectural sinks, task-relevant signal and near-zero background on
concentrated heads (Section 4.1), vertical stripes and a local slash band
(Section 3), and diffuse heads whose mass is spread out (Appendix F).

Channel plan (head_dim = 128, logits are q.k / sqrt(128))
---------------------------------------------------------
* channels 0..15   one marker channel per sink token 0..15
* channel 16       shared marker of a 64-token distributed sink
* channels 17..32  one marker channel per candidate stripe key
* channels 33..64  local band: one channel per window of 1024 queries
* channel 65       per-key-block cluster value (diffuse heads)
* channels 66..127 i.i.d. noise, scaled so background logits are N(0, 1)

Keys carry unit markers; the query side carries (boost * sqrt(128)), so a
planted key's logit is raised by exactly ``boost`` (up to bf16 rounding, which
both consumers see identically).  Sink and stripe tokens carry no noise, so
their logit is the planted boost (plus the band term near the diagonal).

The band is exact and has no far field: the one-sided kernel 3*rho^(q-k) is
separable, rho^(q-e) * rho^(e-k), so band channel c holds rho^(e_c-k) on keys
k <= e_c (0 after) and the query side holds 3*rho^(q-e_c) for queries of its
window (e_c - 1023 .. e_c).  The 32 windows end at n-1 and tile backwards, so
every query has its band for n <= 32768 and the last 32768 queries do beyond
(the representative last block always does).  A random code would add
block-correlated cross-talk of std ~ 3/sqrt(32) at every distance, i.e. O(n)
spurious above-floor blocks; a rank-32 dot product cannot realise a noise-free
band on all queries of a longer sequence.

Boost conventions (a planted "scale s" is read as a logit boost (s/4)*ln n):
* sink group of w tokens: per-token boost ln(4n/w) (total weight 4n, i.e.
  scale 4 for w = 4),
* stripe (scale 3): boost 0.75*ln n,
* band: boost 3*rho^(q-k) with rho = exp(-1/256) for keys at or before q,
* diffuse heads: per-(KV head, key block) boost c ~ N(0, 0.5^2), zero on the
  first and last key block.

All randomness comes from numpy PCG64 seeded by
``SeedSequence(20260903 + 100*config_id + n_index)``.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

D = 128
BLOCK = 128
SINK_CH = list(range(0, 16))
DSINK_CH = 16
STRIPE_CH = list(range(17, 33))
BAND_CH = list(range(33, 65))
CLUSTER_CH = 65
NOISE_CH = list(range(66, 128))
N_NOISE = len(NOISE_CH)
RHO = math.exp(-1.0 / 256.0)
BAND_AMP = 3.0
BAND_WINDOW = 1024
SEED_BASE = 20260903

# head kinds
VS = "vs"                    # sink + band + stripes
DIFFUSE = "diffuse"          # noise + weak block clustering
CONC = "concentrated"        # token-0 sink holding a target mass (mass-cliff sweep)
DIST = "distributed"         # 64-token sink holding a target mass (mass-cliff sweep)


@dataclass
class HeadPlan:
    kind: str
    sink_width: int = 0          # VS heads: number of sink tokens (0..16)
    stripes: list = field(default_factory=list)  # indices into the KV head's candidates
    target_mass: float = 0.0     # CONC / DIST heads


@dataclass
class Spec:
    name: str
    config_id: int
    n: int
    hq: int
    hkv: int
    heads: list                  # HeadPlan per query head
    n_index: int = 0
    n_candidates: int = 16

    @property
    def group(self) -> int:
        return self.hq // self.hkv


@dataclass
class Inputs:
    q: "object"                  # torch.bfloat16 [hq, n, 128] (CPU)
    k: "object"                  # torch.bfloat16 [hkv, n, 128]
    v: "object"                  # torch.bfloat16 [hkv, n, 128]
    spec: Spec
    stripe_pos: np.ndarray       # int64 [hkv, n_candidates] key positions
    cluster: np.ndarray          # float64 [hkv, n_blocks] diffuse block boosts
    boosts: dict                 # per-head planted boosts, for logging


MASS_CLIFF_NS = (8192, 32768, 131072, 262144)


def config_spec(name: str, n: int | None = None) -> Spec:
    """The workloads, as concrete specs.

    c1  : 4096 tokens, 4 q / 1 kv, heads 0-1 VS (2 stripes), 2-3 diffuse
    c2  : Llama-3.1-8B layer shape at 32768 tokens, 24 VS + 8 diffuse
          (the last query head of each KV group is diffuse), 4..16 stripes
    c3  : Qwen2.5-7B layer shape (28 / 4) at 131072 tokens, 21 VS + 7 diffuse
          (one per KV group plus three more, seeded), sink width 1..16
    h128: config c2's head mix at 131072 tokens (the headline workload)
    c4  : Llama shape at 524288 tokens, 28 VS + 4 diffuse (heads 3,11,19,27)
    c5  : mass-cliff sweep, Llama shape, n in {8192, 32768, 131072, 262144};
          heads 0-15 concentrated token-0 sink (mass 0.96), heads 16-31 a
          64-token distributed sink (mass 0.45), 4 stripes each
    """
    ids = {"c1": 1, "c2": 2, "c3": 3, "c4": 4, "c5": 5, "h128": 6}
    if name not in ids:
        raise ValueError(f"unknown config {name!r}")
    cid = ids[name]
    plan_rng = None
    if name == "c1":
        n = n or 4096
        return _spec_vs_mix(name, cid, n, 4, 1, diffuse=[2, 3], stripes=(2, 2), n_index=0)
    if name in ("c2", "h128"):
        n = n or (32768 if name == "c2" else 131072)
        return _spec_vs_mix(name, cid, n, 32, 8, diffuse=[h for h in range(32) if h % 4 == 3],
                            stripes=(4, 16), n_index=0)
    if name == "c3":
        n = n or 131072
        return _spec_vs_mix(name, cid, n, 28, 4, diffuse="seeded", stripes=(4, 16), n_index=0,
                            sink_width=(1, 16))
    if name == "c4":
        n = n or 524288
        return _spec_vs_mix(name, cid, n, 32, 8, diffuse=[3, 11, 19, 27], stripes=(4, 16), n_index=0)
    # c5
    n = n or MASS_CLIFF_NS[0]
    if n not in MASS_CLIFF_NS:
        raise ValueError(f"c5 takes n in {MASS_CLIFF_NS}")
    n_index = MASS_CLIFF_NS.index(n)
    ss = np.random.SeedSequence(SEED_BASE + 100 * cid + n_index)
    plan_rng = np.random.Generator(np.random.PCG64(ss.spawn(1)[0]))
    heads = []
    for h in range(32):
        perm = plan_rng.permutation(16)[:4].tolist()
        if h < 16:
            heads.append(HeadPlan(CONC, sink_width=1, stripes=perm, target_mass=0.96))
        else:
            heads.append(HeadPlan(DIST, sink_width=64, stripes=perm, target_mass=0.45))
    del plan_rng
    return Spec(name, cid, n, 32, 8, heads, n_index=n_index)


def _spec_vs_mix(name, cid, n, hq, hkv, diffuse, stripes, n_index, sink_width=None):
    ss = np.random.SeedSequence(SEED_BASE + 100 * cid + n_index)
    rng = np.random.Generator(np.random.PCG64(ss.spawn(1)[0]))
    g = hq // hkv
    if diffuse == "seeded":
        # one diffuse head per KV group, then the rest chosen among the others
        per_group = [grp * g + int(rng.integers(g)) for grp in range(hkv)]
        others = [h for h in range(hq) if h not in per_group]
        extra = rng.choice(others, size=hq // 4 - len(per_group), replace=False).tolist()
        diffuse = sorted(per_group + [int(x) for x in extra])
    heads = []
    for h in range(hq):
        if h in diffuse:
            heads.append(HeadPlan(DIFFUSE))
            continue
        lo, hi = stripes
        ns = int(rng.integers(lo, hi + 1))
        perm = rng.permutation(16)[:ns].tolist()
        w = 4 if sink_width is None else int(rng.integers(sink_width[0], sink_width[1] + 1))
        heads.append(HeadPlan(VS, sink_width=w, stripes=perm))
    return Spec(name, cid, n, hq, hkv, heads, n_index=n_index)


def custom_spec(n: int, hq: int, hkv: int, kinds, *, stripes: int = 2, sink_width: int = 4,
                seed_id: int = 90, target_mass=None) -> Spec:
    """A small spec for tests: ``kinds`` lists one head kind per query head."""
    if len(kinds) != hq:
        raise ValueError("one kind per query head")
    ss = np.random.SeedSequence(SEED_BASE + 100 * seed_id)
    rng = np.random.Generator(np.random.PCG64(ss.spawn(1)[0]))
    heads = []
    for kind in kinds:
        perm = rng.permutation(16)[:stripes].tolist()
        if kind == VS:
            heads.append(HeadPlan(VS, sink_width=sink_width, stripes=perm))
        elif kind == DIFFUSE:
            heads.append(HeadPlan(DIFFUSE))
        elif kind == CONC:
            heads.append(HeadPlan(CONC, sink_width=1, stripes=perm,
                                  target_mass=0.96 if target_mass is None else target_mass))
        elif kind == DIST:
            heads.append(HeadPlan(DIST, sink_width=64, stripes=perm,
                                  target_mass=0.45 if target_mass is None else target_mass))
        else:
            raise ValueError(kind)
    return Spec(f"custom{seed_id}", seed_id, n, hq, hkv, heads)


def _band_windows(n):
    """(channel, first query, last query e_c) of each band window."""
    out = []
    for c in range(len(BAND_CH)):
        e = n - 1 - (len(BAND_CH) - 1 - c) * BAND_WINDOW
        if e < 0:
            continue
        out.append((c, max(0, e - BAND_WINDOW + 1), e))
    return out


def _band_boost(n, q):
    """Band logit boost of every key for the query at position q (keys > q: 0)."""
    k = np.arange(n, dtype=np.float64)
    b = BAND_AMP * RHO ** np.maximum(q - k, 0.0)
    covered = any(lo <= q <= e for _, lo, e in _band_windows(n))
    b[k > q] = 0.0
    return b if covered else np.zeros(n)


def _expected_rest_weight(n, noisy, extra_boost):
    """Expected sum of exp(logit) over the keys of the query at n-1 that the
    calibrated sink does not cover: noisy keys weigh e^(1/2) e^band, quiet
    keys e^band, and extra_boost adds planted boosts (stripes) per key."""
    b = _band_boost(n, n - 1) + extra_boost
    w = np.exp(b)
    w[noisy] *= math.exp(0.5)
    return float(w.sum())


def generate(spec: Spec, threads: int = 8) -> Inputs:
    """Draw Q, K, V (bf16, round-to-nearest-even) for ``spec``."""
    import torch

    n, hq, hkv, g = spec.n, spec.hq, spec.hkv, spec.group
    if n < 1:
        raise ValueError("n must be positive")
    nb = -(-n // BLOCK)                 # the last block may be partial
    ss = np.random.SeedSequence(SEED_BASE + 100 * spec.config_id + spec.n_index)
    kids = ss.spawn(2 + 3 * hkv + hq)
    plan = np.random.Generator(np.random.PCG64(kids[1]))

    # stripe candidate positions: distinct key blocks in [1, nb-3], random offset
    ncand = spec.n_candidates
    lo_b, hi_b = (1, nb - 3) if nb >= 4 else (0, nb - 1)
    stripe_pos = np.zeros((hkv, ncand), dtype=np.int64)
    cluster = np.zeros((hkv, nb), dtype=np.float64)
    for gi in range(hkv):
        span = hi_b - lo_b + 1
        if span >= ncand:
            blocks = lo_b + plan.choice(span, size=ncand, replace=False)
        else:
            blocks = lo_b + plan.integers(0, span, size=ncand)
        offs = plan.integers(0, BLOCK, size=ncand)
        stripe_pos[gi] = np.minimum(blocks * BLOCK + offs, n - 1)
        c = plan.normal(0.0, 0.5, size=nb)
        c[0] = 0.0
        c[nb - 1] = 0.0
        cluster[gi] = c

    q = torch.empty((hq, n, D), dtype=torch.bfloat16)
    k = torch.empty((hkv, n, D), dtype=torch.bfloat16)
    v = torch.empty((hkv, n, D), dtype=torch.bfloat16)
    k_noise_scale = math.sqrt(D / N_NOISE)
    quiet = 64 if any(h.kind == DIST for h in spec.heads) else 16
    # quiet keys: sink tokens and stripe candidates carry no noise
    noisy = np.ones((hkv, n), dtype=bool)
    noisy[:, :min(quiet, n)] = False
    for gi in range(hkv):
        noisy[gi, stripe_pos[gi]] = False
    windows = _band_windows(n)
    pos = np.arange(n, dtype=np.float64)
    band_k = np.zeros((n, len(BAND_CH)), dtype=np.float32)
    for c, lo, e in windows:
        band_k[:e + 1, c] = (RHO ** (e - pos[:e + 1])).astype(np.float32)

    def make_kv(gi):
        rk = np.random.Generator(np.random.PCG64(kids[2 + 3 * gi]))
        rv = np.random.Generator(np.random.PCG64(kids[3 + 3 * gi]))
        kk = np.zeros((n, D), dtype=np.float32)
        kk[:, NOISE_CH] = rk.standard_normal((n, N_NOISE), dtype=np.float32) * k_noise_scale
        kk[np.ix_(~noisy[gi], NOISE_CH)] = 0.0
        kk[:, BAND_CH] = band_k
        kk[:, CLUSTER_CH] = np.repeat(cluster[gi], BLOCK)[:n].astype(np.float32)
        for t in range(min(16, n)):
            kk[t, SINK_CH[t]] = 1.0
        kk[:min(64, n), DSINK_CH] = 1.0
        for j in range(ncand):
            kk[stripe_pos[gi, j], STRIPE_CH[j]] = 1.0
        k[gi] = torch.from_numpy(kk).to(torch.bfloat16)
        vv = rv.standard_normal((n, D), dtype=np.float32)
        v[gi] = torch.from_numpy(vv).to(torch.bfloat16)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(make_kv, range(hkv)))

    sq = math.sqrt(D)
    ln_n = math.log(n)
    boosts = {}
    band_q = np.zeros((n, len(BAND_CH)), dtype=np.float32)
    for c, lo, e in windows:
        band_q[lo:e + 1, c] = (BAND_AMP * sq * RHO ** (pos[lo:e + 1] - e)).astype(np.float32)

    def make_q(h):
        hp = spec.heads[h]
        gi = h // g
        rq = np.random.Generator(np.random.PCG64(kids[2 + 3 * hkv + h]))
        qq = np.zeros((n, D), dtype=np.float32)
        qq[:, NOISE_CH] = rq.standard_normal((n, N_NOISE), dtype=np.float32)
        info = {"kind": hp.kind}
        if hp.kind == DIFFUSE:
            qq[:, CLUSTER_CH] = sq
        else:
            qq[:, BAND_CH] = band_q
            z_stripe = 0.75 * ln_n
            for j in hp.stripes:
                qq[:, STRIPE_CH[j]] = z_stripe * sq
            info["stripe_boost"] = z_stripe
            info["stripes"] = [int(stripe_pos[gi, j]) for j in hp.stripes]
            if hp.kind == VS:
                w = hp.sink_width
                z = math.log(4.0 * n / w)
                for t in range(w):
                    qq[:, SINK_CH[t]] = z * sq
                info["sink_boost"] = z
                info["sink_width"] = w
            else:
                extra = np.zeros(n)
                for j in hp.stripes:
                    extra[stripe_pos[gi, j]] = z_stripe
                m = hp.target_mass
                if hp.kind == CONC:
                    rest = _expected_rest_weight(n, noisy[gi], extra)
                    rest -= math.exp(_band_boost(n, n - 1)[0])  # token 0 is the sink
                    z = math.log(m / (1.0 - m) * rest)
                    qq[:, SINK_CH[0]] = z * sq
                    info["sink_width"] = 1
                else:
                    bb = _band_boost(n, n - 1)
                    rest = _expected_rest_weight(n, noisy[gi], extra)
                    rest -= float(np.exp(bb[:min(64, n)]).sum())
                    z = math.log(m / (1.0 - m) * rest / 64.0)
                    qq[:, DSINK_CH] = z * sq
                    info["sink_width"] = 64
                info["sink_boost"] = z
        boosts[h] = info
        q[h] = torch.from_numpy(qq).to(torch.bfloat16)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(make_q, range(hq)))
    return Inputs(q, k, v, spec, stripe_pos, cluster, boosts)


def growing_scores(n: int, hq: int, hkv: int, beta: float, seed: int):
    """Q, K, V (CPU bfloat16, [heads, n, 128]) whose logits grow along the keys:
    q_i . k_j is close to f_i * beta * j, with f_i from 0.6 to 1.4 by the
    row's position i % 32 (so neighbouring rows of a 32-row group grow at
    different rates).  All queries and keys point along one random unit
    direction u (query norms 8 f_i, key norms beta * j / 8), plus i.i.d. noise
    of 0.01 per channel; V is i.i.d. N(0, 1).  A row's largest logit among
    keys 0 .. i is then near its last key, so a block-by-block pass over the
    keys sees the running maximum grow at every step."""
    import torch
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    f = 0.6 + 0.8 * (np.arange(n) % 32) / 31.0
    q = (8.0 * f)[None, :, None] * u[None, None, :] + 0.01 * rng.standard_normal((hq, n, D))
    j = np.arange(n, dtype=np.float64)
    k = (beta * j / 8.0)[None, :, None] * u[None, None, :] + 0.01 * rng.standard_normal((hkv, n, D))
    v = rng.standard_normal((hkv, n, D))
    return tuple(torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v))


def bf16_bits(t):
    """Raw bf16 bit patterns of a CPU bfloat16 tensor as a uint16 numpy array."""
    import torch
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
