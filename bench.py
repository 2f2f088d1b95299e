"""Benchmark of the CRISP sparse-prefill hot path on one MI355X.

One step = crisp_prefill (route -> select -> attend, every step of Alg. 1)
on the headline workload: one attention layer of Llama-3.1-8B head shape
(32 query / 8 KV heads, head_dim 128) at 131072 tokens, alpha = 1.0, with
24 vertical-slash and 8 diffuse heads (seeded synthetic inputs resident in
HBM before timing starts).  Dense causal attention with the same kernel is
timed on the same inputs for the speedup, and so is the FlexPrefill baseline
(JSD routing + cumulative gamma VS selection) that the paper compares with.
Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
    python bench.py --workload c4        # another configuration (context)
    python bench.py --crossover          # sparse/dense crossover sweep
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention-only prefill ms + speedup vs dense at 128k, Llama-8B head shape"
WORKLOAD = "h128"
B = 128
PAIR_FLOP = 4 * B * B * 128          # QK^T + PV of one 128x128 block pair, d = 128
# A diagonal (causal) pair is counted as the matrix work the attention kernel
# runs for it: its 64-key half above every query < 64 is skipped, so 3/4.
DIAG_FLOP = 3 * PAIR_FLOP // 4


def pair_flop(pairs, diag_pairs):
    """Matrix work of `pairs` computed block pairs, `diag_pairs` of them on
    the causal diagonal."""
    return (pairs - diag_pairs) * PAIR_FLOP + diag_pairs * DIAG_FLOP
PEAK_BF16_TFLOPS = 2500.0            # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
ATTEND_SRC = os.path.join(ROOT, "dynamic_sparse_attention_map_amd", "csrc", "attend.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attend_kernel_h128_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(path):
    """Hash of the kernel source with // comments and blank lines removed, so
    that an edit to the commentary alone keeps the counters valid."""
    lines = []
    for ln in open(path, encoding="utf-8").read().splitlines():
        code = ln.split("//", 1)[0].rstrip()
        if code:
            lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per attend launch from the committed PMC summary, or None if
    the kernel source changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    if rec.get("attend_hip_sha256_16") != source_hash(ATTEND_SRC):
        return None
    return rec.get("hbm_bytes_per_launch")


def stratified_blocks(nb, per_head, seed):
    """Query blocks of one head for a sample: 0, N_b - 1 and per_head - 2
    distinct uniform others (all blocks when N_b <= per_head)."""
    if nb <= per_head:
        return np.arange(nb)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, nb - 1), size=per_head - 2, replace=False)
    return np.sort(np.concatenate([[0, nb - 1], mid]))


def cpu_baseline(inp, plan_pairs, nb, hq, hkv, n, blocks_per_head=64, full_below=32768):
    """The oracle as it stands, on the host cores: routing + selection of every
    head in full; attention in full for n <= full_below, else on
    blocks_per_head stratified query blocks per head (0, N_b - 1 and uniform
    others), extrapolated by the ratio of total to sampled selected block
    pairs."""
    from oracle import oracle as O
    t0 = time.perf_counter()
    plan = O.plan(inp.q, inp.k, n, hq, hkv, alpha=1.0)
    t_rs = time.perf_counter() - t0
    full = n <= full_below
    if full:
        rows = np.arange(hq * nb, dtype=np.int32)
    else:
        rows = np.concatenate([h * nb + stratified_blocks(nb, blocks_per_head, seed=1000 + h)
                               for h in range(hq)]).astype(np.int32)
    lens = plan.row_ptr[:, 1:] - plan.row_ptr[:, :-1]
    sampled_pairs = int(lens.reshape(-1)[rows].sum())
    total_pairs = int(lens.sum())
    t0 = time.perf_counter()
    O.attend(inp.q, inp.k, inp.v, n, hq, hkv, 128, plan.row_ptr, plan.col_idx, rows)
    t_att = time.perf_counter() - t0
    att_est = t_att * total_pairs / max(sampled_pairs, 1)
    est_s = t_rs + att_est
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                             None)
    except OSError:
        pass
    if full:
        what = f"attention of all {hq * nb} query blocks ({total_pairs} block pairs, {t_att:.1f} s)"
    else:
        what = (f"attention of {blocks_per_head} stratified query blocks per head (qb = 0, N_b - 1 "
                f"and {blocks_per_head - 2} uniform; {len(rows)} blocks, {sampled_pairs} of "
                f"{total_pairs} block pairs, {t_att:.1f} s) extrapolated by block pairs to "
                f"{att_est:.1f} s")
    return {
        "value": round(est_s * 1e3, 1), "unit": "ms", "cores": O.threads(), "kind": "oracle",
        "cpu_model": cpu_model,
        "sample": f"route+select of all {hq} heads in full ({t_rs:.1f} s); {what}",
        "measured_s": round(t_rs + t_att, 1),
        "extrapolated_s": round(est_s, 1),
        "pairs_match_gpu": total_pairs == plan_pairs,
    }


def crossover(args):
    """Where sparse prefill starts to beat dense attention (the context-length
    gate of Sec. 5.3, "Short contexts"): crisp_prefill (route + select +
    attend) against crisp_attend_dense on the headline head mix at growing n.
    Prints one JSON line."""
    import torch
    from dynamic_sparse_attention_map_amd import crisp, synth

    rows = []
    for n in (1024, 2048, 4096, 8192, 16384, 32768, 65536):
        spec = synth.config_spec(WORKLOAD, n=n)
        inp = synth.generate(spec, threads=16)
        q, k, v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
        ws = crisp.alloc_workspace(n, spec.hq, spec.hkv)
        out = torch.empty_like(q)

        def timed(fn, reps=10):
            for _ in range(3):
                fn()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(reps)]
            for e0, e1 in ev:
                e0.record()
                fn()
                e1.record()
            torch.cuda.synchronize()
            return sorted(e0.elapsed_time(e1) for e0, e1 in ev)[reps // 2]

        sp = timed(lambda: crisp.crisp_prefill(q, k, v, args.alpha, ws, out))
        de = timed(lambda: crisp.crisp_attend_dense(q, k, v, ws, out))
        rows.append({"n": n, "prefill_ms": round(sp, 4), "dense_ms": round(de, 4),
                     "speedup": round(de / sp, 3)})
        log(f"crossover n={n}: prefill {sp:.4f} ms, dense {de:.4f} ms, x{de / sp:.2f}")
        del q, k, v, ws, out, inp
    faster = [r["n"] for r in rows if r["speedup"] > 1.0]
    print(json.dumps({"metric": "sparse_vs_dense_crossover", "workload": WORKLOAD + " head mix",
                      "alpha": args.alpha, "rows": rows,
                      "first_n_sparse_faster": faster[0] if faster else None}), flush=True)


def batch_bench(args):
    """Many short sequences: crisp_prefill_batch with a workspace for one
    attention launch over the whole batch ("fused") against the same call
    sequence by sequence ("serial") and against separate crisp_prefill calls,
    on the headline head mix.  Prints one JSON line."""
    import torch
    from dynamic_sparse_attention_map_amd import crisp, synth

    count, n = args.batch
    spec0 = synth.config_spec(WORKLOAD, n=n)
    hq, hkv = spec0.hq, spec0.hkv
    log(f"batch of {count} x {n} tokens, {hq}/{hkv} heads")
    qs, ks, vs = [], [], []
    for i in range(count):
        sp = synth.custom_spec(n, hq, hkv, [hp.kind for hp in spec0.heads], seed_id=900 + i)
        inp = synth.generate(sp, threads=16)
        qs.append(inp.q.cuda())
        ks.append(inp.k.cuda())
        vs.append(inp.v.cuda())
    outs = [torch.empty_like(x) for x in qs]
    ws_f = crisp.alloc_batch_workspace([n] * count, hq, hkv)
    ws_s = crisp.alloc_workspace(n, hq, hkv)

    def timed(fn, reps):
        for _ in range(2):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    reps = max(3, args.steps // 4)
    fused = timed(lambda: crisp.crisp_prefill_batch(qs, ks, vs, outs, args.alpha, ws_f), reps)
    serial = timed(lambda: crisp.crisp_prefill_batch(qs, ks, vs, outs, args.alpha, ws_s), reps)

    def singles():
        for q, k, v, o in zip(qs, ks, vs, outs):
            crisp.crisp_prefill(q, k, v, args.alpha, ws_s, o)
    single = timed(singles, reps)
    log(f"batch fused {fused:.3f} ms, serial {serial:.3f} ms, separate calls {single:.3f} ms")
    print(json.dumps({"metric": "varlen_batch_prefill_ms", "sequences": count, "seq_len": n,
                      "n_heads": hq, "n_kv_heads": hkv, "fused_ms": round(fused, 3),
                      "serial_ms": round(serial, 3), "separate_calls_ms": round(single, 3),
                      "fused_speedup_vs_separate": round(single / fused, 3)}), flush=True)


def gemm_ceiling():
    """The practical bf16 matrix-core rate of this part, for scale: the
    vendor library's GEMM (torch.matmul on rocBLAS / hipBLASLt) on random and
    on all-zero inputs (the part is power-limited, so data toggling moves the
    clock).  Prints one JSON line."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(0)
    rows = []
    for (m, n, k) in ((8192, 8192, 8192), (16384, 16384, 8192)):
        for kind in ("random", "zeros"):
            a = torch.randn(m, k, device="cuda", dtype=torch.bfloat16, generator=g)
            b = torch.randn(k, n, device="cuda", dtype=torch.bfloat16, generator=g)
            if kind == "zeros":
                a.zero_()
                b.zero_()
            c = a @ b
            torch.cuda.synchronize()
            reps = 30
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                c = a @ b
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            rows.append({"m": m, "n": n, "k": k, "inputs": kind, "ms": round(ms, 3),
                         "tflops": round(2.0 * m * n * k / (ms * 1e-3) / 1e12, 1)})
            log(f"gemm {m}x{n}x{k} {kind}: {ms:.3f} ms, {rows[-1]['tflops']} TFLOP/s")
            del a, b, c
    print(json.dumps({"metric": "bf16_gemm_ceiling", "library": "torch.matmul", "rows": rows,
                      "peak_tflops": PEAK_BF16_TFLOPS}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--alpha", type=float, default=1.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense timing")
    ap.add_argument("--no-flexprefill", action="store_true",
                    help="skip the FlexPrefill-baseline timing")
    ap.add_argument("--no-head-types", action="store_true",
                    help="skip the attention-per-head-type breakdown (profiled runs: it adds "
                         "attention calls on partial lists)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="end with a 1 GiB device-to-device copy (reference for counter runs)")
    ap.add_argument("--workload", default=WORKLOAD,
                    help="configuration to time (h128, the headline, by default; c1-c4 for context)")
    ap.add_argument("--seq-len", type=int, default=None,
                    help="the workload's head mix at another sequence length (context runs; "
                         "no traffic figure or CPU baseline)")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="only time the vendor bf16 GEMM (the practical matrix-core rate)")
    ap.add_argument("--crossover", action="store_true",
                    help="only sweep n for the sparse/dense crossover and print it")
    ap.add_argument("--batch", type=int, nargs=2, metavar=("COUNT", "SEQ_LEN"), default=None,
                    help="only time a batch of COUNT sequences of SEQ_LEN tokens (one attention "
                         "launch for the batch against sequence by sequence)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: every step is per query head and runs on a single "
              f"MI355X; the head-sharded multi-GPU layout is a design, not code "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    from dynamic_sparse_attention_map_amd import crisp, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    crisp.lib()
    if args.crossover:
        crossover(args)
        return
    if args.batch:
        batch_bench(args)
        return
    if args.gemm_ceiling:
        gemm_ceiling()
        return
    workload = args.workload
    spec = synth.config_spec(workload, n=args.seq_len) if args.seq_len else synth.config_spec(workload)
    full_size = workload == WORKLOAD and args.seq_len is None
    n, hq, hkv = spec.n, spec.hq, spec.hkv
    nb = -(-n // B)
    log(f"generating {workload}: n={n} hq={hq} hkv={hkv}")
    t0 = time.perf_counter()
    inp = synth.generate(spec, threads=16)
    log(f"generated in {time.perf_counter() - t0:.1f} s")
    q, k, v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
    ws = crisp.alloc_workspace(n, hq, hkv)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    # computed block pairs of this input (same kernels as the prefill)
    ws2 = crisp.alloc_workspace(n, hq, hkv)
    pattern = torch.zeros(hq, dtype=torch.uint8, device="cuda")
    cs = torch.zeros(hq, device="cuda")
    pv = torch.zeros(hq, nb, device="cuda")
    ps = torch.zeros(hq, nb, device="cuda")
    crisp.crisp_route(q, k, ws2, pattern, cs, pv, ps)
    _, cap = crisp.crisp_workspace_size(n, hq, hkv)
    sel_v = torch.zeros(hq, nb, dtype=torch.int32, device="cuda")
    sel_s = torch.zeros_like(sel_v)
    counts = torch.zeros(hq, 3, dtype=torch.int32, device="cuda")
    row_ptr = torch.zeros(hq, nb + 1, dtype=torch.int32, device="cuda")
    col_idx = torch.zeros(cap, dtype=torch.int32, device="cuda")
    crisp.crisp_select(q, k, pattern, pv, ps, args.alpha, ws2, sel_v, sel_s, counts, row_ptr, col_idx)
    torch.cuda.synchronize()
    rp = row_ptr.cpu().numpy()
    pairs = int((rp[:, nb] - rp[:, 0]).sum())
    dense_pairs = hq * nb * (nb + 1) // 2
    pattern_h = pattern.cpu().numpy()
    row_pairs = rp[:, nb] - rp[:, 0]
    del ws2

    def events(m):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(m)]
        for e in evs:
            e.record(stream)       # materialise the HIP event handles
        return evs

    # ---- sparse prefill: the step ----
    for _ in range(args.warmup):
        crisp.crisp_prefill(q, k, v, args.alpha, ws, out)
    step_ev = [events(5) for _ in range(args.steps)]
    t_start, t_end = events(2)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(args.steps):
        crisp.crisp_set_stage_events(step_ev[s])
        crisp.crisp_prefill(q, k, v, args.alpha, ws, out)
    crisp.crisp_set_stage_events(None)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    stage = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in step_ev])
    per_step = np.array([e[0].elapsed_time(e[4]) for e in step_ev])
    st = stage.mean(axis=0)
    route_ms, select_ms, vt_ms, attend_ms = [float(x) for x in st]
    log(f"prefill {ms_step:.3f} ms/step (wall {wall / args.steps * 1e3:.3f}); stages "
        f"route {route_ms:.3f} select {select_ms:.3f} v-relayout {vt_ms:.3f} attend {attend_ms:.3f}")

    # ---- FlexPrefill baseline (JSD routing + cumulative gamma VS rule, the
    # paper's comparison system) on the same inputs and kernels ----
    fp = None
    if not args.no_flexprefill:
        fopts = crisp.flexprefill_opts()
        out_f = torch.empty_like(q)
        ws_f = crisp.alloc_workspace(n, hq, hkv)
        pat_f = torch.zeros(hq, dtype=torch.uint8, device="cuda")
        crisp.crisp_route(q, k, ws_f, pat_f, cs, pv, ps, opts=fopts)
        rp_f = torch.zeros(hq, nb + 1, dtype=torch.int32, device="cuda")
        ci_f = torch.zeros(cap, dtype=torch.int32, device="cuda")
        crisp.crisp_select(q, k, pat_f, pv, ps, args.alpha, ws_f, sel_v, sel_s, counts, rp_f, ci_f,
                           opts=fopts)
        torch.cuda.synchronize()
        rpf = rp_f.cpu().numpy()
        fp_pairs = int((rpf[:, nb] - rpf[:, 0]).sum())
        fp_vs = int(pat_f.sum().item())
        del ci_f
        for _ in range(min(args.warmup, 2)):
            crisp.crisp_prefill(q, k, v, args.alpha, ws_f, out_f, opts=fopts)
        fsteps = max(3, args.steps // 2)
        f_ev = [events(5) for _ in range(fsteps)]
        f0, f1 = events(2)
        torch.cuda.synchronize()
        f0.record(stream)
        for s in range(fsteps):
            crisp.crisp_set_stage_events(f_ev[s])
            crisp.crisp_prefill(q, k, v, args.alpha, ws_f, out_f, opts=fopts)
        crisp.crisp_set_stage_events(None)
        f1.record(stream)
        torch.cuda.synchronize()
        fp_ms = f0.elapsed_time(f1) / fsteps
        fst = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in f_ev]).mean(axis=0)
        fp = {"ms": round(fp_ms, 3), "computed_pairs": fp_pairs, "vs_heads": fp_vs,
              "stages_ms": {"route": round(float(fst[0]), 3), "select": round(float(fst[1]), 3),
                            "attend": round(float(fst[2] + fst[3]), 3)},
              "crisp_speedup": round(fp_ms / ms_step, 3),
              "rule": "JSD routing (tau 0.1) + cumulative gamma = 0.95 VS rule with k_min 8 blocks; "
                      "PE path as CRISP"}
        log(f"flexprefill {fp_ms:.3f} ms/step, {fp_pairs} pairs, {fp_vs} VS heads")
        del out_f, ws_f

    # ---- dense baseline: same kernel, every causal block ----
    dense_ms = dense_attend_ms = None
    if not args.no_dense:
        out_d = torch.empty_like(q)
        for _ in range(min(args.warmup, 2)):
            crisp.crisp_attend_dense(q, k, v, ws, out_d)
        dsteps = max(3, args.steps // 2)
        d_ev = [events(5) for _ in range(dsteps)]
        d0, d1 = events(2)
        torch.cuda.synchronize()
        d0.record(stream)
        for s in range(dsteps):
            crisp.crisp_set_stage_events(d_ev[s])
            crisp.crisp_attend_dense(q, k, v, ws, out_d)
        crisp.crisp_set_stage_events(None)
        d1.record(stream)
        torch.cuda.synchronize()
        dense_ms = d0.elapsed_time(d1) / dsteps
        dense_attend_ms = float(np.mean([e[3].elapsed_time(e[4]) for e in d_ev]))
        log(f"dense {dense_ms:.3f} ms (attention kernel {dense_attend_ms:.3f} ms)")
        del out_d

    # ---- attention time per head type: the same lists with the other
    # type's rows emptied.  Empty rows still cost their work items' set-up,
    # so the time of a run with every row empty, scaled by the share of
    # emptied heads, is also taken off ("net") ----
    by_type = {}
    out_t = torch.empty_like(q)

    def attend_ms_on(keep):
        rp_t = row_ptr.clone()
        drop = torch.from_numpy(np.nonzero(~keep)[0]).cuda()
        if drop.numel():
            rp_t[drop] = rp_t[drop, :1].expand(-1, nb + 1)
        crisp.crisp_attend(q, k, v, rp_t, col_idx, ws, out_t)
        t_ev = [events(5) for _ in range(3)]
        for e in t_ev:
            crisp.crisp_set_stage_events(e)
            crisp.crisp_attend(q, k, v, rp_t, col_idx, ws, out_t, check_lists=False)
        crisp.crisp_set_stage_events(None)
        torch.cuda.synchronize()
        return float(np.median([e[3].elapsed_time(e[4]) for e in t_ev]))

    empty_ms = None if args.no_head_types else attend_ms_on(np.zeros(hq, dtype=bool))
    for name, sel in (("vertical_slash", pattern_h == 1), ("pooled_estimation", pattern_h == 0)):
        if args.no_head_types or not sel.any():
            continue
        t_ms = attend_ms_on(sel)
        net_ms = t_ms - empty_ms * float((~sel).sum()) / hq
        t_pairs = int(row_pairs[sel].sum())
        by_type[name] = {"heads": int(sel.sum()), "computed_pairs": t_pairs,
                         "pairs_per_head": round(t_pairs / int(sel.sum()), 1),
                         "attend_ms": round(t_ms, 3), "attend_ms_net": round(net_ms, 3),
                         "attend_tflops_net": round(pair_flop(t_pairs, int(sel.sum()) * nb)
                                                    / (net_ms * 1e-3) / 1e12, 1)}
        log(f"attention on {name} heads only: {t_ms:.3f} ms ({net_ms:.3f} net), {t_pairs} pairs")
    if empty_ms is not None:
        by_type["all_rows_empty_ms"] = round(empty_ms, 3)
    del out_t, col_idx

    # every list holds its diagonal block qb (rows always contain 0 and qb)
    achieved = pair_flop(pairs, hq * nb) / (attend_ms * 1e-3) / 1e12
    traffic = measured_traffic() if full_size else None
    roofline = {
        "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
        "kernel": "attend_kernel", "kernel_ms": round(attend_ms, 3),
        "work": f"{pairs} computed 128x128 block pairs x {PAIR_FLOP} FLOP, the {hq * nb} "
                f"diagonal ones x {DIAG_FLOP} (the kernel skips the quarter of a causal "
                f"diagonal pair that lies above every query)",
    }
    causal_flop = 2.0 * 2 * 128 * hq * n * (n + 1) / 2
    res = {
        "metric": METRIC, "value": round(ms_step, 3), "unit": "ms", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{workload}: one attention layer, {hq} query / {hkv} KV heads, "
                               f"head_dim 128, {n} tokens, alpha {args.alpha:g}, "
                               f"{sum(1 for hp in spec.heads if hp.kind != synth.DIFFUSE)} "
                               f"vertical-slash + "
                               f"{sum(1 for hp in spec.heads if hp.kind == synth.DIFFUSE)} diffuse heads",
                   "seq_len": n, "n_heads": hq, "n_kv_heads": hkv, "head_dim": 128,
                   "block": B, "alpha": args.alpha, "global_batch": 1, "parallelism": "none"},
        "speedup_vs_dense": round(dense_ms / ms_step, 3) if dense_ms else None,
        "dense_ms": round(dense_ms, 3) if dense_ms else None,
        "dense_attend_tflops": round(pair_flop(dense_pairs, hq * nb) / (dense_attend_ms * 1e-3) / 1e12, 1)
        if dense_attend_ms else None,
        "stages_ms": {"route": round(route_ms, 3), "select": round(select_ms, 3),
                      "v_relayout": round(vt_ms, 3), "attend": round(attend_ms, 3)},
        "route_select_frac": round((route_ms + select_ms) / ms_step, 4),
        "step_ms": {"p10": round(float(np.percentile(per_step, 10)), 3),
                    "median": round(float(np.median(per_step)), 3),
                    "p90": round(float(np.percentile(per_step, 90)), 3)},
        "per_head_type": by_type,
        "effective_tflops": round(causal_flop / (ms_step * 1e-3) / 1e12, 1),
        "computed_pairs": pairs, "dense_pairs": dense_pairs,
        "density": round(pairs / dense_pairs, 4),
        "vs_heads": int(pattern_h.sum()), "pe_heads": int(hq - pattern_h.sum()),
        "roofline": roofline,
        "flexprefill_baseline": fp,
    }
    if args.calibrate_copy:
        src = torch.ones(1 << 29, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)             # reads and writes exactly 1 GiB
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu and args.seq_len is None:
        log("timing the CPU oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline(inp, pairs, nb, hq, hkv, n)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
