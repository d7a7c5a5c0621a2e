#!/usr/bin/env python3
"""Mixed-resolution decode benchmark on one MI355X.

One step = one decode step of one attention layer for the whole batch: route
(per-head routing + compaction) then mixed-resolution attention (full-res +
size-corrected summaries + expanded spans rebuilt from their factors) and the
log-sum-exp combine.  Default workload: Llama-3-8B-shaped layer (32 query
heads, 8 KV heads, head dim 128, bf16), 128K context, batch 4, device-resident
factors, 5% union expansion per step, ranks 16..64 (synthetic seeded inputs;
the pages' own evaluation sets are not available).  Inputs are resident in HBM
before timing; the cache is rotated over >= 2 copies so the 256 MB last-level
cache cannot hold the working set.

Timed region: exactly --steps steps, replayed from captured HIP graphs of at
most --graph-steps steps each (the last graph takes the remainder), after
--warmup eager steps and one untimed replay of every graph.  Per-kernel
durations come from HIP events recorded around each library kernel on its
launch stream, in an eager pass over exactly the timed steps (same caches,
queries and order) just before the timed replays.

Prints ONE JSON line on stdout (``--sweep`` adds one line per further sweep
point and workload); progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "memory_counters.json")
COUNTER_SOURCES = ["hierarchical_kv_cache_sekv_amd/csrc/sekv_kernels.hip",
                   "hierarchical_kv_cache_sekv_amd/csrc/sekv_internal.h",
                   "hierarchical_kv_cache_sekv_amd/csrc/sekv_host.cpp"]
# library kernels named in rocprofv3 output -> short names
KERNELS = ("attend_fused_kernel", "attend_full_kernel", "attend_expanded_kernel", "attend_expanded_wide_kernel",
           "route_kernel", "fold_query_kernel", "combine_kernel", "seal_build_kernel", "seal_compact_kernel",
           "build_spans_kernel", "build_full_kernel", "cache_fill_kernel")


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


# reading variants (each swaps one reading the pages leave open)
VARIANTS = {"rank-cap-half": dict(rank_cap="half"), "separate-bases": dict(basis="separate"),
            "folded-route": dict(route_keys="folded"), "boundary-q97": dict(boundary_quantile=0.97)}


# ------------------------------------------------------------------ schedule
def graph_chunks(start: int, steps: int, per_graph: int):
    """Consecutive chunks (first global step, n steps) covering global steps
    [start, start + steps), each at most ``per_graph`` long; only the last one
    may be shorter.  Every step is covered exactly once."""
    if steps < 0 or per_graph < 1:
        raise ValueError("steps must be >= 0 and per_graph >= 1")
    out, i = [], 0
    while i < steps:
        n = min(per_graph, steps - i)
        out.append((start + i, n))
        i += n
    return out


def graph_key(first: int, n: int, period: int):
    """Graphs are shared by chunks whose steps use the same cache copies and
    queries: step s uses copy s % ncopy and query s % Q, which repeat with
    ``period`` = lcm(ncopy, Q)."""
    return (first % period, n)


# ------------------------------------------------------------------ bytes
def algorithmic_bytes(w, plan, counts, lists, e):
    """Bytes the method must move per step (the dense work it avoids excluded).

    Per sequence: queries and outputs Hq*d*(e+4); per KV head the full-res K/V
    e*2d*n_full, the summaries kbar, vbar and rho e*3d*n_seg, and for each
    listed span its factors e*r*(L+2d) + 8r (sigma and gate in float32).
    Returns per-kernel shares {route: q + rho, attend: q + full-res K/V +
    kbar, vbar + factors, full: q + full-res K/V (the part of attend that
    decode_step overlaps with the route)} and the step total."""
    import numpy as np
    d, Hq, Hkv = w.head_dim, w.n_q_heads, w.n_kv_heads
    route = attend = total = fac_all = full = 0
    for b in range(w.batch):
        nf, ns = int(plan.n_full[b]), int(plan.n_seg[b])
        so = plan.seg_off[b]
        L = (so[1:ns + 1] - so[:ns] - 1).astype(np.int64)
        r = plan.rank[b, :ns].astype(np.int64)
        fac = 0
        for kv in range(Hkv):
            c = int(counts[b, kv])
            idx = lists[b, kv, :c]
            fac += int((e * r[idx] * (L[idx] + 2 * d) + 8 * r[idx]).sum())
        qb = Hq * d * e
        route += qb + Hkv * ns * d * e
        attend += qb + Hkv * e * 2 * d * (nf + ns) + fac
        full += qb + Hkv * e * 2 * d * nf
        total += Hq * d * (e + 4) + Hkv * (e * 2 * d * nf + e * 3 * d * ns) + fac
        fac_all += fac
    return {"route": route, "attend": attend, "total": total, "factors": fac_all, "full": full}


def resident_bytes(w, plan, cache):
    """GPU-resident bytes of the span cache (factor pools in HBM or in host
    memory) against the dense K/V cache of the same context."""
    e = 2 if w.dtype == "bf16" else 4
    dense = w.batch * w.n_kv_heads * w.n_ctx * w.head_dim * 2 * e
    pools = cache.fac.numel() * cache.fac.element_size() + cache.sg.numel() * 4
    dev = cache.device_bytes()
    on_dev = dev if not w.factors_on_host else dev + pools
    gpu_only = on_dev - pools
    return {"dense_kv_bytes": dense, "resident_bytes_factors_on_device": on_dev,
            "resident_bytes_factors_on_host": gpu_only,
            "resident_ratio_factors_on_device": on_dev / dense, "resident_ratio_factors_on_host": gpu_only / dense}


# ------------------------------------------------------------------ memory counters
def measured_traffic(kernel):
    """HBM bytes per launch of ``kernel`` from the committed FETCH_SIZE /
    WRITE_SIZE counter runs (scaled by a 1 GiB copy's counts), or None when a
    source they depend on (the kernels, launch constants and host plan) has
    changed since they were taken: the record holds the SHA-256 of those
    sources' contents, concatenated in the listed order."""
    import hashlib
    try:
        rec = json.load(open(COUNTERS))
        h = hashlib.sha256()
        for path in rec["sources"]:
            h.update(open(os.path.join(ROOT, path), "rb").read())
    except (OSError, ValueError, KeyError):
        return None
    if h.hexdigest() != rec.get("sources_sha256") or kernel not in rec.get("kernels", {}):
        return None
    return rec["kernels"][kernel]["hbm_bytes_per_launch"]


def summarize_counters(ev_dir, workload):
    """Turn four rocprofv3 --pmc runs (subdirectories cal_FETCH_SIZE,
    bench_FETCH_SIZE, cal_WRITE_SIZE, bench_WRITE_SIZE of ``ev_dir``, CSV
    output) into the counter record bench.py reads: per library kernel the mean
    KiB per dispatch, scaled to bytes by what the same counter reads for the
    1 GiB device copy of ``--copy-calibration``."""
    import csv
    import glob
    import hashlib
    from collections import defaultdict

    def load(sub):
        files = glob.glob(os.path.join(ev_dir, sub, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {os.path.join(ev_dir, sub)}")
        per = defaultdict(list)
        for f in files:
            for row in csv.DictReader(open(f)):
                per[row["Kernel_Name"]].append(float(row["Counter_Value"]))
        return per

    def short(name):
        for k in KERNELS:
            if k in name:
                return k
        return None

    res = {}
    for cnt in ("FETCH_SIZE", "WRITE_SIZE"):
        cal = load("cal_" + cnt)
        calk = max(v for n, vs in cal.items() if "copyBuffer" in n for v in vs)
        scale = (1 << 30) / (calk * 1024.0)
        agg = defaultdict(list)
        for n, vs in load("bench_" + cnt).items():
            k = short(n)
            if k:
                agg[k] += vs
        res[cnt] = (calk, scale, {k: (sum(v) / len(v), len(v)) for k, v in agg.items()})
    h = hashlib.sha256()
    for p in COUNTER_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    fcal, fs, fk = res["FETCH_SIZE"]
    wcal, ws, wk = res["WRITE_SIZE"]
    out = {"sources": COUNTER_SOURCES, "sources_sha256": h.hexdigest(), "workload": workload,
           "fetch_scale": round(fs, 5), "write_scale": round(ws, 5),
           "calibration_kib": {"FETCH_SIZE": fcal, "WRITE_SIZE": wcal}, "kernels": {}}
    for k, (f, nf) in fk.items():
        wv, nw = wk.get(k, (0.0, 0))
        out["kernels"][k] = {"fetch_kib": round(f, 1), "write_kib": round(wv, 1), "dispatches": [nf, nw],
                             "hbm_bytes_per_launch": int(round(f * 1024 * fs + wv * 1024 * ws))}
    return out


# ------------------------------------------------------------------ CPU oracle baseline
class OraclePool:
    """Worker processes that time the CPU oracle on the same workload.

    Created with fork BEFORE this process touches the GPU, so the workers are
    plain numpy processes that inherit the seeded inputs without copying.  Each
    worker takes every n-th (sequence, KV head) group, builds the oracle's
    cache for its groups (untimed), waits for the others, then runs decode
    steps (canonical route scores + expansion decisions + mixed-resolution
    attention) of its groups for a fixed wall time, one BLAS thread each."""

    def __init__(self, w, x, n_workers):
        import multiprocessing as mp
        self.w = w
        self.n_groups = w.batch * w.n_kv_heads
        self.n = max(1, min(n_workers, self.n_groups))
        mpc = mp.get_context("fork")
        self.tasks = [mpc.SimpleQueue() for _ in range(self.n)]
        self.results = mpc.SimpleQueue()
        self.barrier = mpc.Barrier(self.n)
        self.procs = [mpc.Process(target=_oracle_worker, args=(i, self.n, w, x, self.tasks[i], self.results,
                                                               self.barrier), daemon=True)
                      for i in range(self.n)]
        for p in self.procs:
            p.start()

    def run(self, theta, budget_s):
        for q in self.tasks:
            q.put((theta, budget_s))
        res = [self.results.get() for _ in range(self.n)]
        for p in self.procs:
            p.join(timeout=30)
        return res

    def close(self):
        for q, p in zip(self.tasks, self.procs):
            if p.is_alive():
                q.put(None)
        for p in self.procs:
            p.join(timeout=10)


def _oracle_worker(i, n, w, x, tasks, results, barrier):
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle as O
    msg = tasks.get()
    if msg is None:
        return
    theta, budget_s = msg
    G = w.group
    groups = [(g // w.n_kv_heads, g % w.n_kv_heads) for g in range(w.batch * w.n_kv_heads) if g % n == i]
    with threadpool_limits(1):
        t0 = time.perf_counter()
        caches = {}
        for b, kv in groups:
            caches[(b, kv)] = O.build_cache(
                x.k[b:b + 1, kv:kv + 1], x.v[b:b + 1, kv:kv + 1], x.surprisal[b:b + 1], x.boundary_thr[b:b + 1],
                x.route_proj[kv:kv + 1], x.rank_req[b:b + 1], x.gate[b:b + 1, kv:kv + 1],
                n_sink=w.n_sink, n_recent=w.n_recent, lo=w.min_span, hi=w.max_span, dtype=w.dtype)
        build_s = time.perf_counter() - t0
        barrier.wait()
        rounds = 0
        t1 = time.perf_counter()
        while True:
            st = rounds % x.q.shape[0]
            for b, kv in groups:
                c = caches[(b, kv)]
                hs = slice(kv * G, (kv + 1) * G)
                q = x.q[st, b, hs]
                dec = O.route_scores(q, c.rho[0][0]) > theta[b, hs][:, None]
                O.mixed_attention(c, 0, q, dec, G)
            rounds += 1
            el = time.perf_counter() - t1
            if el >= budget_s:
                break
    results.put((i, len(groups), rounds, el, build_s))


def oracle_baseline(pool, theta, budget_s):
    res = pool.run(theta, budget_s)
    rate = sum(ng * r / el for _, ng, r, el, _ in res) / pool.n_groups      # full steps per second
    gsteps = sum(ng * r for _, ng, r, _, _ in res)
    w = pool.w
    return {"value": rate, "unit": "steps/s", "cores": pool.n, "kind": "oracle",
            "sample": (f"all {pool.n_groups} (sequence, KV head) groups of {w.name}, split over {pool.n} worker "
                       f"processes (1 BLAS thread each); {gsteps} group decode steps (canonical fp32 route scores, "
                       f"decisions, fp64 mixed attention) in {budget_s:.0f} s of wall time per worker; "
                       f"steps/s = sum over workers of group-steps/s / {pool.n_groups}"),
            "blas_threads_per_process": 1,
            "eff_ctx_tokens_per_s": rate * w.batch * w.n_ctx}


# ------------------------------------------------------------------ device-resident measurement
def calibrate(B, w, plan, cache, x, frac, Q):
    """Per-head thresholds from the routing scores of the query set (torch
    GEMM on the device; the decisions themselves are taken by the route
    kernel)."""
    import numpy as np
    import torch
    from hierarchical_kv_cache_sekv_amd import synth
    G = w.group
    qf = torch.from_numpy(x.q[:Q]).cuda()
    rho = cache.rho.float()
    theta = np.empty((w.batch, w.n_q_heads), np.float32)
    for b in range(w.batch):
        ns = int(plan.n_seg[b])
        if frac is None:
            theta[b] = -np.inf
            continue
        z = torch.empty((Q, w.n_q_heads, ns), device="cuda")
        for kv in range(w.n_kv_heads):
            z[:, kv * G:(kv + 1) * G] = qf[:, b, kv * G:(kv + 1) * G] @ rho[b, kv, :ns].T
        theta[b] = synth.calibrate_theta(z.cpu().numpy(), float(frac[b]), G)
    return theta


def measure_device(w, x, fracs, args, label, full_rank=False):
    """Build the library cache for workload ``w`` and time graph-replayed
    decode steps at every expansion fraction in ``fracs`` (None = every span
    expanded).  Returns one record per fraction."""
    import numpy as np
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B

    e = 2 if w.dtype == "bf16" else 4
    Q = min(args.queries, x.q.shape[0])
    ctx = B.Context(0)
    ctx.set_split(args.split)
    cfg = B.make_config(w, False)
    plan = B.plan_spans(cfg, x.surprisal, x.boundary_thr, x.rank_req)
    cache = B.SpanCache(cfg, plan)
    t0 = time.time()
    kd = torch.from_numpy(x.k).to(cache.elem).cuda()
    vd = torch.from_numpy(x.v).to(cache.elem).cuda()
    B.build_spans(ctx, cache, kd, vd, x.surprisal, x.route_proj, x.gate)
    del kd, vd
    torch.cuda.synchronize()
    build_s = time.time() - t0
    log(f"{label}: library build (plan + summaries + rank-r factors) in {build_s:.2f}s; "
        f"n_seg={plan.n_seg.tolist()}")
    qd = torch.from_numpy(x.q[:Q]).to(cache.elem).cuda().contiguous()
    resident = cache.device_bytes()
    ncopy = args.copies or max(2, math.ceil((1 << 30) / resident))
    caches = [cache] + [cache.clone() for _ in range(ncopy - 1)]
    structs = [c.struct() for c in caches]
    outs = [B.RouteOut(cfg, cache.seg_cap) for _ in range(ncopy)]
    rws = B.route_workspace(cache)
    dws = B.DecodeWorkspace(cache, ctx=ctx)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    log(f"{label}: {ncopy} cache copies of {resident / 2**20:.0f} MiB each resident in HBM")
    stream = torch.cuda.Stream()
    period = math.lcm(ncopy, Q)
    gs = max(1, args.graph_steps)
    nseg_tot = sum(int(plan.n_seg[b]) for b in range(w.batch)) * w.n_kv_heads
    recs = []
    for frac in fracs:
        target = None if frac is None else ([float(frac)] * w.batch if np.isscalar(frac) else [float(f) for f in frac])
        theta = calibrate(B, w, plan, cache, x, target, Q)
        theta_d = torch.from_numpy(theta).cuda()

        def step(i, theta_d=theta_d):
            c = i % ncopy
            qs = qd[i % Q]
            if args.overlap:
                B.decode_step(ctx, caches[c], qs, theta_d, outs[c], out, rws, dws, stream=stream, spans=structs[c])
            else:
                B.route(ctx, caches[c], qs, theta_d, outs[c], rws, stream=stream, spans=structs[c])
                B.decode(ctx, caches[c], qs, outs[c], out, dws, stream=stream, spans=structs[c])

        chunks = graph_chunks(args.warmup, args.steps, gs)
        with torch.cuda.stream(stream):
            for i in range(args.warmup):
                step(i)
        torch.cuda.synchronize()
        # per-kernel durations: HIP events around each library kernel on its
        # launch stream, over an eager pass of exactly the timed steps (events
        # recorded during graph capture are not re-recorded by graph replays)
        ctx.profile(True)
        with torch.cuda.stream(stream):
            for i in range(args.steps):
                step(args.warmup + i)
        torch.cuda.synchronize()
        prof = ctx.profile_read()
        ctx.profile(False)
        kern_us = {k: (v[0] / v[1]) * 1e3 for k, v in prof.items() if v[1] > 0}
        kern_n = {k: v[1] for k, v in prof.items() if v[1] > 0}
        graphs = {}
        for first, n in chunks:
            key = graph_key(first, n, period)
            if key in graphs:
                continue
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=stream):
                for u in range(n):
                    step(first + u)
            graphs[key] = gr
        for gr in graphs.values():                    # one untimed replay of each graph
            gr.replay()
        torch.cuda.synchronize()
        log(f"{label} f={frac}: {len(graphs)} graphs for {len(chunks)} chunks of <= {gs} steps; per launch (events): "
            + ", ".join(f"{k} {u:.1f} us" for k, u in kern_us.items()))
        t1 = time.perf_counter()
        for first, n in chunks:
            graphs[graph_key(first, n, period)].replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t1
        del graphs
        ms_per_step = wall * 1e3 / args.steps
        log(f"{label} f={frac}: timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step")
        # algorithmic bytes of the timed steps (lists realized per query)
        per_q = []
        for qi in range(Q):
            B.route(ctx, cache, qd[qi], theta_d, outs[0], rws)
            torch.cuda.synchronize()
            cnt = outs[0].exp_count.cpu().numpy()
            by = algorithmic_bytes(w, plan, cnt, outs[0].exp_list.cpu().numpy(), e)
            by["frac"] = float(cnt.sum()) / max(1, nseg_tot)
            per_q.append(by)
        idx = [(args.warmup + i) % Q for i in range(args.steps)]
        avg = {k: sum(per_q[i][k] for i in idx) / args.steps for k in per_q[0]}
        qb = w.batch * w.n_q_heads * w.head_dim * e
        names, shares = {}, {"route": avg["route"]}
        rest = avg["attend"]
        if "overlap" in kern_us:          # decode_step: the full-resolution pass beside the route
            names["overlap"] = "attend_full_kernel"
            shares["overlap"] = avg["full"]
            rest = avg["attend"] - avg["full"] + qb
        if "expand" in kern_us:           # separate summary and expanded-span launches
            names.update(full="attend_full_kernel", expand="attend_expanded_kernel")
            shares.update(full=rest - avg["factors"], expand=avg["factors"] + qb)
        else:                             # one fused attention launch, timed under "full"
            names["attend"] = "attend_fused_kernel"
            kern_us["attend"] = kern_us.pop("full")
            kern_n["attend"] = kern_n.pop("full")
            shares["attend"] = rest
        gbs = {k: shares[k] / (kern_us[k] * 1e-6) / 1e9 for k in shares}
        dom = max(names, key=lambda k: kern_us[k])
        step_gbs = avg["total"] / (ms_per_step / 1e3) / 1e9
        steps_per_s = 1e3 / ms_per_step
        rec = {
            "metric": "mixed-res decode steps/s and effective ctx tokens/s @128K; % of HBM peak",
            "value": steps_per_s, "unit": "steps/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": w.dtype,
            "data": "synthetic (seeded; Llama-3-8B layer shape, lognormal surprisal, rank-4 block structure)",
            "config": {"workload": w.name, "batch": w.batch, "n_ctx": w.n_ctx, "n_q_heads": w.n_q_heads,
                       "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "rank_range": [w.rank_lo, w.rank_hi],
                       "expand_frac_target": "full" if target is None else
                       (target[0] if len(set(target)) == 1 else [round(f, 4) for f in target]),
                       "expand_frac_realized": round(float(avg["frac"]), 4), "full_rank_unit_gates": full_rank,
                       "factors": "device", "layers": 1, "cache_copies_rotated": ncopy, "launch": "hip-graph",
                       "steps_per_graph": gs,
                       "route_overlap": "full-resolution pass on a second stream" if args.overlap else "none",
                       "reading": {"rank_cap": w.rank_cap, "basis": w.basis, "route_keys": w.route_keys,
                                   "boundary_quantile": w.boundary_quantile}},
            "eff_ctx_tokens_per_s": steps_per_s * w.batch * w.n_ctx,
            "algorithmic_bytes_per_step": int(avg["total"]),
            "step_hbm_gbs": step_gbs, "step_hbm_frac": step_gbs / PEAK_HBM_GBS,
            "kernels": {k: {"us_per_launch": kern_us[k], "launches_timed": kern_n.get(k),
                            "algorithmic_bytes": int(shares[k]), "gbs": gbs[k], "hbm_frac": gbs[k] / PEAK_HBM_GBS}
                        for k in shares},
            "roofline": {"bound": "hbm", "kernel": names[dom], "achieved": gbs[dom], "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": gbs[dom] / PEAK_HBM_GBS,
                         "traffic": measured_traffic(names[dom]), "bytes_per_launch": int(shares[dom]),
                         "duration_source": "HIP events around each launch on its stream, eager pass over the "
                                            "same steps as the timed region"},
            "memory": resident_bytes(w, plan, cache),
            "build": {"seconds": build_s, "where": "device" if w.basis == "joint" else "host",
                      "includes": "plan, K/V upload, summaries, routing keys, factors, synchronised"},
        }
        recs.append((rec, theta))
    ctx.close()
    return recs


# ------------------------------------------------------------------ dense baseline
def measure_dense(w, x, args, label):
    """Dense flash-decode over all T cached tokens (the full-KV decode SeKV is
    compared with), timed like the mixed path: graph replays of the timed
    steps, per-kernel events in an eager pass, >= 1 GiB of rotated K/V copies."""
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B

    e = 2 if w.dtype == "bf16" else 4
    Q = min(args.queries, x.q.shape[0])
    ctx = B.Context(0)
    cfg = B.make_config(w, False)
    et = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    k0 = torch.from_numpy(x.k).to(et).cuda()
    v0 = B.tile_values_device(torch.from_numpy(x.v).to(et).cuda())
    kv_bytes = k0.numel() * e + v0.numel() * e
    ncopy = args.copies or max(2, math.ceil((1 << 30) / kv_bytes))
    ks = [k0] + [k0.clone() for _ in range(ncopy - 1)]
    vs = [v0] + [v0.clone() for _ in range(ncopy - 1)]
    qd = torch.from_numpy(x.q[:Q]).to(et).cuda().contiguous()
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    ws = B.dense_workspace(ctx, cfg)
    stream = torch.cuda.Stream()
    period = math.lcm(ncopy, Q)

    def step(i):
        c = i % ncopy
        B.dense_decode(ctx, cfg, ks[c], vs[c], qd[i % Q], out, ws, stream=stream)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
        ctx.profile(True)
        for i in range(args.steps):
            step(args.warmup + i)
    torch.cuda.synchronize()
    prof = ctx.profile_read()
    ctx.profile(False)
    us = prof["full"][0] / prof["full"][1] * 1e3
    chunks = graph_chunks(args.warmup, args.steps, max(1, args.graph_steps))
    graphs = {}
    for first, n in chunks:
        key = graph_key(first, n, period)
        if key not in graphs:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=stream):
                for u in range(n):
                    step(first + u)
            graphs[key] = gr
    for gr in graphs.values():
        gr.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for first, n in chunks:
        graphs[graph_key(first, n, period)].replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t1) * 1e3 / args.steps
    del graphs
    T, d = w.n_ctx, w.head_dim
    step_bytes = w.batch * (w.n_kv_heads * T * 2 * d * e + w.n_q_heads * d * (e + 4))
    kern_bytes = w.batch * (w.n_kv_heads * T * 2 * d * e + w.n_q_heads * d * e)
    log(f"{label} dense: {ms * 1e3:.1f} us/step, attend_full_kernel {us:.1f} us")
    ctx.close()
    return {
        "metric": "dense flash-decode steps/s (baseline: softmax over all T cached tokens)",
        "value": 1e3 / ms, "unit": "steps/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "dtype": w.dtype, "data": "synthetic (seeded)",
        "config": {"workload": w.name + "-dense", "batch": w.batch, "n_ctx": T, "cache_copies_rotated": ncopy,
                   "launch": "hip-graph"},
        "eff_ctx_tokens_per_s": 1e3 / ms * w.batch * T,
        "algorithmic_bytes_per_step": step_bytes,
        "step_hbm_frac": step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "roofline": {"bound": "hbm", "kernel": "attend_full_kernel", "achieved": kern_bytes / (us * 1e-6) / 1e9,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": kern_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                     "bytes_per_launch": kern_bytes},
    }


# ------------------------------------------------------------------ host-resident measurement
def measure_append(args):
    """Online span sealing: the headline workload's caches in the decode-time
    (sealed) layout at 128K, grown by --append tokens with one
    sekv_append_token call per token (append every (b, kv) row; summarise,
    route-key and factor each span that seals).  One record: calls/s and
    microseconds per call (host decisions and upload included, synchronised
    once at the end), spans sealed."""
    import numpy as np
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    from hierarchical_kv_cache_sekv_amd import synth

    base = synth.workload(args.workload, factors_on_host=False)
    T0, N = base.n_ctx, args.append
    w = base.with_(n_ctx=T0 + N)
    x = synth.make_inputs(w, n_steps=1)
    ctx = B.Context(0)
    cfg = B.make_config(w)
    cfg.sealed, cfg.n_ctx_max, cfg.n_ctx = 1, T0 + N, T0
    plan = B.plan_spans(cfg, x.surprisal[:, :T0], x.boundary_thr, x.rank_req)
    cmax = B.make_config(w)
    cmax.sealed, cmax.n_ctx_max = 1, T0 + N
    pmax = B.plan_spans(cmax, x.surprisal, x.boundary_thr, x.rank_req)
    cache = B.SpanCache(cfg, plan, fac_capacity=pmax.fac_elems, sg_capacity=pmax.sg_elems)
    et = cache.elem
    kd = torch.from_numpy(x.k).to(et).cuda()
    vd = torch.from_numpy(x.v).to(et).cuda()
    B.build_spans(ctx, cache, kd[:, :, :T0].contiguous(), vd[:, :, :T0].contiguous(), x.surprisal[:, :T0],
                  x.route_proj, x.gate)
    P = torch.from_numpy(np.ascontiguousarray(x.route_proj, np.float32)).cuda()
    ws = B.append_workspace(cache)
    kn = [kd[:, :, t].contiguous() for t in range(T0, T0 + N)]
    vn = [vd[:, :, t].contiguous() for t in range(T0, T0 + N)]
    del kd, vd
    torch.cuda.synchronize()
    sealed = 0
    t1 = time.perf_counter()
    for i in range(N):
        sealed += int(B.append_token(ctx, cache, kn[i], vn[i], x.surprisal, x.boundary_thr, P, x.gate, x.rank_req,
                                     ws).sum())
    torch.cuda.synchronize()
    dt = time.perf_counter() - t1
    ctx.close()
    log(f"append: {N} calls, {sealed} spans sealed, {dt * 1e6 / N:.1f} us/call")
    return {"metric": "online span sealing (sekv_append_token) calls/s", "value": N / dt, "unit": "calls/s",
            "n_gpus": 1, "steps": N, "warmup": 0, "ms_per_step": dt * 1e3 / N, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded)",
            "config": {"workload": base.name + " decode-time layout, +%d tokens" % N, "batch": w.batch,
                       "n_ctx_start": T0, "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                       "spans_sealed": sealed, "spans_sealed_per_call": sealed / N,
                       "timing": "host wall clock over all calls (decisions, one upload, two kernels each), "
                                 "synchronised at the end"}}


def measure_host_resident(args):
    """The host-resident workload: 128K context, batch 1, ranks 8..32, factor
    pools in pinned host memory, the listed spans' factor blocks gathered and
    copied to the device every step (a host wait on the route list, a copy
    stream overlapped with the full-resolution pass).  Not graph-capturable;
    eager steps.  One record: end-to-end steps/s including the PCIe copy, the
    factor bytes that cross PCIe per step and their rate, and the kernels' HBM
    fraction on their algorithmic bytes."""
    import numpy as np
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    from hierarchical_kv_cache_sekv_amd import synth

    w = synth.workload(3, factors_on_host=True)
    e = 2 if w.dtype == "bf16" else 4
    Q = args.queries
    log(f"workload {w.name}: B={w.batch} T={w.n_ctx} ranks {w.rank_lo}..{w.rank_hi} f={w.expand_frac}, pinned host factors")
    x = synth.make_inputs(w, n_steps=Q)
    ctx = B.Context(0)
    cfg = B.make_config(w)
    plan = B.plan_spans(cfg, x.surprisal, x.boundary_thr, x.rank_req)
    cache = B.SpanCache(cfg, plan)
    kd = torch.from_numpy(x.k).to(cache.elem).cuda()
    vd = torch.from_numpy(x.v).to(cache.elem).cuda()
    B.build_spans(ctx, cache, kd, vd, x.surprisal, x.route_proj, x.gate)
    del kd, vd
    torch.cuda.synchronize()
    theta = calibrate(B, w, plan, cache, x, [w.expand_frac] * w.batch, Q)
    theta_d = torch.from_numpy(theta).cuda()
    qd = torch.from_numpy(x.q[:Q]).to(cache.elem).cuda().contiguous()
    ro = B.RouteOut(cfg, cache.seg_cap)
    rws = B.route_workspace(cache)
    ctx.set_fetch_mode(B.SEKV_FETCH_DIRECT if args.fetch == "direct" else B.SEKV_FETCH_STAGED)
    dws = B.DecodeWorkspace(cache, ctx=ctx)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    copy_stream = torch.cuda.Stream()

    def step(i):
        qs = qd[i % Q]
        B.route(ctx, cache, qs, theta_d, ro, rws)
        B.decode(ctx, cache, qs, ro, out, dws, copy_stream=copy_stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ctx.profile(True)
    t1 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t1) * 1e3 / args.steps
    prof = ctx.profile_read()
    ctx.profile(False)
    kern_us = {k: (v[0] / max(v[1], 1)) * 1e3 for k, v in prof.items()}
    host = ctx.host_timing() if args.fetch == "staged" else None
    per_q = []
    nseg_tot = sum(int(plan.n_seg[b]) for b in range(w.batch)) * w.n_kv_heads
    for qi in range(Q):
        B.route(ctx, cache, qd[qi], theta_d, ro, rws)
        torch.cuda.synchronize()
        cnt = ro.exp_count.cpu().numpy()
        by = algorithmic_bytes(w, plan, cnt, ro.exp_list.cpu().numpy(), e)
        by["frac"] = float(cnt.sum()) / max(1, nseg_tot)
        per_q.append(by)
    idx = [(args.warmup + i) % Q for i in range(args.steps)]
    avg = {k: sum(per_q[i][k] for i in idx) / args.steps for k in per_q[0]}
    pcie = avg["factors"]
    kern_total_us = kern_us["route"] + kern_us["full"] + kern_us["expand"]
    fetch = {"staged": "host gather into pinned staging + hipMemcpyAsync on a copy stream, one host wait per step",
             "direct": "kernels read the listed factor blocks from the pinned pools over the bus, no host wait"}
    rec = {
        "metric": "host-resident mixed-res decode steps/s (PCIe copy of the listed factors included)",
        "value": 1e3 / ms, "unit": "steps/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "launch": "eager", "fetch": fetch[args.fetch],
        "dtype": w.dtype, "data": "synthetic (seeded; Llama-3-8B layer shape)",
        "config": {"workload": w.name, "batch": w.batch, "n_ctx": w.n_ctx, "rank_range": [w.rank_lo, w.rank_hi],
                   "expand_frac_target": w.expand_frac, "expand_frac_realized": round(float(avg["frac"]), 4),
                   "factors": "pinned host"},
        "eff_ctx_tokens_per_s": 1e3 / ms * w.batch * w.n_ctx,
        "pcie_factor_bytes_per_step": int(pcie),
        "pcie_gbs_over_step": pcie / (ms * 1e-3) / 1e9,
        "host_phases_us_per_step": host,
        "kernels_us": {k: round(v, 2) for k, v in kern_us.items()},
        "kernel_hbm_frac": avg["total"] / (kern_total_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
        "kernel_time_fraction_of_step": kern_total_us / (ms * 1e3),
        "algorithmic_bytes_per_step": int(avg["total"]),
        "memory": resident_bytes(w, plan, cache),
    }
    ctx.close()
    return rec


# ------------------------------------------------------------------ multi-layer host-resident decode
def measure_layers(args):
    """Multi-layer decode with host-resident factors: --layers layers of the
    128K batch-1 host-factor workload, each with its own seeded K/V, spans,
    pinned host factor pools and queries (step-to-step correlation
    --query-corr), decoded layer after layer every step (route, then
    attention).  The listed spans' factor blocks reach the GPU through one
    device factor cache of --cache-mb shared by all layers; the same steps are
    also timed with the direct fetch (every listed block over the bus).  Eager
    steps (one host wait per layer in the cached mode).  The step's first layer
    output is compared bit for bit between the two fetches."""
    import numpy as np
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    from hierarchical_kv_cache_sekv_amd import synth

    N, W, K = args.layers, args.warmup, args.steps
    Q = max(args.queries, W + K)
    e = 2
    ctx = B.Context(0)
    layers = []
    t0 = time.time()
    for li in range(N):
        w = synth.workload(3, factors_on_host=True, layer=li, query_corr=args.query_corr)
        x = synth.make_inputs(w, n_steps=Q)
        cfg = B.make_config(w)
        plan = B.plan_spans(cfg, x.surprisal, x.boundary_thr, x.rank_req)
        cache = B.SpanCache(cfg, plan)
        kd = torch.from_numpy(x.k).to(cache.elem).cuda()
        vd = torch.from_numpy(x.v).to(cache.elem).cuda()
        B.build_spans(ctx, cache, kd, vd, x.surprisal, x.route_proj, x.gate)
        del kd, vd
        torch.cuda.synchronize()
        theta = torch.from_numpy(calibrate(B, w, plan, cache, x, [w.expand_frac] * w.batch, Q)).cuda()
        qd = torch.from_numpy(x.q[:Q]).to(cache.elem).cuda().contiguous()
        layers.append(dict(w=w, plan=plan, cache=cache, theta=theta, qd=qd, ro=B.RouteOut(cfg, cache.seg_cap),
                           rws=B.route_workspace(cache), dws=B.DecodeWorkspace(cache, ctx=ctx),
                           cws=B.CachedDecodeWorkspace(cache, ctx=ctx),
                           out=torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")))
        del x
        log(f"layer {li}: {w.name} built ({time.time() - t0:.1f}s so far)")
    w0 = layers[0]["w"]
    fc = B.FactorCache(ctx, args.cache_mb << 20)
    cs = torch.cuda.Stream()

    def step(i, cached):
        for li, L in enumerate(layers):
            qs = L["qd"][i]
            B.route(ctx, L["cache"], qs, L["theta"], L["ro"], L["rws"])
            if cached:
                B.cached_decode(ctx, fc, li, L["cache"], qs, L["ro"], L["out"], L["cws"], copy_stream=cs)
            else:
                B.decode(ctx, L["cache"], qs, L["ro"], L["out"], L["dws"])

    # bitwise check of one step, then warm the cache
    step(0, False)
    torch.cuda.synchronize()
    ref = layers[0]["out"].clone()
    step(0, True)
    torch.cuda.synchronize()
    same = bool(torch.equal(ref, layers[0]["out"]))
    fc.invalidate(-1)
    res = {}
    for mode in ("direct", "cached"):
        cached = mode == "cached"
        # pass 1 timed (no timing events); pass 2 the same steps from the same
        # (empty) cache with per-kernel events
        for timed in (True, False):
            fc.invalidate(-1)
            for i in range(W):
                step(i, cached)
            torch.cuda.synchronize()
            fc.stats(reset=True)
            ctx.host_timing()
            ctx.profile(not timed)
            t1 = time.perf_counter()
            for i in range(W, W + K):
                step(i, cached)
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t1) * 1e3 / K
            if timed:
                res[mode] = dict(ms=ms, stats=fc.stats(), host=ctx.host_timing())
                log(f"{mode}: {ms:.3f} ms per step ({N} layers)")
            else:
                prof = ctx.profile_read()
                ctx.profile(False)
                res[mode].update(kern={k: v[0] * 1e3 / max(v[1], 1) for k, v in prof.items()},
                                 launches={k: v[1] for k, v in prof.items()})
    # listed factor bytes per step (what the direct fetch moves over the bus)
    listed = 0.0
    for L in layers:
        for i in range(W, W + K):
            B.route(ctx, L["cache"], L["qd"][i], L["theta"], L["ro"], L["rws"])
            torch.cuda.synchronize()
            cnt = L["ro"].exp_count.cpu().numpy()
            listed += algorithmic_bytes(L["w"], L["plan"], cnt, L["ro"].exp_list.cpu().numpy(), e)["factors"]
    listed /= K
    st = res["cached"]["stats"]
    bus = (st["bytes_filled"] + st["bytes_bypassed"]) / K
    kc = res["cached"]["kern"]
    rec = {
        "metric": "multi-layer host-resident decode steps/s (all layers, PCIe included)",
        "value": 1e3 / res["cached"]["ms"], "unit": "steps/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": res["cached"]["ms"], "higher_is_better": True, "launch": "eager",
        "fetch": "device factor cache (HBM, LRU across steps and layers; misses pulled by a fill kernel beside "
                 "the full-resolution pass)",
        "dtype": w0.dtype, "data": "synthetic (seeded per layer; Llama-3-8B layer shape)",
        "config": {"workload": f"{N} x {w0.name}", "layers": N, "batch": w0.batch, "n_ctx": w0.n_ctx,
                   "rank_range": [w0.rank_lo, w0.rank_hi], "expand_frac_target": w0.expand_frac,
                   "query_corr": args.query_corr, "cache_bytes": st["pages_total"] * B.CACHE_PAGE_BYTES},
        "bitwise_equal_to_direct_fetch": same,
        "direct_fetch": {"ms_per_step": res["direct"]["ms"], "steps_per_s": 1e3 / res["direct"]["ms"],
                         "bus_bytes_per_step": int(listed),
                         "bus_gbs_over_step": listed / (res["direct"]["ms"] * 1e-3) / 1e9},
        "speedup_vs_direct": res["direct"]["ms"] / res["cached"]["ms"],
        "cache": {"lookups_per_step": st["lookups"] / K, "hit_rate": st["hits"] / max(1, st["lookups"]),
                  "byte_hit_rate": st["bytes_hit"] / max(1, st["bytes_hit"] + st["bytes_filled"] + st["bytes_bypassed"]),
                  "bus_bytes_per_step": int(bus), "evictions_per_step": st["evictions"] / K,
                  "bypasses_per_step": st["bypasses"] / K, "resident_bytes": st["resident_bytes"],
                  "pages_used": st["pages_used"], "pages_total": st["pages_total"]},
        "kernels_us_per_launch": {k: round(v, 2) for k, v in kc.items() if res["cached"]["launches"][k]},
        "launches_per_layer": {k: v / (K * N) for k, v in res["cached"]["launches"].items() if v},
        "host_us_per_layer": res["cached"]["host"],
        "fill_kernel_gbs": (st["bytes_filled"] / res["cached"]["launches"]["fill"]) / (kc["fill"] * 1e-6) / 1e9
        if res["cached"]["launches"]["fill"] else None,
    }
    fc.close()
    ctx.close()
    return rec


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--frac", type=float, default=0.05, help="target union expansion fraction")
    ap.add_argument("--workload", type=int, default=5)
    ap.add_argument("--copies", type=int, default=0, help="cache copies to rotate (0: auto, >= 2)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle decode per worker")
    ap.add_argument("--cpu-workers", type=int, default=0, help="oracle worker processes (0: host cores, at most 16)")
    ap.add_argument("--queries", type=int, default=64)
    ap.add_argument("--graph-steps", type=int, default=8, help="decode steps captured per HIP graph")
    ap.add_argument("--split", type=int, default=0,
                    help="full-resolution entries per split-K chunk of the mixed decode (0: the library chooses)")
    ap.add_argument("--overlap", action="store_true",
                    help="one sekv_decode_step call per step (full-resolution pass on a second stream beside the "
                         "route) instead of sekv_route + sekv_mixed_attention_decode")
    ap.add_argument("--sweep", action="store_true",
                    help="after the headline line, one line per further point: 0/20/50%% and full expansion of the "
                         "headline workload, the 32K batch-1 and batch-8 workloads, and the host-resident workload")
    ap.add_argument("--append", type=int, default=0, metavar="N",
                    help="only measure online span sealing: N sekv_append_token calls on the workload's caches")
    ap.add_argument("--layers", type=int, default=0, metavar="N",
                    help="multi-layer host-resident decode of N layers through the device factor cache")
    ap.add_argument("--cache-mb", type=int, default=1024, help="device factor cache size (MiB) for --layers")
    ap.add_argument("--query-corr", type=float, default=0.9,
                    help="step-to-step query correlation of the --layers workload")
    ap.add_argument("--host-resident", action="store_true",
                    help="only measure the host-resident workload (pinned host factors fetched per step)")
    ap.add_argument("--fetch", choices=("staged", "direct"), default="direct",
                    help="host-resident fetch: host gather + copy (staged) or kernels reading pinned memory (direct)")
    ap.add_argument("--variant", choices=sorted(VARIANTS), default=None,
                    help="measure a reading variant of the workload instead of the default readings")
    ap.add_argument("--dense", action="store_true",
                    help="only measure the dense flash-decode baseline on the workload's K/V")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device-to-device copy three times (reference kernel for memory counters)")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="write the memory-counter record from rocprofv3 --pmc runs under DIR and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        rec = summarize_counters(args.summarize_counters, f"workload {args.workload}, f={args.frac}")
        with open(COUNTERS, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec, indent=1))
        return
    if args.copy_calibration:
        import torch
        a = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copied 1 GiB three times")
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (--gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    if args.host_resident:
        print(json.dumps(measure_host_resident(args)), flush=True)
        return
    if args.layers:
        print(json.dumps(measure_layers(args)), flush=True)
        return
    if args.append:
        print(json.dumps(measure_append(args)), flush=True)
        return

    from hierarchical_kv_cache_sekv_amd import synth
    w = synth.workload(args.workload, factors_on_host=False, **(VARIANTS[args.variant] if args.variant else {}))
    Q = args.queries
    log(f"workload {w.name}: B={w.batch} T={w.n_ctx} Hq={w.n_q_heads} Hkv={w.n_kv_heads} d={w.head_dim} "
        f"{w.dtype} ranks {w.rank_lo}..{w.rank_hi} f={args.frac}")
    t0 = time.time()
    x = synth.make_inputs(w, n_steps=Q)
    log(f"inputs drawn in {time.time() - t0:.1f}s")
    if args.dense:
        print(json.dumps(measure_dense(w, x, args, w.name)), flush=True)
        return
    pool = None
    if not args.no_cpu_baseline:
        nw = args.cpu_workers or min(16, len(os.sched_getaffinity(0)))
        pool = OraclePool(w, x, nw)          # forked before any GPU call
    try:
        import torch
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        fracs = [args.frac] + ([0.0, 0.20, 0.50] if args.sweep else [])
        recs = measure_device(w, x, fracs, args, w.name)
        head, theta = recs[0]
        if pool is not None:
            log(f"timing the CPU oracle on {pool.n} worker processes")
            head["cpu_baseline"] = oracle_baseline(pool, theta, args.cpu_budget)
            log(f"oracle: {head['cpu_baseline']['value']:.4f} steps/s on {pool.n} cores")
        else:
            head["cpu_baseline"] = None
        print(json.dumps(head), flush=True)
        if args.sweep:
            for r, _ in recs[1:]:
                print(json.dumps(r), flush=True)
            print(json.dumps(measure_dense(w, x, args, w.name)), flush=True)
            for name, over in VARIANTS.items():
                wv = w.with_(**over)
                xv = x if "boundary_quantile" not in over else synth.make_inputs(wv, n_steps=Q)
                for r, _ in measure_device(wv, xv, [args.frac], args, f"{w.name} {name}"):
                    print(json.dumps(r), flush=True)
                del xv
            del x
            xf = synth.make_inputs(w, n_steps=Q, full_rank_unit_gates=True)
            for r, _ in measure_device(w, xf, [None], args, w.name + " full rank", full_rank=True):
                print(json.dumps(r), flush=True)
            del xf
            for wid in (2, 4):
                w2 = synth.workload(wid)
                x2 = synth.make_inputs(w2, n_steps=Q)
                fr = [w2.expand_frac] if w2.expand_frac >= 0 else [x2.expand_frac]
                for r, _ in measure_device(w2, x2, fr, args, w2.name):
                    print(json.dumps(r), flush=True)
                del x2
            print(json.dumps(measure_host_resident(args)), flush=True)
            args.append = args.append or 512
            print(json.dumps(measure_append(args)), flush=True)
            args.layers = args.layers or 4
            print(json.dumps(measure_layers(args)), flush=True)
    finally:
        if pool is not None:
            pool.close()


if __name__ == "__main__":
    main()
