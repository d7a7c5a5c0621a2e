#!/usr/bin/env python3
"""Mixed-resolution decode benchmark on one MI355X.

One step = one decode step of one attention layer for the whole batch: route
(per-head routing + compaction) then mixed-resolution attention (full-res +
size-corrected summaries + expanded spans rebuilt from their factors) and the
log-sum-exp combine.  Workload: Llama-3-8B-shaped layer (32 query heads, 8 KV
heads, head dim 128, bf16), 128K context, batch 4, device-resident factors,
5% union expansion per step, ranks 16..64 (synthetic seeded inputs; the
pages' own evaluation sets are not available).  Inputs are resident in HBM
before timing; the cache is rotated over >= 2 copies so the 256 MB last-level
cache cannot hold the working set.

Prints ONE JSON line on stdout; progress goes to stderr.
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


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE / WRITE_SIZE
    counter runs (scaled by a 1 GiB copy's counts), or None when a source they
    depend on (the kernels and the launch constants and plan) has changed since
    they were taken: the record holds the SHA-256 of the sources' contents,
    concatenated in the listed order."""
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


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(w, plan, counts, lists, e):
    """Bytes the method must move per step (the dense work it avoids excluded).

    Per sequence: queries and outputs Hq*d*(e+4); per KV head the full-res K/V
    e*2d*n_full, the summaries kbar, vbar and rho e*3d*n_seg, and for each
    listed span its factors e*r*(L+2d) + 8r (sigma and gate in float32).
    Returns per-kernel shares {route: q + rho, full: q + full-res K/V + kbar,
    vbar, expand: q + factors} and the step total."""
    import numpy as np
    d, Hq, Hkv = w.head_dim, w.n_q_heads, w.n_kv_heads
    route = full = expand = total = 0
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
        full += qb + Hkv * e * 2 * d * (nf + ns)
        expand += qb + fac
        total += Hq * d * (e + 4) + Hkv * (e * 2 * d * nf + e * 3 * d * ns) + fac
    return {"route": route, "full": full, "expand": expand, "total": total}


def cpu_baseline(w, x, theta, budget_s=12.0):
    """The oracle, as it stands, on one sequence of the workload (b = 0),
    single-threaded BLAS; steps are timed until the budget is spent.  Scaled to
    full steps by the batch size."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle as O
    t0 = time.time()
    with threadpool_limits(1):
        cache = O.build_cache(x.k[:1], x.v[:1], x.surprisal[:1], x.boundary_thr[:1], x.route_proj, x.rank_req[:1],
                              x.gate[:1], n_sink=w.n_sink, n_recent=w.n_recent, lo=w.min_span, hi=w.max_span,
                              dtype=w.dtype)
        log(f"oracle cache for sequence 0 built in {time.time() - t0:.1f}s")
        G = w.group
        n = 0
        t1 = time.perf_counter()
        while True:
            st = n % x.q.shape[0]
            q = x.q[st, 0]
            z = np.concatenate([O.route_scores(q[kv * G:(kv + 1) * G], cache.rho[0][kv])
                                for kv in range(w.n_kv_heads)])
            dec = z > theta[0][:, None]
            O.mixed_attention(cache, 0, q, dec, G)
            n += 1
            el = time.perf_counter() - t1
            if el >= budget_s or n >= 64:
                break
    per_seq_step = el / n
    steps_per_s = 1.0 / (per_seq_step * w.batch)
    return {"value": steps_per_s, "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"sequence 0 of {w.batch} (all {w.n_q_heads} heads), {n} decode steps (route + mixed "
                      f"attention, fp64 numpy, 1 BLAS thread) in {el:.1f}s; steps/s = 1/(time per sequence-step "
                      f"x batch {w.batch})",
            "eff_ctx_tokens_per_s": steps_per_s * w.batch * w.n_ctx}


def host_resident(args):
    """The host-resident workload: 128K context, batch 1, ranks 8..32, factor
    pools in pinned host memory, the listed spans' factor blocks gathered and
    copied to the device every step (a host wait on the route list, a copy
    stream overlapped with the full-resolution pass).  Not graph-capturable;
    eager steps.  Prints one JSON line: end-to-end steps/s including the PCIe
    copy, the factor bytes that cross PCIe per step and their rate, and the
    kernels' HBM fraction on their algorithmic bytes."""
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
    et = cache.elem
    kd = torch.from_numpy(x.k).to(et).cuda()
    vd = torch.from_numpy(x.v).to(et).cuda()
    B.build_spans(ctx, cache, kd, vd, x.surprisal, x.route_proj, x.gate)
    del kd, vd
    torch.cuda.synchronize()
    G = w.group
    qf = torch.from_numpy(x.q).cuda()
    rho = cache.rho.float()
    theta = np.empty((w.batch, w.n_q_heads), np.float32)
    for b in range(w.batch):
        ns = int(plan.n_seg[b])
        z = torch.empty((Q, w.n_q_heads, ns), device="cuda")
        for kv in range(w.n_kv_heads):
            z[:, kv * G:(kv + 1) * G] = qf[:, b, kv * G:(kv + 1) * G] @ rho[b, kv, :ns].T
        theta[b] = synth.calibrate_theta(z.cpu().numpy(), w.expand_frac, G)
    theta_d = torch.from_numpy(theta).cuda()
    qd = qf.to(et).contiguous()
    del qf, rho
    ro = B.RouteOut(cfg, cache.seg_cap)
    rws = B.route_workspace(cache)
    dws = B.DecodeWorkspace(cache)
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
    # algorithmic bytes and PCIe bytes of the timed steps (lists realized per query)
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
    pcie = avg["expand"] - w.batch * w.n_q_heads * w.head_dim * e      # the listed spans' factors and sigma, gate
    kern_total_us = kern_us["route"] + kern_us["full"] + kern_us["expand"]
    rec = {
        "metric": "host-resident mixed-res decode steps/s (PCIe copy of the listed factors included)",
        "value": 1e3 / ms, "unit": "steps/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "launch": "eager (host wait on the route list each step)",
        "dtype": w.dtype, "data": "synthetic (seeded; Llama-3-8B layer shape)",
        "config": {"workload": w.name, "batch": w.batch, "n_ctx": w.n_ctx, "rank_range": [w.rank_lo, w.rank_hi],
                   "expand_frac_target": w.expand_frac, "expand_frac_realized": round(float(avg["frac"]), 4),
                   "factors": "pinned host"},
        "eff_ctx_tokens_per_s": 1e3 / ms * w.batch * w.n_ctx,
        "pcie_factor_bytes_per_step": int(pcie),
        "pcie_gbs_over_step": pcie / (ms * 1e-3) / 1e9,
        "kernels_us": {k: round(v, 2) for k, v in kern_us.items()},
        "kernel_hbm_frac": avg["total"] / (kern_total_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
        "kernel_time_fraction_of_step": kern_total_us / (ms * 1e3),
        "algorithmic_bytes_per_step": int(avg["total"]),
    }
    print(json.dumps(rec), flush=True)
    ctx.close()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--frac", type=float, default=0.05, help="target union expansion fraction")
    ap.add_argument("--workload", type=int, default=5)
    ap.add_argument("--copies", type=int, default=0, help="cache copies to rotate (0: auto, >= 2)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--queries", type=int, default=64)
    ap.add_argument("--launch", choices=("graph", "eager"), default="graph",
                    help="timed pass: replay of captured HIP graphs (default) or eager launches")
    ap.add_argument("--graph-steps", type=int, default=8, help="decode steps captured per HIP graph")
    ap.add_argument("--host-resident", action="store_true",
                    help="only measure the host-resident workload (pinned host factors fetched per step) and print its own line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device-to-device copy three times (reference kernel for memory counters)")
    args = ap.parse_args()
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
    if args.host_resident:
        host_resident(args)
        return

    import numpy as np
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    from hierarchical_kv_cache_sekv_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = synth.workload(args.workload, factors_on_host=False)
    e = 2 if w.dtype == "bf16" else 4
    Q = args.queries
    log(f"workload {w.name}: B={w.batch} T={w.n_ctx} Hq={w.n_q_heads} Hkv={w.n_kv_heads} d={w.head_dim} "
        f"{w.dtype} ranks {w.rank_lo}..{w.rank_hi} f={args.frac}")
    t0 = time.time()
    x = synth.make_inputs(w, n_steps=Q)
    log(f"inputs drawn in {time.time() - t0:.1f}s")

    ctx = B.Context(0)
    cfg = B.make_config(w)
    plan = B.plan_spans(cfg, x.surprisal, x.boundary_thr, x.rank_req)
    cache = B.SpanCache(cfg, plan)
    et = cache.elem
    t0 = time.time()
    kd = torch.from_numpy(x.k).to(et).cuda()
    vd = torch.from_numpy(x.v).to(et).cuda()
    B.build_spans(ctx, cache, kd, vd, x.surprisal, x.route_proj, x.gate)
    del kd, vd
    torch.cuda.synchronize()
    log(f"library build (plan + summaries + rank-r factors) in {time.time() - t0:.1f}s; n_seg={plan.n_seg.tolist()}")

    # thresholds: per-head quantiles of the routing scores over the query set
    G = w.group
    qf = torch.from_numpy(x.q).cuda()                      # [Q][B][Hq][d] f32 (bf16-exact)
    rho = cache.rho.float()
    theta = np.empty((w.batch, w.n_q_heads), np.float32)
    for b in range(w.batch):
        ns = int(plan.n_seg[b])
        z = torch.empty((Q, w.n_q_heads, ns), device="cuda")
        for kv in range(w.n_kv_heads):
            z[:, kv * G:(kv + 1) * G] = qf[:, b, kv * G:(kv + 1) * G] @ rho[b, kv, :ns].T
        theta[b] = synth.calibrate_theta(z.cpu().numpy(), args.frac, G)
    theta_d = torch.from_numpy(theta).cuda()
    qd = qf.to(et).contiguous()
    del qf, rho

    resident = cache.device_bytes()
    ncopy = args.copies or max(2, math.ceil((1 << 30) / resident))
    caches = [cache] + [cache.clone() for _ in range(ncopy - 1)]
    structs = [c.struct() for c in caches]
    outs = [B.RouteOut(cfg, cache.seg_cap) for _ in range(ncopy)]
    rws = B.route_workspace(cache)
    dws = B.DecodeWorkspace(cache)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    log(f"{ncopy} cache copies of {resident / 2**20:.0f} MiB each resident in HBM")

    gs = max(1, args.graph_steps)
    nstep_combo = math.lcm(ncopy, Q, gs)

    def step(i):
        c = i % ncopy
        qs = qd[i % Q]
        B.route(ctx, caches[c], qs, theta_d, outs[c], rws, spans=structs[c])
        B.decode(ctx, caches[c], qs, outs[c], out, dws, spans=structs[c])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # profiled pass: the same steps launched eagerly, HIP events around every
    # kernel on the stream it is launched on (per-kernel durations)
    ctx.profile(True)
    t1 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t1) * 1e3 / args.steps
    prof = ctx.profile_read()
    ctx.profile(False)
    kern_us = {k: (v[0] / max(v[1], 1)) * 1e3 for k, v in prof.items()}
    log(f"eager: {eager_ms * 1e3:.1f} us/step; per launch: " + ", ".join(f"{k} {u:.1f} us" for k, u in kern_us.items()))

    # timed pass: HIP graphs of `gs` consecutive steps (cycling cache copies and
    # queries), replayed; a multi-layer model would likewise launch many
    # layer-steps per graph
    graphs = None
    if args.launch == "graph":
        assert args.steps % gs == 0 and args.warmup % gs == 0, "--steps and --warmup must be multiples of --graph-steps"
        graphs = []
        cap_stream = torch.cuda.Stream()
        for j in range(nstep_combo // gs):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=cap_stream):
                for u in range(gs):
                    step(j * gs + u)
            graphs.append(gr)
        for i in range(0, args.warmup, gs):
            graphs[(i // gs) % len(graphs)].replay()
        torch.cuda.synchronize()
        log(f"captured {len(graphs)} graphs of {gs} steps")
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if graphs is not None:
        for i in range(0, args.steps, gs):
            graphs[((args.warmup + i) // gs) % len(graphs)].replay()
    else:
        for i in range(args.steps):
            step(args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t1
    ms_per_step = wall * 1e3 / args.steps
    log(f"timed {args.steps} steps ({args.launch}): {ms_per_step * 1e3:.1f} us/step")
    del graphs

    # algorithmic bytes of the timed steps (lists realized per query step)
    nseg_tot = sum(int(plan.n_seg[b]) for b in range(w.batch)) * w.n_kv_heads
    per_q = []
    for qi in range(Q):
        B.route(ctx, cache, qd[qi], theta_d, outs[0], rws)
        torch.cuda.synchronize()
        cnt = outs[0].exp_count.cpu().numpy()
        lst = outs[0].exp_list.cpu().numpy()
        by = algorithmic_bytes(w, plan, cnt, lst, e)
        by["frac"] = float(cnt.sum()) / max(1, nseg_tot)
        per_q.append(by)
    idx = [(args.warmup + i) % Q for i in range(args.steps)]
    avg = {k: sum(per_q[i][k] for i in idx) / args.steps for k in per_q[0]}
    # kernels timed by the library's events: "route" (decide + compact), and either
    # one fused attention launch (reported under "full") or separate full-res /
    # expanded-span launches
    fused = prof["expand"][1] == 0
    if fused:
        avg["attend"] = avg["full"] + avg["expand"]
        kern_us["attend"] = kern_us["full"]
        keys = ("route", "attend")
        names = {"attend": "attend_fused_kernel"}
    else:
        keys = ("route", "full", "expand")
        names = {"full": "attend_full_kernel", "expand": "attend_expanded_kernel"}
    gbs = {k: avg[k] / (kern_us[k] * 1e-6) / 1e9 for k in keys}
    dom = max(names, key=lambda k: kern_us[k])
    step_gbs = avg["total"] / (ms_per_step / 1e3) / 1e9
    steps_per_s = 1e3 / ms_per_step

    base = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        base = cpu_baseline(w, x, theta)
        log(f"oracle: {base['value']:.4f} steps/s ({base['sample']})")

    rec = {
        "metric": "mixed-res decode steps/s and effective ctx tokens/s @128K; % of HBM peak",
        "value": steps_per_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; Llama-3-8B layer shape, lognormal surprisal, rank-4 block structure)",
        "config": {"workload": w.name, "batch": w.batch, "n_ctx": w.n_ctx, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "rank_range": [w.rank_lo, w.rank_hi],
                   "expand_frac_target": args.frac, "expand_frac_realized": round(float(avg["frac"]), 4),
                   "factors": "device", "layers": 1, "cache_copies_rotated": ncopy, "launch": args.launch,
                   "steps_per_graph": gs if args.launch == "graph" else None},
        "eff_ctx_tokens_per_s": steps_per_s * w.batch * w.n_ctx,
        "algorithmic_bytes_per_step": int(avg["total"]),
        "step_hbm_gbs": step_gbs,
        "step_hbm_frac": step_gbs / PEAK_HBM_GBS,
        "kernels": {k: {"us_per_launch": kern_us[k], "algorithmic_bytes": int(avg[k]), "gbs": gbs[k],
                        "hbm_frac": gbs[k] / PEAK_HBM_GBS} for k in keys},
        "roofline": {"bound": "hbm", "kernel": names[dom], "achieved": gbs[dom], "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": gbs[dom] / PEAK_HBM_GBS, "traffic": measured_traffic(names[dom]),
                     "bytes_per_launch": int(avg[dom])},
        "eager_ms_per_step": eager_ms,
        "cpu_baseline": base,
    }
    print(json.dumps(rec), flush=True)
    ctx.close()


if __name__ == "__main__":
    main()
