"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Inputs are seeded (hierarchical_kv_cache_sekv_amd.synth); the span cache is
built by the oracle and marshalled into the library's arrays, so decode parity
does not depend on the library's own build (checked separately).  Bar: the
expanded-span set (count, ascending list, head masks) bit-exact; outputs within
1e-4 (float32 cache) or 2e-2 (bfloat16 cache, float32 accumulation).
Sizes here span several tiles and ragged tails and finish in seconds; the
full-size workloads are in test_gpu_fullsize.py.
"""
import numpy as np
import pytest

import oracle as O
from hierarchical_kv_cache_sekv_amd import synth

from _harness import TOL, Device, compare_route, log, oracle_out, oracle_route, prepare, realized_fraction

pytestmark = pytest.mark.gpu

CASES = {
    "tiny-f32-T2K": dict(wid=1, steps=[0, 5, 15]),
    "bf16-d128-T4K": dict(wid=2, over=dict(n_ctx=4096), steps=[0, 1]),
    "bf16-ragged-B3-T4K": dict(wid=4, over=dict(n_ctx=4096, batch=3), steps=[0]),
    "bf16-g8-d64-T3000": dict(wid=2, over=dict(n_ctx=3000, n_q_heads=16, n_kv_heads=2, head_dim=64, min_span=3,
                                               max_span=40, rank_lo=1, rank_hi=24), steps=[0, 3]),
    "f32-g1-d128-T1500": dict(wid=1, over=dict(n_ctx=1500, n_q_heads=4, n_kv_heads=4, head_dim=128, rank_hi=20),
                              steps=[0, 1]),
    "bf16-g2-T2500-wide-rank": dict(wid=5, over=dict(n_ctx=2500, batch=2, n_q_heads=8, n_kv_heads=4, min_span=2,
                                                     max_span=128, rank_lo=30, rank_hi=128, boundary_quantile=0.995),
                                    steps=[0], frac=0.3),
    "f32-d64-T3000-wide-rank": dict(wid=1, over=dict(n_ctx=3000, min_span=2, max_span=128, rank_lo=40, rank_hi=128,
                                                     boundary_quantile=0.995), steps=[0], frac=0.3),
    "f32-len1-spans": dict(wid=1, over=dict(n_ctx=700, min_span=1, max_span=1), steps=[0, 1]),
    "f32-no-spans": dict(wid=1, over=dict(n_ctx=69, n_recent=64, n_sink=4), steps=[0]),
    "bf16-one-span": dict(wid=2, over=dict(n_ctx=300, n_recent=200, n_sink=4, min_span=8, max_span=128), steps=[0]),
    # reading variants
    "bf16-rank-cap-half": dict(wid=5, over=dict(n_ctx=4096, batch=2, rank_cap="half"), steps=[0, 1]),
    "bf16-separate-bases": dict(wid=5, over=dict(n_ctx=4096, batch=2, basis="separate"), steps=[0, 1]),
    "bf16-folded-route": dict(wid=2, over=dict(n_ctx=4096, batch=2, route_keys="folded"), steps=[0, 1]),
    "bf16-boundary-q97": dict(wid=2, over=dict(n_ctx=8192, boundary_quantile=0.97), steps=[0, 1]),
    "f32-d64-all-variants": dict(wid=1, over=dict(n_ctx=3000, rank_cap="half", basis="separate",
                                                  route_keys="folded"), steps=[0, 3]),
    "bf16-separate-wide-rank": dict(wid=5, over=dict(n_ctx=2500, batch=2, n_q_heads=8, n_kv_heads=4, min_span=2,
                                                     max_span=128, rank_lo=30, rank_hi=128, boundary_quantile=0.995,
                                                     basis="separate"), steps=[0], frac=0.3),
}

_PREP = {}


def _prep(name):
    if name not in _PREP:
        c = CASES[name]
        w = synth.workload(c["wid"], **c.get("over", {}))
        _PREP[name] = prepare(w, c["steps"], frac=c.get("frac"))
    return _PREP[name]


@pytest.fixture(scope="module")
def ctx():
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    assert torch.cuda.is_available()
    c = B.Context(0)
    yield c
    torch.cuda.synchronize()
    c.close()


@pytest.mark.parametrize("name", list(CASES))
def test_route_and_decode_parity(ctx, name):
    import torch
    p = _prep(name)
    log(f"case {name}: n_seg={[p.cache.n_seg(b) for b in range(p.w.batch)]}")
    dev = Device(p)
    tol = TOL[p.w.dtype]
    for si in range(len(p.steps)):
        ref = oracle_route(p, si)
        dev.route(ctx, si)
        compare_route(dev, ref)
        dev.route(ctx, si)                       # second run: identical bits (no races)
        compare_route(dev, ref)
        dev.decode(ctx, si)
        torch.cuda.synchronize()
        out = dev.out.cpu().numpy()
        want = oracle_out(p, si)
        err = max(float(np.abs(out[b] - want[b]).max()) for b in want)
        log(f"case {name} step {p.steps[si]}: f={realized_fraction(p, si):.3f} max|err|={err:.3e} tol={tol}")
        assert err <= tol
        out2 = dev.out.clone()
        dev.decode(ctx, si)
        torch.cuda.synchronize()
        assert torch.equal(out2, dev.out)        # deterministic
        # one sekv_decode_step call (full-resolution pass beside the route):
        # the same route outputs and the same output bits
        dev.out.zero_()
        dev.route_out.exp_count.fill_(-7)
        dev.step(ctx, si)
        torch.cuda.synchronize()
        compare_route(dev, ref)
        assert torch.equal(out2, dev.out)


def test_route_out_of_range_keys_stay_bit_exact(ctx):
    """Routing keys with extreme magnitudes (tiny, a bf16 subnormal, huge) in
    some spans: products that underflow to subnormals or carry large
    exponents still follow the canonical separately rounded chain, so the
    expanded set stays bit-exact."""
    from _harness import scores
    w = synth.workload(2, n_ctx=4096, batch=2)
    p = prepare(w, [0, 1])
    rng = np.random.default_rng(17)
    c = p.cache
    tiny = O.storage_round(2.0 ** -80 * 1.5, "bf16")
    sub = float(np.array([1 << 16], np.uint32).view(np.float32)[0])     # smallest bf16 subnormal
    huge = O.storage_round(2.0 ** 70 * 1.25, "bf16")
    for b in range(w.batch):
        n = c.n_seg(b)
        for kv in range(w.n_kv_heads):
            for S in rng.choice(n, 6, replace=False).tolist():
                rho = c.rho[b][kv][S].copy()
                rho[int(rng.integers(0, 64))] = tiny
                rho[int(rng.integers(0, 64))] = sub
                rho[64 + int(rng.integers(0, 64))] = huge * (1 if S % 2 else -1)
                c.rho[b][kv][S] = rho
    p.decisions = [[scores(c, p.x.q[st, b], b, w.group) > p.theta[b][:, None] for b in range(w.batch)]
                   for st in p.steps]
    dev = Device(p)
    for si in range(len(p.steps)):
        dev.route(ctx, si)
        compare_route(dev, oracle_route(p, si))


def test_route_ticket_order_on_a_grid_larger_than_the_gpu_holds(ctx):
    """64 sequences x 4 KV heads x >= 5 tiles of 256 spans: more route
    workgroups than the GPU holds at once, so tiles are taken by per-group
    tickets.  Route only (the cache holds the oracle's routing keys); every
    list bit-exact on two consecutive calls, workspace zero afterwards."""
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    w = synth.workload(1, batch=64, n_q_heads=8, n_kv_heads=4, head_dim=64, dtype="bf16", n_ctx=4096,
                       min_span=1, max_span=8, boundary_quantile=0.5, rank_lo=1, rank_hi=4)
    x = synth.make_inputs(w, n_steps=2)
    cfg = B.make_config(w)
    segs = [O.segment(x.surprisal[b], float(x.boundary_thr[b]), w.n_sink, w.n_recent, w.min_span, w.max_span)
            for b in range(w.batch)]
    plan = B.layout_from_segments(cfg, segs, [np.ones(len(so) - 1, np.int32) for so in segs])
    cache = B.SpanCache(cfg, plan)
    nblk = -(-max(len(so) - 1 for so in segs) // 256)
    assert nblk * w.n_kv_heads * w.batch >= 1280          # more than 4 workgroups per compute unit
    rho = np.zeros((w.batch, w.n_kv_heads, cache.seg_cap, w.head_dim), np.float32)
    G = w.group
    theta = np.empty((w.batch, w.n_q_heads), np.float32)
    z = {}
    for b in range(w.batch):
        for kv in range(w.n_kv_heads):
            kbar, _ = O.span_summaries(x.k[b, kv], x.v[b, kv], x.surprisal[b], segs[b])
            r = O.storage_round(O.routing_keys(kbar, x.route_proj[kv]), w.dtype)
            rho[b, kv, :len(r)] = r
            for st in range(2):
                z[(st, b, kv)] = O.route_scores(x.q[st, b, kv * G:(kv + 1) * G], r)
        zb = np.stack([np.concatenate([z[(st, b, kv)] for kv in range(w.n_kv_heads)]) for st in range(2)])
        theta[b] = synth.calibrate_theta(zb, 0.15, G)
    cache.rho.copy_(torch.from_numpy(rho).to(cache.elem))
    td = torch.from_numpy(theta).cuda()
    ro = B.RouteOut(cfg, cache.seg_cap)
    ws = B.route_workspace(cache)
    for st in range(2):
        B.route(ctx, cache, torch.from_numpy(np.ascontiguousarray(x.q[st])).to(cache.elem).cuda(), td, ro, ws)
        torch.cuda.synchronize()
        cnt, lst, msk = ro.exp_count.cpu().numpy(), ro.exp_list.cpu().numpy(), ro.exp_mask.cpu().numpy()
        for b in range(w.batch):
            dec = np.concatenate([z[(st, b, kv)] for kv in range(w.n_kv_heads)]) > theta[b][:, None]
            lists, masks = O.compact(dec, G)
            for kv in range(w.n_kv_heads):
                n = len(lists[kv])
                assert cnt[b, kv] == n
                assert lst[b, kv, :n].tolist() == lists[kv].tolist()
                assert msk[b, kv, :n].tolist() == masks[kv].tolist()
    assert int(ws.count_nonzero()) == 0
    log(f"ticket-ordered route: {nblk * w.n_kv_heads * w.batch} workgroups, lists bit-exact")


def _route_raw(ctx, w, rho, q, theta):
    """Route a hand-made set of routing keys rho [B][Hkv][n][d] (one sequence
    layout shared by the batch) with queries q [B][Hq][d] and thresholds
    theta [B][Hq]; returns (count, list, mask) on the host."""
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    cfg = B.make_config(w)
    n = rho.shape[2]
    L = w.min_span
    so = np.arange(w.n_sink, w.n_sink + (n + 1) * (L + 1), L + 1, dtype=np.int64)
    assert so[-1] == w.n_ctx - w.n_recent
    segs = [so] * w.batch
    plan = B.layout_from_segments(cfg, segs, [np.ones(n, np.int32)] * w.batch)
    cache = B.SpanCache(cfg, plan)
    full = np.zeros((w.batch, w.n_kv_heads, cache.seg_cap, w.head_dim), np.float32)
    full[:, :, :n] = rho
    cache.rho.copy_(torch.from_numpy(full).to(cache.elem))
    ro = B.RouteOut(cfg, cache.seg_cap)
    ws = B.route_workspace(cache)
    B.route(ctx, cache, torch.from_numpy(np.ascontiguousarray(q, np.float32)).to(cache.elem).cuda(),
            torch.from_numpy(np.ascontiguousarray(theta, np.float32)).cuda(), ro, ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    return ro.exp_count.cpu().numpy(), ro.exp_list.cpu().numpy(), ro.exp_mask.cpu().numpy()


def test_route_keeps_separate_rounding_where_fused_steps_would_differ(ctx):
    """Two tiles hold spans on which a fused multiply-add chain and the
    canonical chain (separately rounded products) decide differently, and
    thresholds sit exactly on the canonical score:
      - a product below the subnormal grid: 2^-16 * 3*2^-133 = 3*2^-149, then
        2^-17 * 2^-133 = 2^-150, which rounds to 0 on its own (ties to even)
        but carries 3.5*2^-149 -> 4*2^-149 inside a fused step;
      - an overflowing product: -1.5*2^64 * 2^63 = -1.5*2^127, then
        2^64 * 2^64 = 2^128, which overflows to +inf on its own but cancels
        to 2^126 inside a fused step.
    A third tile holds ordinary keys.  Every decision must equal the oracle's
    separately rounded chain."""
    import warnings
    n = 700                                      # three tiles of 256 spans of length 2
    w = synth.workload(2, batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, dtype="bf16",
                       n_ctx=4 + 3 * n + 256, n_sink=4, n_recent=256, min_span=2, max_span=8)
    G, d = w.group, w.head_dim
    rng = np.random.default_rng(31)
    rho = O.storage_round(rng.standard_normal((w.batch, w.n_kv_heads, n, d)) / 8, "bf16")
    q = O.storage_round(rng.standard_normal((w.batch, w.n_q_heads, d)), "bf16")
    theta = np.zeros((w.batch, w.n_q_heads), np.float32)
    # sequence 0: sub-grid products in group 0 tile 1 (span 300) and group 1
    # tile 0 (span 5); the queries are zero past their first two entries, so
    # the other keys of those spans (tiny, nonzero) add exact zeros
    q[0, :, :2] = [2.0 ** -16, 2.0 ** -17]
    q[0, :, 2:] = 0.0
    for kv, S in ((0, 300), (1, 5)):
        rho[0, kv, S, :2] = [3 * 2.0 ** -133, 2.0 ** -133]
        rho[0, kv, S, 2:] = 2.0 ** -120
    # sequence 1: overflow with cancellation in group 1 tile 2 (span 650)
    q[1, :, :2] = [-1.5 * 2.0 ** 64, 2.0 ** 64]
    rho[1, 1, 650] = 0.0
    rho[1, 1, 650, :2] = [2.0 ** 63, 2.0 ** 64]
    with warnings.catch_warnings():
        warnings.simplefilter("ignore", RuntimeWarning)     # the canonical overflow to inf
        z = np.stack([np.concatenate([O.route_scores(q[b, kv * G:(kv + 1) * G], rho[b, kv])[:, None, :]
                                      for kv in range(w.n_kv_heads)], 1) for b in range(w.batch)])
    # z [B][G][Hkv][n]; the planted spans' canonical scores, and what a fused
    # chain would give there (exact sums in float64, one rounding to float32)
    assert (z[0, :, 0, 300] == np.float32(3 * 2.0 ** -149)).all() and (z[0, :, 1, 5] == z[0, :, 0, 300]).all()
    assert np.float32(3.5 * 2.0 ** -149) == np.float32(4 * 2.0 ** -149)
    assert np.isinf(z[1, :, 1, 650]).all() and (z[1, :, 1, 650] > 0).all()
    assert np.float32(-1.5 * 2.0 ** 127 + 2.0 ** 128) == np.float32(2.0 ** 126) < np.float32(3e38)
    # thresholds: on the canonical sub-grid score (fused would be above it),
    # and between the fused and canonical overflow results
    theta[0, :] = np.float32(3 * 2.0 ** -149)
    theta[1, :] = rng.standard_normal(w.n_q_heads).astype(np.float32)
    theta[1, G:2 * G] = np.float32(3e38)
    cnt, lst, msk = _route_raw(ctx, w, rho, q, theta)
    for b in range(w.batch):
        dec = np.concatenate([z[b, :, kv] for kv in range(w.n_kv_heads)]) > theta[b][:, None]
        lists, masks = O.compact(dec, G)
        for kv in range(w.n_kv_heads):
            m = len(lists[kv])
            assert cnt[b, kv] == m, (b, kv)
            assert lst[b, kv, :m].tolist() == lists[kv].tolist()
            assert msk[b, kv, :m].tolist() == masks[kv].tolist()
    assert 650 in lst[1, 1, :cnt[1, 1]].tolist()            # +inf > 3e38: expanded
    assert 300 not in lst[0, 0, :cnt[0, 0]].tolist()        # z == theta: not expanded
    log("route: sub-grid and overflowing products bit-exact")


def test_decode_step_in_a_hip_graph_replays_like_eager(ctx):
    """sekv_decode_step captured into a HIP graph (its second stream forks
    from and joins the capture stream): several replays, with eager library
    work and host synchronisation between them, each bit-identical to the
    eager call of the same step."""
    import torch
    p = _prep("bf16-d128-T4K")
    dev = Device(p)
    stream = torch.cuda.Stream()
    want = []
    for si in range(len(p.steps)):
        with torch.cuda.stream(stream):
            dev.step(ctx, si, stream=stream)
        torch.cuda.synchronize()
        want.append((dev.out.clone(), dev.route_numpy()))
    q0 = dev.q(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        dev.step(ctx, 0, stream=stream, q=q0)
    torch.cuda.synchronize()
    for rep in range(4):
        dev.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dev.out, want[0][0]), rep
        cnt, lst, msk = dev.route_numpy()
        assert np.array_equal(cnt, want[0][1][0])
        # eager work between replays: the other step, eagerly
        with torch.cuda.stream(stream):
            dev.step(ctx, len(p.steps) - 1, stream=stream)
        torch.cuda.synchronize()
        assert torch.equal(dev.out, want[-1][0])
    assert int(dev.route_ws.count_nonzero()) == 0
    log("decode_step: 4 graph replays bit-identical to eager")


@pytest.mark.parametrize("mode", ["plus_inf", "minus_inf"])
def test_infinite_thresholds(ctx, mode):
    import torch
    w = synth.workload(2, n_ctx=3000, batch=2, rank_lo=2, rank_hi=40)
    p = prepare(w, [0], theta_mode=mode)
    dev = Device(p)
    dev.route(ctx, 0)
    cnt, lst, msk = dev.route_numpy()
    for b in range(w.batch):
        n = p.cache.n_seg(b)
        if mode == "plus_inf":
            assert np.all(cnt[b] == 0)
        else:
            assert np.all(cnt[b] == n)
            assert np.array_equal(lst[b, :, :n], np.tile(np.arange(n), (w.n_kv_heads, 1)))
            assert np.all(msk[b, :, :n] == (1 << w.group) - 1)
    dev.decode(ctx, 0)
    torch.cuda.synchronize()
    out = dev.out.cpu().numpy()
    want = oracle_out(p, 0)
    err = max(float(np.abs(out[b] - want[b]).max()) for b in want)
    log(f"theta {mode}: max|err|={err:.3e}")
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_full_expansion_full_rank_equals_dense(ctx, dtype):
    """Every span expanded at full rank with unit gates reduces to dense
    softmax attention over the stored K/V."""
    import torch
    w = synth.workload(5, n_ctx=4096, batch=2, dtype=dtype)
    p = prepare(w, [0, 1], full_rank=True, theta_mode="minus_inf")
    dev = Device(p)
    for si in range(2):
        dev.route(ctx, si)
        dev.decode(ctx, si)
        torch.cuda.synchronize()
        out = dev.out.cpu().numpy()
        for b in range(w.batch):
            dense = O.dense_attention(p.x.q[p.steps[si], b], p.x.k[b], p.x.v[b], w.group)
            err = float(np.abs(out[b] - dense).max())
            log(f"full expansion {dtype} b={b}: max|gpu - dense|={err:.3e}")
            # bf16-stored factors reconstruct to ~1e-2 relative; fp32 to ~1e-6
            assert err <= (2e-2 if dtype == "bf16" else 1e-4)


@pytest.mark.parametrize("basis", ["joint", "separate"])
def test_host_resident_factors_match_device_resident_bitwise(ctx, basis):
    """Staged fetch (host gather + copy): same factor bits as the
    device-resident path, so the same output bits."""
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    w = synth.workload(3, n_ctx=8192, basis=basis)
    p = prepare(w, [0, 1])
    dev_d = Device(p, factors_on_host=False)
    side = torch.cuda.Stream()
    try:
        ctx.set_fetch_mode(B.SEKV_FETCH_STAGED)
        dev_h = Device(p, factors_on_host=True, ctx=ctx)
        for si in range(2):
            dev_d.route(ctx, si)
            dev_d.decode(ctx, si)
            dev_h.route(ctx, si)
            dev_h.decode(ctx, si, copy_stream=side)
            torch.cuda.synchronize()
            assert torch.equal(dev_d.out, dev_h.out)
            want = oracle_out(p, si)
            out = dev_h.out.cpu().numpy()
            assert max(float(np.abs(out[b] - want[b]).max()) for b in want) <= TOL[w.dtype]
    finally:
        ctx.set_fetch_mode(B.SEKV_FETCH_DIRECT)


@pytest.mark.parametrize("basis", ["joint", "separate"])
def test_reconstruct_matches_oracle(ctx, basis):
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    w = synth.workload(2, n_ctx=3000, batch=2, rank_lo=1, rank_hi=40, basis=basis)
    p = prepare(w, [0], frac=0.2)
    dev = Device(p)
    dev.route(ctx, 0)
    tok_off, k_out, v_out = B.reconstruct(ctx, dev.cache, dev.route_out)
    torch.cuda.synchronize()
    cnt, lst, _ = dev.route_numpy()
    to = tok_off.cpu().numpy()
    K = k_out.cpu().numpy()
    V = v_out.cpu().numpy()
    worst = 0.0
    for b in range(w.batch):
        L = p.cache.span_len(b)
        for kv in range(w.n_kv_heads):
            n = int(cnt[b, kv])
            assert to[b, kv, 0] == 0 and to[b, kv, n] == int(L[lst[b, kv, :n]].sum())
            for j in range(n):
                S = int(lst[b, kv, j])
                kh, vh = O.reconstruct_span(p.cache, b, kv, S)
                r0 = int(to[b, kv, j])
                worst = max(worst, float(np.abs(K[b, kv, r0:r0 + L[S]] - kh).max()),
                            float(np.abs(V[b, kv, r0:r0 + L[S]] - vh).max()))
    log(f"reconstruct max|err|={worst:.3e}")
    assert worst <= 1e-4


def test_split_invariance(ctx):
    """The result does not depend on how the memory is cut into split-K chunks,
    up to rounding: with a bfloat16 cache the softmax weights enter the P.V
    matrix-core product rounded to bfloat16 (relative 2^-9) after subtracting a
    running maximum that depends on the split, so outputs (|o| < 4 here) may
    move by a few 2^-9 * |v| ulps; 2e-3 bounds that, 10x under the parity
    tolerance."""
    import torch
    p = _prep("bf16-ragged-B3-T4K")
    outs = []
    try:
        for chunk in (128, 512, 2048):
            ctx.set_split(chunk)
            dev = Device(p, ctx=ctx)
            dev.route(ctx, 0)
            dev.decode(ctx, 0)
            torch.cuda.synchronize()
            outs.append(dev.out.cpu().numpy())
    finally:
        ctx.set_split(0)
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 2e-3


def test_host_resident_direct_fetch_matches_device_resident_bitwise(ctx):
    """Direct fetch: the kernels read the pinned host pools over the bus.  Same
    kernels and same factor bits as the device-resident path, so the same
    output bits; graph capture needs no host wait in this mode."""
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    w = synth.workload(3, n_ctx=8192)
    p = prepare(w, [0, 1])
    dev_d = Device(p, factors_on_host=False)
    try:
        ctx.set_fetch_mode(B.SEKV_FETCH_DIRECT)      # the default
        dev_h = Device(p, factors_on_host=True, ctx=ctx)
        assert dev_h.dec_ws.host is None
        for si in range(2):
            dev_d.route(ctx, si)
            dev_d.decode(ctx, si)
            dev_h.route(ctx, si)
            dev_h.decode(ctx, si)
            torch.cuda.synchronize()
            assert torch.equal(dev_d.out, dev_h.out)
    finally:
        ctx.set_fetch_mode(B.SEKV_FETCH_DIRECT)


def test_injected_gather_fault_leaves_out_untouched_and_context_usable(ctx):
    """A forced failure of the staged host gather (set from the host, after the
    one host wait) returns SEKV_EHIP without writing `out`; the next call on
    the same context and workspace gives the normal result."""
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    w = synth.workload(3, n_ctx=8192)
    p = prepare(w, [0])
    dev_d = Device(p, factors_on_host=False)
    dev_d.route(ctx, 0)
    dev_d.decode(ctx, 0)
    side = torch.cuda.Stream()
    try:
        ctx.set_fetch_mode(B.SEKV_FETCH_STAGED)
        dev_h = Device(p, factors_on_host=True, ctx=ctx)
        dev_h.route(ctx, 0)
        sentinel = torch.full_like(dev_h.out, -7.0)
        dev_h.out.copy_(sentinel)
        torch.cuda.synchronize()
        ctx.inject_fault(B.SEKV_FAULT_GATHER)
        with pytest.raises(B.SekvError) as ei:
            dev_h.decode(ctx, 0, copy_stream=side)
        assert ei.value.status == B.SEKV_EHIP and "injected" in str(ei.value)
        torch.cuda.synchronize()
        assert torch.equal(dev_h.out, sentinel)
        dev_h.decode(ctx, 0, copy_stream=side)
        torch.cuda.synchronize()
        assert torch.equal(dev_h.out, dev_d.out)
    finally:
        ctx.set_fetch_mode(B.SEKV_FETCH_DIRECT)


@pytest.mark.parametrize("variant", ["default", "variants"])
def test_library_build_matches_oracle_build(ctx, variant):
    """sekv_plan_spans + sekv_build_spans against the oracle's build: offsets
    and ranks exact; summaries, routing keys and key scales within one storage
    rounding; fold matrices within fp64 rounding; factors through their
    invariants (orthonormality, singular values, reconstruction error = tail
    energy), per part for separate bases."""
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    if variant == "default":
        wls = [synth.workload(1), synth.workload(2, n_ctx=4096, batch=2)]
    else:
        wls = [synth.workload(1, rank_cap="half", basis="separate", route_keys="folded"),
               synth.workload(2, n_ctx=4096, batch=2, basis="separate", route_keys="folded"),
               synth.workload(5, n_ctx=4096, batch=1, rank_cap="half")]
    for w in wls:
        sep = w.basis == "separate"
        x = synth.make_inputs(w, n_steps=1)
        cfg = B.make_config(w)
        plan = B.plan_spans(cfg, x.surprisal, x.boundary_thr, x.rank_req)
        cache = B.SpanCache(cfg, plan)
        et = cache.elem
        kd = torch.from_numpy(x.k).to(et).cuda()
        vd = torch.from_numpy(x.v).to(et).cuda()
        B.build_spans(ctx, cache, kd, vd, x.surprisal, x.route_proj, x.gate)
        torch.cuda.synchronize()
        oc = O.build_cache(x.k, x.v, x.surprisal, x.boundary_thr, x.route_proj, x.rank_req, x.gate,
                           n_sink=w.n_sink, n_recent=w.n_recent, lo=w.min_span, hi=w.max_span, dtype=w.dtype,
                           rank_cap=w.rank_cap, basis=w.basis)
        rel = 2.0 ** -7 if w.dtype == "bf16" else 2.0 ** -22
        fk = cache.full_k.float().cpu().numpy()
        sk = cache.sum_k.float().cpu().numpy()
        sv = B.untile_values(cache.sum_v.float().cpu().numpy(), cache.seg_cap)
        fv = B.untile_values(cache.full_v.float().cpu().numpy(), cache.full_cap)
        rh = cache.rho.float().cpu().numpy()
        ks = cache.key_scale.cpu().numpy()
        fold = cache.fold.cpu().numpy()
        for kv in range(w.n_kv_heads):
            assert np.allclose(fold[kv], oc.fold[kv], rtol=1e-12, atol=1e-14)
        worst_recon = 0.0
        utol = 0.05 if w.dtype == "bf16" else 1e-5
        for b in range(w.batch):
            n = oc.n_seg(b)
            assert int(plan.n_seg[b]) == n
            assert plan.seg_off[b, :n + 1].tolist() == oc.seg_off[b].tolist()
            assert plan.rank[b, :n].tolist() == oc.rank[b].tolist()
            for kv in range(w.n_kv_heads):
                nf = len(oc.full_idx[b])
                assert np.array_equal(fk[b, kv, :nf], oc.full_k[b][kv])
                assert np.array_equal(fv[b, kv, :nf], oc.full_v[b][kv])
                for arr, ref in ((sk, oc.sum_k), (sv, oc.sum_v), (rh, oc.rho)):
                    r = ref[b][kv]
                    assert np.all(np.abs(arr[b, kv, :n] - r) <= rel * np.abs(r) + 1e-30)
                assert np.allclose(ks[b, kv, :n], oc.key_scale[b][kv], rtol=2.0 ** -22, atol=0)
                for i in range(0, n, max(1, n // 40)):
                    rk = int(plan.rank[b, i])
                    t0, t1 = oc.seg_off[b][i] + 1, oc.seg_off[b][i + 1]
                    got = B.read_factors(cache, b, kv, i)
                    if sep:
                        parts = [(got[0], x.k[b, kv, t0:t1], oc.U[b][kv][i], oc.sigma[b][kv][i], oc.Vh[b][kv][i]),
                                 (got[1], x.v[b, kv, t0:t1], oc.U_V[b][kv][i], oc.sigma_V[b][kv][i],
                                  oc.Vh_V[b][kv][i])]
                    else:
                        parts = [(got, np.concatenate([x.k[b, kv, t0:t1], x.v[b, kv, t0:t1]], axis=1), oc.U[b][kv][i],
                                  oc.sigma[b][kv][i], oc.Vh[b][kv][i])]
                    for (U, sig, gt, Vh), M, Uo, so_, Vo in parts:
                        assert np.allclose(sig, so_, rtol=1e-5, atol=1e-6)
                        assert np.array_equal(gt, oc.gate[b][kv][i].astype(np.float32))
                        assert np.allclose(U.T @ U, np.eye(rk), atol=utol)
                        assert np.allclose(Vh @ Vh.T, np.eye(rk), atol=utol)
                        M = M.astype(np.float64)
                        e_lib = np.linalg.norm(M - (U * sig) @ Vh)
                        e_orc = np.linalg.norm(M - (np.asarray(Uo) * so_) @ np.asarray(Vo))
                        worst_recon = max(worst_recon, abs(e_lib - e_orc) / max(np.linalg.norm(M), 1e-30))
        log(f"build {w.name} ({w.rank_cap}, {w.basis}, {w.route_keys}): worst relative reconstruction-error gap "
            f"{worst_recon:.2e}")
        assert worst_recon <= (2e-2 if w.dtype == "bf16" else 1e-5)


@pytest.mark.parametrize("wid,over", [(1, {}), (2, dict(n_ctx=4096, batch=2)),
                                      (1, dict(max_span=120, boundary_quantile=0.995, route_keys="folded"))])
def test_device_build_matches_host_build(ctx, wid, over):
    """sekv_build_spans in build mode DEVICE (GPU kernels) against build mode
    HOST (host threads): full-resolution rows, summaries, routing keys and key
    scales bit for bit (same fp64 operation order); factors (Gram-matrix
    Jacobi against one-sided Jacobi) through their reconstructions, which
    agree within a storage rounding.  The third case has forced spans longer
    than the eigenvectors kept in LDS."""
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    w = synth.workload(wid, **over)
    x = synth.make_inputs(w, n_steps=1)
    cfg = B.make_config(w)
    plan = B.plan_spans(cfg, x.surprisal, x.boundary_thr, x.rank_req)
    et = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    kd = torch.from_numpy(x.k).to(et).cuda()
    vd = torch.from_numpy(x.v).to(et).cuda()
    caches = []
    for mode in (B.SEKV_BUILD_DEVICE, B.SEKV_BUILD_HOST):
        c = B.SpanCache(cfg, plan)
        ctx.set_build_mode(mode)
        B.build_spans(ctx, c, kd, vd, x.surprisal, x.route_proj, x.gate)
        caches.append(c)
    ctx.set_build_mode(B.SEKV_BUILD_DEVICE)
    torch.cuda.synchronize()
    dev, host = caches
    for name in ("full_k", "full_v", "sum_k", "sum_v", "rho", "key_scale", "fold"):
        assert torch.equal(getattr(dev, name), getattr(host, name)), name
    Lmax = int(max((plan.seg_off[b, 1:plan.n_seg[b] + 1] - plan.seg_off[b, :plan.n_seg[b]] - 1).max()
                   for b in range(w.batch)))
    tol = 2.0 ** -7 if w.dtype == "bf16" else 1e-5
    worst = 0.0
    for b in range(w.batch):
        n = int(plan.n_seg[b])
        for kv in range(w.n_kv_heads):
            for i in range(0, n, max(1, n // 60)):
                U1, s1, g1, V1 = B.read_factors(dev, b, kv, i)
                U2, s2, g2, V2 = B.read_factors(host, b, kv, i)
                assert np.array_equal(g1, g2)
                R1, R2 = (U1 * s1) @ V1, (U2 * s2) @ V2
                worst = max(worst, float(np.abs(R1 - R2).max() / max(np.abs(R2).max(), 1e-30)))
    log(f"device vs host build ({w.name}, L up to {Lmax}): factors' reconstructions differ by {worst:.2e} relative")
    assert worst <= tol


def test_abi_errors_need_context(ctx):
    """Argument checks of the GPU entry points: documented status, nothing written."""
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    p = _prep("tiny-f32-T2K")
    dev = Device(p)
    dev.route(ctx, 0)
    torch.cuda.synchronize()
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.SekvError) as ei:
        B.route(ctx, dev.cache, dev.q(0), dev.theta, dev.route_out, small)
    assert ei.value.status == B.SEKV_ECAPACITY
    sentinel = torch.full_like(dev.out, 123.0)
    dev.out.copy_(sentinel)
    ws = B.DecodeWorkspace(dev.cache)
    ws.dev = ws.dev[:64]
    with pytest.raises(B.SekvError) as ei:
        B.decode(ctx, dev.cache, dev.q(0), dev.route_out, dev.out, ws)
    assert ei.value.status == B.SEKV_ECAPACITY
    torch.cuda.synchronize()
    assert torch.equal(dev.out, sentinel)
    # host-resident mode with pageable pools is refused
    cfg_h = B.make_config(p.w, True)
    st = dev.cache.struct()
    with pytest.raises(B.SekvError) as ei:
        import ctypes
        B._check(B.LIB.sekv_mixed_attention_decode(ctx.handle, ctypes.byref(cfg_h), ctypes.byref(st),
                                                   B._ptr(dev.q(0)), B._ptr(dev.route_out.exp_list),
                                                   B._ptr(dev.route_out.exp_mask), B._ptr(dev.route_out.exp_count),
                                                   B._ptr(dev.out), B._ptr(ws.dev), 1 << 40, None, 0, None, None))
    assert ei.value.status == B.SEKV_EINVAL and "pinned" in str(ei.value)
    # null query
    with pytest.raises(B.SekvError) as ei:
        import ctypes
        B._check(B.LIB.sekv_route(ctx.handle, ctypes.byref(dev.cfg), ctypes.byref(st), None, B._ptr(dev.theta),
                                  B._ptr(dev.route_out.exp_list), B._ptr(dev.route_out.exp_mask),
                                  B._ptr(dev.route_out.exp_count), B._ptr(dev.route_ws), dev.route_ws.numel(), None))
    assert ei.value.status == B.SEKV_EINVAL
    torch.cuda.synchronize()
    assert torch.equal(dev.out, sentinel)


@pytest.mark.parametrize("dtype,T,G,d", [("bf16", 4113, 4, 128), ("f32", 3000, 2, 64), ("bf16", 70, 8, 64)])
def test_dense_baseline_matches_oracle(ctx, dtype, T, G, d):
    """The dense flash-decode baseline (all T tokens, no spans) against the
    oracle's dense softmax attention; ragged last tile."""
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    w = synth.workload(2, n_ctx=T, batch=2, dtype=dtype, n_q_heads=2 * G, n_kv_heads=2, head_dim=d,
                       n_recent=min(64, T - 4))
    x = synth.make_inputs(w, n_steps=1)
    cfg = B.make_config(w)
    et = torch.bfloat16 if dtype == "bf16" else torch.float32
    k = torch.from_numpy(x.k).to(et).cuda()
    vt = B.tile_values_device(torch.from_numpy(x.v).to(et).cuda())
    q = torch.from_numpy(np.ascontiguousarray(x.q[0])).to(et).cuda()
    out = torch.zeros((w.batch, w.n_q_heads, d), dtype=torch.float32, device="cuda")
    B.dense_decode(ctx, cfg, k, vt, q, out, B.dense_workspace(ctx, cfg))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    err = max(float(np.abs(got[b] - O.dense_attention(x.q[0, b], x.k[b], x.v[b], G)).max()) for b in range(w.batch))
    log(f"dense baseline {dtype} T={T} G={G} d={d}: max|err|={err:.3e}")
    assert err <= TOL[dtype]
