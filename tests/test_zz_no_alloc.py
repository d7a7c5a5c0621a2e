"""sekv_route_noalloc, the route entry point for callers that cannot allocate
(its state lives in the library's static device array), against sekv_route:
two calls in a row on one context, the second with a smaller input; count,
list and head masks must be bit-identical to sekv_route's and to the
oracle's.  A configuration whose route state exceeds the static array is
refused before anything runs."""
import ctypes

import numpy as np
import pytest

from hierarchical_kv_cache_sekv_amd import synth
from _harness import Device, log, oracle_route, prepare

pytestmark = pytest.mark.gpu


def _route_arrays(out):
    return out.exp_count.cpu().numpy(), out.exp_list.cpu().numpy(), out.exp_mask.cpu().numpy()


def _same_route(a, b):
    ca, la, ma = a
    cb, lb, mb = b
    assert np.array_equal(ca, cb), (ca, cb)
    for bb in range(ca.shape[0]):
        for kv in range(ca.shape[1]):
            n = int(ca[bb, kv])
            assert np.array_equal(la[bb, kv, :n], lb[bb, kv, :n]), (bb, kv)
            assert np.array_equal(ma[bb, kv, :n], mb[bb, kv, :n]), (bb, kv)


def test_route_noalloc_matches_route_on_consecutive_calls():
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    assert torch.cuda.is_available()
    ctx = B.Context(0)
    try:
        # the second call has a smaller input: fewer sequences, a shorter context
        for w in (synth.workload(4, n_ctx=16384, batch=3), synth.workload(2, n_ctx=4096, batch=1)):
            p = prepare(w, [0])
            dev = Device(p)
            dev.route(ctx, 0)                          # sekv_route, with its own workspace
            ref = dev.route_numpy()
            out = B.RouteOut(dev.cfg, dev.cache.seg_cap)
            out.exp_count.fill_(-5)
            B.route_noalloc(ctx, dev.cache, dev.q(0), dev.theta, out)
            torch.cuda.synchronize()
            got = _route_arrays(out)
            _same_route(got, ref)
            _same_route(got, oracle_route(p, 0))
            log(f"route_noalloc {w.name} B={w.batch} T={w.n_ctx}: counts {got[0].sum()} bit-identical to sekv_route")
    finally:
        ctx.close()


def test_route_noalloc_refuses_state_beyond_the_static_array():
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    assert torch.cuda.is_available()
    ctx = B.Context(0)
    try:
        # 256 groups of spans over a 1M-token context need more route state than
        # the static array holds; nothing is read before the size check
        w = synth.workload(1, batch=64, n_q_heads=4, n_kv_heads=4, n_ctx=1 << 20, n_sink=4, n_recent=4,
                           min_span=1, max_span=8)
        cfg = B.make_config(w)
        cap, fcap = B.capacities(cfg)
        assert B.LIB.sekv_route_workspace_bytes(ctypes.byref(cfg), ctypes.byref(B.Spans(cap, fcap))) > 1 << 20
        dummy = torch.zeros(64, dtype=torch.int32, device="cuda")
        nseg = np.zeros(w.batch, np.int32)
        nfull = np.ones(w.batch, np.int32)
        p = B._ptr(dummy)
        st = B.Spans(cap, fcap, B._ptr(nseg), B._ptr(nfull), p, p, p, p, p, p, p, p, p, p, p, 0, 0,
                     None, None, None, None)
        with pytest.raises(B.SekvError) as ei:
            B._check(B.LIB.sekv_route_noalloc(ctx.handle, ctypes.byref(cfg), ctypes.byref(st), p, p, p, p, p, None))
        assert ei.value.status == B.SEKV_ECAPACITY and "static" in str(ei.value)
    finally:
        ctx.close()
