"""GPU tests of the device factor cache (sekv_cached_attention_decode).

The cached decode reads the same factor bits as the direct host fetch (hits
and fills from the HBM arena, bypasses from the pinned pools), through the
same kernels, so its output must equal the direct fetch's bit for bit on every
call: across layers sharing one cache, across steps, and while the cache
evicts and bypasses.  The direct fetch itself is checked against the oracle
in test_gpu_parity.py; one step here is also checked against the oracle.
"""
import numpy as np
import pytest

from hierarchical_kv_cache_sekv_amd import synth

from _harness import TOL, Device, log, oracle_out, prepare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    from hierarchical_kv_cache_sekv_amd import binding as B
    c = B.Context(0)
    yield c
    c.close()


class Layer:
    """One layer: a host-resident span cache (direct fetch) and the cached-decode workspace."""

    def __init__(self, ctx, p):
        import torch
        from hierarchical_kv_cache_sekv_amd import binding as B
        self.B = B
        self.dev = Device(p, factors_on_host=True, ctx=ctx)
        self.ws = B.CachedDecodeWorkspace(self.dev.cache, ctx=ctx)
        self.out_c = torch.zeros_like(self.dev.out)

    def run(self, ctx, fc, layer, si, side):
        import torch
        d = self.dev
        d.route(ctx, si)
        d.decode(ctx, si)                      # direct fetch
        self.B.cached_decode(ctx, fc, layer, d.cache, d.q(si), d.route_out, self.out_c, self.ws, copy_stream=side)
        torch.cuda.synchronize()
        return int(d.route_out.exp_count.sum().item())


def test_cached_decode_matches_direct_fetch_bitwise_across_layers_and_steps(ctx):
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    steps = list(range(6))
    layers = [Layer(ctx, prepare(synth.workload(3, n_ctx=8192), steps)),
              Layer(ctx, prepare(synth.workload(3, n_ctx=6000, rank_lo=4, rank_hi=24), steps))]
    side = torch.cuda.Stream()
    fc = B.FactorCache(ctx, 3 * B.CACHE_PAGE_BYTES, partitions=2)    # small: evictions and bypasses
    listed = 0
    for si in steps:
        for li, L in enumerate(layers):
            log(f"cached decode: step {si} layer {li}")
            listed += L.run(ctx, fc, li, si, side)
            assert torch.equal(L.out_c, L.dev.out), (si, li)
    st = fc.stats()
    log(f"cache stats: {st}")
    assert st["lookups"] == listed == st["hits"] + st["fills"] + st["bypasses"]
    assert st["hits"] > 0 and st["fills"] > 0 and st["evictions"] > 0 and st["bypasses"] > 0
    # one step against the oracle
    want = oracle_out(layers[0].dev.p, 5)
    out = layers[0].out_c.cpu().numpy()
    err = max(float(np.abs(out[b] - want[b]).max()) for b in want)
    assert err <= TOL["bf16"]
    fc.close()


def test_a_repeated_step_is_served_from_the_cache(ctx):
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    L = Layer(ctx, prepare(synth.workload(3, n_ctx=8192), [0, 1]))
    fc = B.FactorCache(ctx, 64 * B.CACHE_PAGE_BYTES)
    n = L.run(ctx, fc, 0, 0, None)
    first = L.out_c.clone()
    s1 = fc.stats(reset=True)
    assert s1["fills"] == n and s1["hits"] == 0
    L.out_c.fill_(-3.0)
    L.run(ctx, fc, 0, 0, None)
    s2 = fc.stats(reset=True)
    assert s2["hits"] == n and s2["fills"] == 0 and s2["bytes_hit"] == s1["bytes_filled"]
    assert torch.equal(L.out_c, first) and torch.equal(L.out_c, L.dev.out)
    # another layer index under the same cache: its own blocks
    L.run(ctx, fc, 3, 0, None)
    assert fc.stats()["fills"] == n
    # after invalidating layer 0 its blocks are fetched again, with the same result
    fc.invalidate(0)
    L.run(ctx, fc, 0, 1, None)
    assert torch.equal(L.out_c, L.dev.out)
    fc.close()


def test_cached_decode_argument_errors(ctx):
    import torch
    from hierarchical_kv_cache_sekv_amd import binding as B
    L = Layer(ctx, prepare(synth.workload(3, n_ctx=4096), [0]))
    d = L.dev
    d.route(ctx, 0)
    torch.cuda.synchronize()
    no_arena = B.FactorCache(None, B.CACHE_PAGE_BYTES, partitions=1)
    with pytest.raises(B.SekvError) as e:
        B.cached_decode(ctx, no_arena, 0, d.cache, d.q(0), d.route_out, L.out_c, L.ws)
    assert e.value.status == B.SEKV_EINVAL
    fc = B.FactorCache(ctx, B.CACHE_PAGE_BYTES, partitions=1)
    with pytest.raises(B.SekvError):
        B.cached_decode(ctx, fc, 70000, d.cache, d.q(0), d.route_out, L.out_c, L.ws)
    dev_d = Device(d.p, factors_on_host=False)
    ws_d = B.CachedDecodeWorkspace(dev_d.cache, ctx=ctx)
    with pytest.raises(B.SekvError) as e:
        B.cached_decode(ctx, fc, 0, dev_d.cache, d.q(0), d.route_out, L.out_c, ws_d)
    assert e.value.status == B.SEKV_EINVAL
    assert fc.stats()["lookups"] == 0
    fc.close()
    no_arena.close()
