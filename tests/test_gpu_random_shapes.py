"""Property test over tiny random shapes: route + mixed attention through the
C ABI against the oracle, on configurations drawn at random within the
library's limits (batch, group size, KV heads, head dim, dtype, context, sink,
recent window, span bounds, rank range, expansion fraction, reading variants).

Properties checked on every draw and step: the expanded set (count, ascending
list, head masks) equals the oracle's bit for bit, and every output is within
the dtype's tolerance of the oracle.  Each case is printed before its GPU work
so that a failure names its configuration.
"""
import numpy as np
import pytest

from hierarchical_kv_cache_sekv_amd import synth

from _harness import TOL, Device, compare_route, log, oracle_out, oracle_route, prepare

pytestmark = pytest.mark.gpu

N_CASES = 24


def draw(seed):
    rng = np.random.default_rng([2026, seed])
    dtype = str(rng.choice(["f32", "bf16"]))
    d = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.integers(1, 3))
    B = int(rng.integers(1, 4))
    T = int(rng.integers(8, 600))
    n_sink = int(rng.integers(0, 6))
    n_recent = int(rng.integers(1, 48))
    n_recent = min(n_recent, T - n_sink)
    lo = int(rng.integers(1, 6))
    hi = int(rng.integers(lo, 100))
    rlo = int(rng.integers(1, 8))
    rhi = int(rng.integers(rlo, 96 if rng.random() < 0.25 else 40))
    frac = float(rng.choice([0.0, 0.1, 0.3, 0.7, 1.0]))
    over = dict(batch=B, n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=d, dtype=dtype, n_ctx=T, n_sink=n_sink,
                n_recent=n_recent, min_span=lo, max_span=hi, rank_lo=rlo, rank_hi=rhi,
                boundary_quantile=float(rng.choice([0.8, 0.9, 0.97])))
    if rng.random() < 0.3:
        over["rank_cap"] = "half"
    if rng.random() < 0.3:
        over["basis"] = "separate"
    if rng.random() < 0.3:
        over["route_keys"] = "folded"
    return synth.workload(1 if dtype == "f32" else 2, **over), frac


@pytest.fixture(scope="module")
def ctx():
    from hierarchical_kv_cache_sekv_amd import binding as B
    c = B.Context(0)
    yield c
    c.close()


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_tiny_shape(ctx, seed):
    import torch
    w, frac = draw(seed)
    log(f"case {seed}: B={w.batch} Hq/Hkv={w.n_q_heads}/{w.n_kv_heads} d={w.head_dim} {w.dtype} T={w.n_ctx} "
        f"sink={w.n_sink} recent={w.n_recent} span={w.min_span}..{w.max_span} ranks={w.rank_lo}..{w.rank_hi} "
        f"q={w.boundary_quantile} f={frac} {w.rank_cap}/{w.basis}/{w.route_keys}")
    p = prepare(w, [0, 1], frac=frac)
    dev = Device(p)
    for si in range(2):
        dev.route(ctx, si)
        compare_route(dev, oracle_route(p, si))
        dev.decode(ctx, si)
        torch.cuda.synchronize()
        out = dev.out.cpu().numpy()
        want = oracle_out(p, si)
        err = max(float(np.abs(out[b] - want[b]).max()) for b in want)
        assert err <= TOL[w.dtype], (seed, si, err)
