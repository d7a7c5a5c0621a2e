"""Pins of the oracle's online span sealing (sealed_segment, seal_next,
build_cache(sealed=True)) against things other than the functions themselves:
brute force over every longer context (a sealed head is never revised), the
step-by-step sealing against the direct statement at every context length, a
hand-worked example, span-for-span equality with the cache of a longer
prefill, and the dense-attention special case."""
import math

import numpy as np
import pytest

import oracle as O


def _params(rng):
    n_sink = int(rng.integers(0, 4))
    n_recent = int(rng.integers(1, 9))
    lo = int(rng.integers(1, 5))
    hi = lo + int(rng.integers(0, 8))
    return n_sink, n_recent, lo, hi


def test_sealing_golden():
    # a = 1, n_recent = 2, lo = 2, hi = 4, thr = 5.  At T = 14 (e = 12) the
    # prefill heads are 1, 6 (forced: body 2..5 reached 4) and 11 (forced),
    # 11 = e - 1 is handed back to the tail: seg_off [1, 6, 11].  Decided
    # tokens are t <= e - 1 - lo = 9, so only the span (1, 6) is sealed and
    # the tail starts at 6.  Token 10 (T = 15) is no head (body 3, s = 0);
    # token 11 (T = 16) is a forced head and seals the span (6, 11).
    s = np.zeros(20)
    s[3] = s[6] = 9.0
    args = (5.0, 1, 2, 2, 4)
    assert O.segment(s[:14], *args).tolist() == [1, 6, 11]
    assert O.sealed_segment(s[:14], *args).tolist() == [1, 6]
    assert O.seal_next([1, 6], s[:15], *args).tolist() == [1, 6]
    assert O.seal_next([1, 6], s[:16], *args).tolist() == [1, 6, 11]
    assert O.sealed_segment(s[:16], *args).tolist() == [1, 6, 11]
    # too short to decide anything: every token full resolution, tail at the sink
    assert O.sealed_segment(s[:6], *args).tolist() == [1]


@pytest.mark.parametrize("seed", range(12))
def test_sealed_heads_are_never_revised(seed):
    """Brute force: every sealed head of a context, with all heads before it,
    is a head of the prefill segmentation of every longer context."""
    rng = np.random.default_rng(seed)
    n_sink, n_recent, lo, hi = _params(rng)
    Tmax = int(rng.integers(30, 90))
    s = rng.lognormal(0, 1, Tmax)
    thr = float(np.quantile(s, rng.uniform(0.5, 0.95)))
    for T in range(n_sink + n_recent, Tmax + 1):
        e = T - n_recent
        so = O.sealed_segment(s[:T], thr, n_sink, n_recent, lo, hi)
        sealed = [h for h in so.tolist() if h <= e - 1 - lo]      # decided heads (none: tail from the sink)
        assert so.tolist() == (sealed or [n_sink])
        for T2 in range(T, Tmax + 1):
            full = O.segment(s[:T2], thr, n_sink, n_recent, lo, hi)[:-1].tolist()
            assert full[:len(sealed)] == sealed, (T, T2, sealed, full)
        # and it is the longest such prefix the rule could still change: the
        # next prefill head at T (if any) lies past the decided tokens
        full_T = O.segment(s[:T], thr, n_sink, n_recent, lo, hi)[:-1].tolist()
        assert all(h > e - 1 - lo for h in full_T[len(sealed):])


@pytest.mark.parametrize("seed", range(12))
def test_sealing_one_token_at_a_time_equals_the_direct_layout(seed):
    rng = np.random.default_rng(100 + seed)
    n_sink, n_recent, lo, hi = _params(rng)
    Tmax = int(rng.integers(40, 160))
    s = rng.lognormal(0, 1, Tmax)
    thr = float(np.quantile(s, rng.uniform(0.5, 0.95)))
    T0 = n_sink + n_recent + int(rng.integers(0, 10))
    so = O.sealed_segment(s[:T0], thr, n_sink, n_recent, lo, hi)
    for T in range(T0 + 1, Tmax + 1):
        so = O.seal_next(so, s[:T], thr, n_sink, n_recent, lo, hi)
        assert so.tolist() == O.sealed_segment(s[:T], thr, n_sink, n_recent, lo, hi).tolist(), T
        L = so[1:] - so[:-1] - 1
        assert np.all((L >= 1) & (L <= hi))


def test_sealed_cache_spans_equal_those_of_a_longer_prefill():
    """The sealed cache of a context holds, span for span, what the prefill
    cache of a longer context holds for the same spans (bounds, ranks,
    summaries, routing keys, factors); its full-resolution rows are the sink,
    the sealed anchors and the tail from the last sealed head."""
    rng = np.random.default_rng(7)
    B, Hkv, d, T, T2 = 2, 2, 8, 160, 230
    k = O.storage_round(rng.standard_normal((B, Hkv, T2, d)), "bf16")
    v = O.storage_round(rng.standard_normal((B, Hkv, T2, d)), "bf16")
    s = rng.lognormal(0, 1, (B, T2))
    thr = np.array([np.quantile(s[b], 0.8) for b in range(B)])
    P = rng.standard_normal((Hkv, d, d)) / math.sqrt(d)
    rreq = rng.integers(1, 9, (B, T2))
    gate = rng.uniform(0.5, 1.0, (B, Hkv, T2, 16))
    kw = dict(n_sink=3, n_recent=12, lo=2, hi=9, dtype="bf16")
    sc = O.build_cache(k[:, :, :T], v[:, :, :T], s[:, :T], thr, P, rreq, gate, sealed=True, **kw)
    pc = O.build_cache(k, v, s, thr, P, rreq, gate, **kw)
    for b in range(B):
        n = sc.n_seg(b)
        assert n > 5
        assert sc.seg_off[b].tolist() == pc.seg_off[b][:n + 1].tolist()
        assert sc.rank[b].tolist() == pc.rank[b][:n].tolist()
        assert sc.full_idx[b].tolist() == (list(range(3)) + sc.seg_off[b][:-1].tolist()
                                            + list(range(int(sc.seg_off[b][-1]), T)))
        for kv in range(Hkv):
            for arr in ("sum_k", "sum_v", "rho"):
                assert np.array_equal(getattr(sc, arr)[b][kv], getattr(pc, arr)[b][kv][:n])
            for i in range(n):
                for arr in ("U", "sigma", "gate", "Vh"):
                    assert np.array_equal(getattr(sc, arr)[b][kv][i], getattr(pc, arr)[b][kv][i])


def test_sealed_cache_full_expansion_is_dense_attention():
    rng = np.random.default_rng(8)
    B, Hkv, d, T, G = 1, 2, 8, 90, 2
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    s = rng.lognormal(0, 1, (B, T))
    c = O.build_cache(k, v, s, np.array([np.quantile(s[0], 0.6)]), rng.standard_normal((Hkv, d, d)),
                      np.full((B, T), 64), np.ones((B, Hkv, T, 64)), n_sink=2, n_recent=7, lo=1, hi=6, dtype="f64",
                      sealed=True)
    assert c.n_seg(0) > 3 and c.seg_off[0][-1] < T - 7     # the tail is longer than the recent window
    q = rng.standard_normal((Hkv * G, d))
    out = O.mixed_attention(c, 0, q, np.ones((Hkv * G, c.n_seg(0)), bool), G)
    assert np.abs(out - O.dense_attention(q, k[0], v[0], G)).max() <= 1e-9
