"""Host bookkeeping of the device factor cache (no GPU): sekv_factor_cache_lookup
on a cache created without a context.

The policy under test is the one include/sekv.h documents for
sekv_factor_cache_create: 2 MiB pages split evenly among partitions (KV group
g in partition g mod partitions), and per partition slot classes growing by
about 1.25x from 1 KiB in 256-byte steps, a page per class on demand,
per-class LRU eviction once the partition's pages are assigned, blocks of the
current call pinned (bypass when a class has nothing else to evict), and a
refill when a key's host address or size changes.  `PolicyModel` restates
that policy in plain Python; the library must agree with it on every status
and slot offset, and the results must also satisfy properties that hold under
any correct policy (disjoint slots, consistent counters, hits at the slot of
the fill).
"""
import ctypes
from collections import OrderedDict

import numpy as np
import pytest

from hierarchical_kv_cache_sekv_amd import binding as B

PAGE = B.CACHE_PAGE_BYTES
HIT, FILL, BYPASS = B.CACHE_HIT, B.CACHE_FILL, B.CACHE_BYPASS
MAX_BLOCK = 65536 * 4 + 2048


def slot_classes():
    out, s = [], 1024
    while True:
        out.append(s)
        if s >= MAX_BLOCK:
            return out
        nx = max(s + 256, (s * 5 + 3) // 4)
        s = (nx + 255) // 256 * 256


class PartModel:
    """One partition: pages [page0, page0 + pages)."""

    def __init__(self, page0, pages):
        self.cls = slot_classes()
        self.page0, self.pages, self.next_page, self.epoch = page0, pages, 0, 0
        self.free = [[] for _ in self.cls]
        self.lru = [OrderedDict() for _ in self.cls]   # least recent first
        self.ent = {}                                  # key -> [tag, bytes, off, epoch, cls]

    def begin(self):
        self.epoch += 1

    def class_of(self, nb):
        for i, s in enumerate(self.cls):
            if s >= nb:
                return i
        return -1

    def take(self, c):
        fr = self.free[c]
        if not fr and self.next_page < self.pages:
            base = (self.page0 + self.next_page) * PAGE
            self.next_page += 1
            fr.extend(base + i * self.cls[c] for i in reversed(range(PAGE // self.cls[c])))
        if fr:
            return fr.pop()
        if self.lru[c]:
            k = next(iter(self.lru[c]))
            if self.ent[k][3] != self.epoch:
                off = self.ent[k][2]
                del self.lru[c][k]
                del self.ent[k]
                return off
        return None

    def lookup(self, key, nb, tag):
        e = self.ent.get(key)
        if e is not None:
            if e[0] == tag and e[1] == nb:
                self.lru[e[4]].move_to_end(key)
                e[3] = self.epoch
                return HIT, e[2]
            del self.lru[e[4]][key]
            self.free[e[4]].append(e[2])
            del self.ent[key]
        c = self.class_of(nb)
        slot = self.take(c) if c >= 0 else None
        if slot is None:
            return BYPASS, -1
        self.ent[key] = [tag, nb, slot, self.epoch, c]
        self.lru[c][key] = None
        return FILL, slot


class PolicyModel:
    def __init__(self, nbytes, parts):
        n = nbytes // PAGE
        self.parts = [PartModel(n * p // parts, n * (p + 1) // parts - n * p // parts) for p in range(parts)]

    def begin(self):
        for p in self.parts:
            p.begin()

    def lookup(self, key, nb, tag):
        g = (key >> 32) & 0xFFFF
        return self.parts[g % len(self.parts)].lookup(key, nb, tag)


def make_layout(seed, B_=2, Hkv=2, D=128, n_spans=60, Lmin=1, Lmax=40, rmin=1, rmax=32, uniform=None,
                tiny_every=0):
    """Config and plan of random (or uniform (L, r)) spans; with tiny_every,
    every tiny_every-th span has L = 2, r = 1 (a block of another slot class)."""
    rng = np.random.default_rng(seed)
    n_sink, n_recent = 4, 64
    segs, ranks = [], []
    for _ in range(B_):
        if uniform:
            L = np.full(n_spans, uniform[0])
            r = np.full(n_spans, uniform[1])
        else:
            L = rng.integers(Lmin, Lmax + 1, n_spans)
            r = np.minimum(rng.integers(rmin, rmax + 1, n_spans), L)
            if tiny_every:
                L[::tiny_every], r[::tiny_every] = 2, 1
        so = n_sink + np.concatenate([[0], np.cumsum(L + 1)])
        segs.append(so)
        ranks.append(r)
    T = int(max(s[-1] for s in segs)) + n_recent
    cfg = B.Config(B_, T, 4 * Hkv, Hkv, D, n_sink, n_recent, 1, 128, B.SEKV_BF16, 1, 0, 0, 0, 0, 0)
    plan = B.layout_from_segments(cfg, segs, ranks)
    return cfg, plan


def spans_of(cfg, plan, fac_base=1 << 40):
    cap, full_cap = B.capacities(cfg)
    keep = [np.ascontiguousarray(a) for a in (plan.n_seg, plan.n_full, plan.seg_off, plan.rank, plan.fac_off,
                                               plan.sg_off)]
    st = B.Spans(cap, full_cap, B._ptr(keep[0]), B._ptr(keep[1]), None, None, None, None, None, None, None,
                 None, None, fac_base, 1 << 41, plan.fac_elems, plan.sg_elems, B._ptr(keep[2]), B._ptr(keep[3]),
                 B._ptr(keep[4]), B._ptr(keep[5]), None, None)
    st._keep = keep
    return st


def block_bytes(cfg, plan, b, S):
    L = int(plan.seg_off[b, S + 1] - plan.seg_off[b, S] - 1)
    r = int(plan.rank[b, S])
    return B.fac_block_elems(L, r, cfg.head_dim) * 2 + B.sg_entry_elems(r) * 4


def model_batch(model, layer, cfg, plan, spans, lists):
    Hkv, cap = cfg.n_kv_heads, plan.rank.shape[1]
    model.begin()
    out = []
    for g, lst in enumerate(lists):
        b, kv = divmod(g, Hkv)
        for S in lst:
            key = (layer << 48) | (g << 32) | int(S)
            tag = spans.fac + int(plan.fac_off[b, kv, S]) * 2
            out.append(model.lookup(key, block_bytes(cfg, plan, b, S), tag))
    return out


def lib_batch(fc, layer, cfg, plan, spans, lists):
    BG, cap = len(lists), plan.rank.shape[1]
    exp_list = np.zeros((BG, cap), np.int32)
    exp_count = np.zeros(BG, np.int32)
    for g, lst in enumerate(lists):
        exp_list[g, :len(lst)] = lst
        exp_count[g] = len(lst)
    status, offset = fc.lookup(layer, cfg, spans, exp_list, exp_count)
    return [(int(status[g, j]), int(offset[g, j])) for g, lst in enumerate(lists) for j in range(len(lst))]


def check_disjoint(res, sizes, arena):
    spans_ = sorted((off, off + nb) for (st, off), nb in zip(res, sizes) if st != BYPASS)
    for (a0, a1), (b0, b1) in zip(spans_, spans_[1:]):
        assert a1 <= b0, "two blocks of one call share arena bytes"
    assert not spans_ or (spans_[0][0] >= 0 and spans_[-1][1] <= arena)


def test_slot_classes_match_the_documented_growth():
    c = slot_classes()
    assert c[0] == 1024 and all(x % 256 == 0 for x in c) and c[-1] >= MAX_BLOCK
    assert all(1.2 <= b / a <= 1.25 + 256 / a for a, b in zip(c, c[1:]))


def test_cache_follows_the_policy_over_random_calls():
    # long spans of high rank (two slot classes) and a few tiny ones (a third
    # class): two pages run full, and one class finds no page (bypasses)
    cfg, plan = make_layout(7, Lmin=24, rmin=24, tiny_every=6)
    spans = spans_of(cfg, plan)
    BG = cfg.batch * cfg.n_kv_heads
    nbytes = 2 * PAGE + 12345
    fc = B.FactorCache(None, nbytes, partitions=1)
    model = PolicyModel(nbytes, 1)
    rng = np.random.default_rng(11)
    prev = {}
    totals = {"lookups": 0, "hits": 0, "fills": 0, "bypasses": 0}
    seen_bypass = False
    for step in range(40):
        for layer in (0, 1, 5):
            lists = []
            for g in range(BG):
                b = g // cfg.n_kv_heads
                n = int(plan.n_seg[b])
                old = prev.get((layer, g), np.zeros(0, np.int64))
                keep = old[rng.random(old.size) < 0.7]
                new = rng.choice(n, size=int(rng.integers(0, 16)), replace=False)
                lists.append(np.unique(np.concatenate([keep, new])).astype(np.int32))
                prev[(layer, g)] = lists[-1]
            want = model_batch(model, layer, cfg, plan, spans, lists)
            got = lib_batch(fc, layer, cfg, plan, spans, lists)
            assert got == want, f"step {step} layer {layer}"
            sizes = [block_bytes(cfg, plan, g // cfg.n_kv_heads, S) for g, lst in enumerate(lists) for S in lst]
            check_disjoint(got, sizes, 2 * PAGE)
            for st, _ in got:
                totals["lookups"] += 1
                totals[("hits", "fills", "bypasses")[st]] += 1
            seen_bypass |= any(st == BYPASS for st, _ in got)
    stats = fc.stats()
    for k, v in totals.items():
        assert stats[k] == v
    assert stats["pages_used"] == stats["pages_total"] == 2
    assert stats["evictions"] > 0 and stats["hits"] > 0 and seen_bypass
    ents = [e for part in model.parts for e in part.ent.values()]
    assert stats["resident_blocks"] == len(ents)
    assert stats["resident_bytes"] == sum(e[1] for e in ents)
    fc.close()


def test_partitions_follow_the_policy_over_random_calls():
    """Four KV groups over three partitions (groups 0 and 3 share one), seven
    pages (2 + 2 + 3): each partition runs the policy on its own pages."""
    cfg, plan = make_layout(8, Lmin=24, rmin=24, tiny_every=5)
    spans = spans_of(cfg, plan)
    BG = cfg.batch * cfg.n_kv_heads
    nbytes = 7 * PAGE
    fc = B.FactorCache(None, nbytes, partitions=3)
    model = PolicyModel(nbytes, 3)
    rng = np.random.default_rng(12)
    prev = {}
    for step in range(30):
        for layer in (0, 2):
            lists = []
            for g in range(BG):
                n = int(plan.n_seg[g // cfg.n_kv_heads])
                old = prev.get((layer, g), np.zeros(0, np.int64))
                keep = old[rng.random(old.size) < 0.6]
                new = rng.choice(n, size=int(rng.integers(0, 24)), replace=False)
                lists.append(np.unique(np.concatenate([keep, new])).astype(np.int32))
                prev[(layer, g)] = lists[-1]
            assert lib_batch(fc, layer, cfg, plan, spans, lists) == model_batch(model, layer, cfg, plan, spans, lists)
    st = fc.stats()
    assert st["evictions"] > 0 and st["hits"] > 0 and st["pages_total"] == 7
    fc.close()


def test_least_recently_used_block_leaves_first_and_the_call_pins_its_blocks():
    cfg, plan = make_layout(3, B_=1, Hkv=1, n_spans=400, uniform=(16, 16))
    spans = spans_of(cfg, plan)
    nb = block_bytes(cfg, plan, 0, 0)
    slot = next(s for s in slot_classes() if s >= nb)
    N = PAGE // slot
    assert N + 3 <= 400
    fc = B.FactorCache(None, PAGE, partitions=1)
    run = lambda lst: lib_batch(fc, 0, cfg, plan, spans, [np.asarray(lst, np.int32)])
    # one call larger than the cache: N fills, then bypasses (nothing of the call is evicted)
    res = run(range(N + 2))
    assert [s for s, _ in res] == [FILL] * N + [BYPASS] * 2
    offs = {j: off for j, (s, off) in enumerate(res) if s == FILL}
    # touch span 0, then a new span evicts the least recently used (span 1)
    assert run([0]) == [(HIT, offs[0])]
    assert run([N + 2]) == [(FILL, offs[1])]
    assert run([0]) == [(HIT, offs[0])]
    assert run([1])[0][0] == FILL          # span 1 was evicted; it now takes span 2's slot
    assert run([2])[0][0] == FILL
    assert fc.stats()["evictions"] == 3
    fc.close()


def test_hits_repeat_and_invalidate_drops_one_layer():
    cfg, plan = make_layout(5)
    spans = spans_of(cfg, plan)
    BG = cfg.batch * cfg.n_kv_heads
    lists = [np.arange(0, 20, 2, dtype=np.int32) for _ in range(BG)]
    fc = B.FactorCache(None, 64 * PAGE)
    a0 = lib_batch(fc, 0, cfg, plan, spans, lists)
    a1 = lib_batch(fc, 1, cfg, plan, spans, lists)
    assert {s for s, _ in a0 + a1} == {FILL}
    assert lib_batch(fc, 0, cfg, plan, spans, lists) == [(HIT, off) for _, off in a0]
    fc.invalidate(0)
    assert {s for s, _ in lib_batch(fc, 0, cfg, plan, spans, lists)} == {FILL}
    assert lib_batch(fc, 1, cfg, plan, spans, lists) == [(HIT, off) for _, off in a1]
    # the same keys from another pool (another host address) refill
    other = spans_of(cfg, plan, fac_base=1 << 42)
    assert {s for s, _ in lib_batch(fc, 1, cfg, plan, other, lists)} == {FILL}
    fc.invalidate(-1)
    st = fc.stats()
    assert st["resident_blocks"] == 0 and st["pages_used"] == 0
    fc.close()


def test_bad_list_is_rejected_and_changes_nothing():
    cfg, plan = make_layout(9)
    spans = spans_of(cfg, plan)
    BG, cap = cfg.batch * cfg.n_kv_heads, plan.rank.shape[1]
    fc = B.FactorCache(None, 4 * PAGE, partitions=2)
    exp_list = np.zeros((BG, cap), np.int32)
    exp_count = np.full(BG, 3, np.int32)
    exp_list[:, :3] = [1, 2, 3]
    fc.lookup(0, cfg, spans, exp_list, exp_count)
    before = fc.stats()
    exp_list[1, 2] = int(plan.n_seg[0]) + 5
    with pytest.raises(B.SekvError) as e:
        fc.lookup(0, cfg, spans, exp_list, exp_count)
    assert e.value.status == B.SEKV_EHIP
    exp_list[1, 2] = 3
    exp_count[0] = cap + 1
    with pytest.raises(B.SekvError):
        fc.lookup(0, cfg, spans, exp_list, exp_count)
    assert fc.stats() == before
    with pytest.raises(B.SekvError):
        B.FactorCache(None, PAGE - 1, partitions=1)
    with pytest.raises(B.SekvError):
        B.FactorCache(None, 3 * PAGE, partitions=4)
    with pytest.raises(B.SekvError):
        B.FactorCache(None, 4 * PAGE, partitions=300)
    with pytest.raises(B.SekvError):
        fc.lookup(70000, cfg, spans, exp_list, np.zeros(BG, np.int32))
    fc.close()
