"""Host-side logic of bench.py (no GPU): the graph schedule covers exactly the
requested steps for any (steps, warmup, steps-per-graph), graph sharing keys
only merge chunks that run identical steps, and the algorithmic byte count
follows its formula on a hand-built plan."""
import subprocess
import sys
import types

import numpy as np
import pytest

import bench


@pytest.mark.parametrize("steps,warmup,gs", [(20, 5, 8), (1, 0, 8), (7, 3, 8), (8, 8, 8), (256, 16, 8),
                                             (63, 1, 16), (5, 0, 1), (33, 7, 32), (64, 8, 64)])
def test_graph_chunks_cover_every_step_once(steps, warmup, gs):
    ch = bench.graph_chunks(warmup, steps, gs)
    covered = [s for first, n in ch for s in range(first, first + n)]
    assert covered == list(range(warmup, warmup + steps))
    assert all(1 <= n <= gs for _, n in ch)
    assert all(n == gs for _, n in ch[:-1])
    assert len(ch) == -(-steps // gs)


@pytest.mark.parametrize("ncopy,Q,gs,steps,warmup", [(2, 64, 8, 20, 5), (3, 16, 8, 100, 7), (2, 64, 8, 256, 16)])
def test_graph_keys_only_merge_identical_chunks(ncopy, Q, gs, steps, warmup):
    import math
    period = math.lcm(ncopy, Q)
    seen = {}
    for first, n in bench.graph_chunks(warmup, steps, gs):
        key = bench.graph_key(first, n, period)
        ident = [((first + u) % ncopy, (first + u) % Q) for u in range(n)]
        if key in seen:
            assert seen[key] == ident
        seen[key] = ident


def test_graph_chunks_rejects_bad_arguments():
    with pytest.raises(ValueError):
        bench.graph_chunks(0, 5, 0)
    assert bench.graph_chunks(3, 0, 8) == []


def test_algorithmic_bytes_formula():
    # two sequences, two KV heads, d = 4, bf16; spans (L, r) chosen by hand
    w = types.SimpleNamespace(head_dim=4, n_q_heads=4, n_kv_heads=2, batch=2)
    plan = types.SimpleNamespace(n_full=np.array([10, 7]), n_seg=np.array([3, 1]),
                                 seg_off=np.array([[4, 7, 9, 15], [4, 6, 6, 6]]),
                                 rank=np.array([[2, 1, 3], [1, 0, 0]]))
    # L: seq 0 -> [2, 1, 5], seq 1 -> [1]
    counts = np.array([[2, 0], [1, 1]])
    lists = np.array([[[0, 2, 0], [0, 0, 0]], [[0, 0, 0], [0, 0, 0]]])
    e, d = 2, 4
    fac = lambda L, r: e * r * (L + 2 * d) + 8 * r
    f0 = fac(2, 2) + fac(5, 3)
    f1 = 2 * fac(1, 1)
    want_total = (4 * d * (e + 4) + 2 * (e * 2 * d * 10 + e * 3 * d * 3) + f0
                  + 4 * d * (e + 4) + 2 * (e * 2 * d * 7 + e * 3 * d * 1) + f1)
    got = bench.algorithmic_bytes(w, plan, counts, lists, e)
    assert got["total"] == want_total
    assert got["factors"] == f0 + f1
    assert got["route"] == (4 * d * e + 2 * 3 * d * e) + (4 * d * e + 2 * 1 * d * e)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2", "--steps", "20", "--warmup", "5"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
