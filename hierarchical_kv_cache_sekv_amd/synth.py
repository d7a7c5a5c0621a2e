"""Seeded synthetic inputs for the SeKV mixed-resolution decode path.

This module only draws random numbers and shapes them.  It holds none of the
method's arithmetic (no segmentation, summaries, routing, factorisation or
attention), so both the CPU oracle's tests and the GPU path can take their
inputs from it without sharing any computation.

The pages evaluate on LongBench, RULER, InfiniteBench and Needle-in-a-Haystack
with Llama-3 / Mistral / Qwen backbones (gist.science explainers, "Technisches
Resümee" > "Experimentelle Ergebnisse"); none of that is available here, so the
five workloads below are synthetic stand-ins with the Llama-3-8B layer shape
(32 query heads, 8 KV heads, head dim 128) at up to 128K context.

Random streams: ``numpy.random.default_rng([workload_id, stream, b])`` with
stream ids 0 surprisal, 1 K/V noise, 2 per-block low-rank component, 3 ranks,
4 rank gates, 5 routing projections, 6 queries, 7 per-sequence expansion
fractions; layer l > 0 of a multi-layer workload appends l to every seed.

Queries are independent across decode steps unless ``query_corr`` = c > 0:
then the query of step t is c q_{t-1} + sqrt(1 - c^2) e_t (e the same normal
draws), a stand-in for the step-to-step similarity of a decoding model's
queries, which the pages do not quantify; it matters only where results carry
over between steps (the device factor cache).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "seg_capacity", "full_capacity",
    "round_bf16", "bf16_bits", "Inputs", "make_inputs", "calibrate_theta",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int                 # stream id used in every seed
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str               # "f32" or "bf16"
    n_ctx: int
    n_sink: int
    n_recent: int
    min_span: int
    max_span: int
    rank_lo: int
    rank_hi: int
    expand_frac: float       # target union expansion per (b, kv); <0: per-seq U(0, -x)
    steps: int
    factors_on_host: bool = False
    boundary_quantile: float = 0.90
    lowrank_rank: int = 4
    # reading variants (the defaults are the default readings)
    rank_cap: str = "full"      # "full": r <= L; "half": r <= ceil(L / 2)
    basis: str = "joint"        # "joint": one basis of [K | V]; "separate": K and V bases
    route_keys: str = "rho"     # "rho": route on rho; "folded": (P^T P q) . kbar / |P kbar|
    # multi-layer workloads: seed namespace of the layer, and step-to-step query correlation
    layer: int = 0
    query_corr: float = 0.0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "tiny-f32-T2K", 1, 4, 1, 64, "f32", 2048, 4, 64, 4, 64, 2, 8, 0.15, 16),
    2: Workload(2, "llama3-8b-layer-T32K-b1", 1, 32, 8, 128, "bf16", 32768, 4, 256, 8, 128, 4, 32, 0.10, 64),
    3: Workload(3, "llama3-8b-layer-T128K-b1-hostfactors", 1, 32, 8, 128, "bf16", 131072, 4, 256, 8, 128, 8, 32, 0.05, 64,
                factors_on_host=True),
    4: Workload(4, "llama3-8b-layer-T32K-b8-ragged", 8, 32, 8, 128, "bf16", 32768, 4, 256, 8, 128, 4, 32, -0.30, 64),
    5: Workload(5, "llama3-8b-layer-T128K-b4", 4, 32, 8, 128, "bf16", 131072, 4, 256, 8, 128, 16, 64, 0.05, 64),
}


def workload(wid: int, **overrides) -> Workload:
    w = WORKLOADS[wid]
    return w.with_(**overrides) if overrides else w


def seg_capacity(T: int, n_sink: int, n_recent: int, min_span: int) -> int:
    """Host-computable bound on the number of spans of one sequence."""
    return max(0, (T - n_sink - n_recent) // (min_span + 1)) + 1


def full_capacity(T: int, n_sink: int, n_recent: int, min_span: int) -> int:
    """Host-computable bound on the full-resolution entries of one sequence."""
    return min(T, n_sink + seg_capacity(T, n_sink, n_recent, min_span) + n_recent + 1)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (via float32, round-to-nearest-even); returned as float32."""
    f = np.array(x, dtype=np.float32, copy=True, order="C")
    u = f.view(np.uint32)
    lsb = u >> 16
    lsb &= 1
    lsb += 0x7FFF
    u += lsb                      # finite inputs only: no carry out of the exponent field
    u &= np.uint32(0xFFFF0000)
    return f


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-representable."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _rng(w: Workload, stream: int, b: int) -> np.random.Generator:
    return np.random.default_rng([w.wid, stream, b] + ([w.layer] if w.layer else []))


@dataclasses.dataclass
class Inputs:
    w: Workload
    surprisal: np.ndarray    # [B][T] f32
    boundary_thr: np.ndarray  # [B] f32
    k: np.ndarray            # [B][Hkv][T][d] f32 (bf16-representable for bf16 workloads)
    v: np.ndarray
    route_proj: np.ndarray   # [Hkv][d][d] f32
    rank_req: np.ndarray     # [B][seg_cap] int32
    gate: np.ndarray         # [B][Hkv][seg_cap][rank_cap] f32
    q: np.ndarray            # [steps][B][Hq][d] f32 (bf16-representable for bf16)
    expand_frac: np.ndarray  # [B] target union expansion fraction per sequence

    @property
    def seg_cap(self) -> int:
        w = self.w
        return seg_capacity(w.n_ctx, w.n_sink, w.n_recent, w.min_span)


def _blocks(s: np.ndarray, thr: float, lo_tok: int, hi_tok: int):
    """Generator-side block structure for the low-rank component: a block
    starts at ``lo_tok`` and at every token in (lo_tok, hi_tok) whose surprisal
    exceeds ``thr``.  (Structure of the synthetic data only; the method's own
    segmentation rule is not used here.)"""
    if hi_tok - lo_tok < 1:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    starts = np.concatenate([[lo_tok], lo_tok + 1 + np.nonzero(s[lo_tok + 1:hi_tok] > thr)[0]])
    ends = np.concatenate([starts[1:], [hi_tok]])
    return starts.astype(np.int64), ends.astype(np.int64)


def make_inputs(w: Workload, *, n_steps: int | None = None, rank_cap: int | None = None,
                full_rank_unit_gates: bool = False) -> Inputs:
    """Draw every input of workload ``w``.

    ``full_rank_unit_gates``: request rank ``max_span`` for every span and set
    every gate to 1 (the full-rank special case).
    """
    B, Hq, Hkv, d, T = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_ctx
    steps = w.steps if n_steps is None else n_steps
    cap = seg_capacity(T, w.n_sink, w.n_recent, w.min_span)
    r_cap = rank_cap if rank_cap is not None else (w.max_span if full_rank_unit_gates else w.rank_hi)
    bf16 = w.dtype == "bf16"

    surprisal = np.empty((B, T), np.float32)
    thr = np.empty(B, np.float32)
    k = np.empty((B, Hkv, T, d), np.float32)
    v = np.empty((B, Hkv, T, d), np.float32)
    rank_req = np.empty((B, cap), np.int32)
    gate = np.empty((B, Hkv, cap, r_cap), np.float32)
    q = np.empty((steps, B, Hq, d), np.float32)
    lo_tok, hi_tok = w.n_sink, T - w.n_recent
    R = w.lowrank_rank
    for b in range(B):
        s = _rng(w, 0, b).lognormal(0.0, 1.0, T).astype(np.float32)
        surprisal[b] = s
        # boundary threshold: lower-interpolated quantile over all T tokens
        thr[b] = np.sort(s)[int(math.floor(w.boundary_quantile * (T - 1)))]
        kv = _rng(w, 1, b).standard_normal((2, Hkv, T, d), dtype=np.float32)
        g2 = _rng(w, 2, b)
        starts, ends = _blocks(s, float(thr[b]), lo_tok, hi_tok)
        n_tok = int(ends[-1] - starts[0]) if starts.size else 0
        for h in range(Hkv):
            k[b, h] = kv[0, h]
            v[b, h] = kv[1, h]
            if n_tok == 0:
                continue
            A = g2.standard_normal((n_tok, R), dtype=np.float32)                  # one row per token
            Bm = g2.standard_normal((starts.size, R, 2 * d), dtype=np.float32) * np.float32(1.0 / math.sqrt(R))
            lens = ends - starts
            comp = np.empty((n_tok, 2 * d), np.float32)
            for ell in np.unique(lens).tolist():                                   # blocks of equal length together
                sel = np.nonzero(lens == ell)[0]
                rows = ((starts[sel] - lo_tok)[:, None] + np.arange(ell)[None, :]).reshape(-1)
                comp[rows] = np.matmul(A[rows].reshape(sel.size, ell, R), Bm[sel]).reshape(-1, 2 * d)
            k[b, h, lo_tok:lo_tok + n_tok] += comp[:, :d]
            v[b, h, lo_tok:lo_tok + n_tok] += comp[:, d:]
        del kv
        if full_rank_unit_gates:
            rank_req[b] = w.max_span
            gate[b] = 1.0
        else:
            rank_req[b] = _rng(w, 3, b).integers(w.rank_lo, w.rank_hi + 1, cap, dtype=np.int32)
            gate[b] = _rng(w, 4, b).uniform(0.0, 1.0, (Hkv, cap, r_cap)).astype(np.float32)
        q[:, b] = _rng(w, 6, b).standard_normal((steps, Hq, d), dtype=np.float32)
        if w.query_corr > 0.0:
            c, s2 = np.float32(w.query_corr), np.float32(math.sqrt(1.0 - w.query_corr ** 2))
            for t in range(1, steps):
                q[t, b] = c * q[t - 1, b] + s2 * q[t, b]
    proj = _rng(w, 5, 0).normal(0.0, 1.0 / math.sqrt(d), (Hkv, d, d)).astype(np.float32)
    if w.expand_frac < 0:
        ef = _rng(w, 7, 0).uniform(0.0, -w.expand_frac, B)
    else:
        ef = np.full(B, w.expand_frac)
    if bf16:
        k, v, q = round_bf16(k), round_bf16(v), round_bf16(q)
    return Inputs(w, surprisal, thr, k, v, proj, rank_req, gate, q, ef)


def calibrate_theta(z: np.ndarray, frac: float, group: int) -> np.ndarray:
    """Per-query-head thresholds (logit space) for a target union expansion.

    ``z``: routing scores of one sequence, shape [n_samples][Hq][n_spans]
    (any number of decode steps stacked).  Each head gets level
    f_h = 1 - (1 - frac)^(1/group) so that the union over a group of ``group``
    heads expands about ``frac`` of the spans; the threshold sits at the float32
    midpoint between the two sorted scores around the (1 - f_h) quantile, so no
    score equals it.  ``frac <= 0`` gives +inf (nothing expands), ``frac >= 1``
    gives -inf (everything expands).
    """
    Hq = z.shape[1]
    out = np.empty(Hq, np.float32)
    if frac <= 0.0:
        out[:] = np.inf
        return out
    if frac >= 1.0:
        out[:] = -np.inf
        return out
    fh = 1.0 - (1.0 - frac) ** (1.0 / group)
    for h in range(Hq):
        zs = np.sort(z[:, h, :].reshape(-1).astype(np.float32))
        n = zs.size
        if n == 0:
            out[h] = np.inf
            continue
        i = int(math.floor((1.0 - fh) * (n - 1)))
        if i >= n - 1:
            out[h] = np.inf
        else:
            out[h] = np.float32((np.float64(zs[i]) + np.float64(zs[i + 1])) * 0.5)
    return out
