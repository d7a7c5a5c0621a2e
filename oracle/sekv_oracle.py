"""CPU oracle for SeKV mixed-resolution decode.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (``libsekv.so`` and its binding) never does, and this module never
imports the product path.  It shares no code with it.

It is a plain, slow, fp64 numpy statement of what the method computes, written
from these pages (cited by tag):

* [abstract]  the authors' abstract (chatpaper.ai paper page, English part;
  repeated on the Lattice summary page).
* [de-1] [de-2] [de-3]  gist.science, German explainer of "SeKV: Resolution-
  Adaptive KV Cache with Hierarchical Semantic Memory for Long-Context LLM
  Inference", section "Technisches Resümee" > "Methodik", parts 1
  (Entropie-gestützte Span-Segmentierung), 2 (Dual-Resolution
  Span-Repräsentation & Speicherhierarchie) and 3 (Trainierter
  Zoom-In-Mechanismus).
* [zh-1] [zh-2] [zh-3]  gist.science, Chinese explainer of the same paper,
  section "技术摘要" > "方法论", parts 1, 2 and 3 (parallel to the German one).

Where the pages leave a step open, the reading taken is named in the function
docstring ("Reading: ...").  Every function is pinned by a ``-m "not gpu"`` test
in ``tests/test_oracle_pins.py`` against something other than itself (brute
force, closed forms, textbook special cases, hand-worked golden values).

Precision: fp64 throughout, except (a) the routing score, defined as one
canonical float32 evaluation so that the expanded set is a function of the
stored bits alone, and (b) the cache arrays, which are *stored* in the
workload's element type (float32 or bfloat16; bfloat16 = float32 rounded to
nearest-even on the upper 16 bits) and read back exactly.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List

import numpy as np

__all__ = [
    "storage_round", "segment", "full_res_tokens", "span_summary", "span_summaries",
    "routing_keys", "span_factors", "OracleCache", "build_cache", "route_scores",
    "route", "compact", "reconstruct", "mixed_attention", "mixed_attention_all",
    "dense_attention", "SIZE_CORRECTION", "span_factors_separate", "span_ranks", "fold_matrix",
    "fold_query", "key_scales", "route_scores_folded", "reconstruct_span", "sealed_segment", "seal_next",
]

# Reading: the size correction of an unexpanded span's summary logit is +ln|S|
# (natural log of the body length), added after the 1/sqrt(d) scaling, so the
# summary acts as |S| copies of one key/value pair.  [de-3], [zh-3] say only
# "with size correction".
SIZE_CORRECTION = True


# --------------------------------------------------------------------------
# storage precision
# --------------------------------------------------------------------------
def storage_round(x, dtype: str) -> np.ndarray:
    """Value of ``x`` after storing it in ``dtype`` ("f32", "bf16" or "f64"), as fp64.

    fp64 -> float32 (round to nearest even); for "bf16" the float32 is then
    rounded to nearest even on its upper 16 bits.
    """
    if dtype == "f64":        # no rounding: used by the exact special-case pins
        return np.array(x, dtype=np.float64)
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return f.astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    bits = f.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# [de-1] / [zh-1]: entropy-guided span segmentation
# --------------------------------------------------------------------------
def segment(s, thr: float, n_sink: int, n_recent: int, lo: int, hi: int) -> np.ndarray:
    """Span offsets of one sequence from its per-token surprisal.

    [de-1]/[zh-1]: tokens of high surprisal mark span boundaries and become
    anchors kept at full resolution; a span is the run of tokens between two
    neighbouring anchors.

    Readings: (i) "high surprisal" = strictly above ``thr``; (ii) each anchor is
    the head of its segment and the span body follows it; (iii) the first token
    after the sink is always a head; (iv) a data head needs at least ``lo`` body
    tokens before it and leaves at least ``lo`` tokens before the recent window;
    a body reaching ``hi`` tokens forces the next token to be a head; (v) the
    sink [0, n_sink) and the recent window are full resolution; a last head with
    an empty body is given back to the tail.

    Returns ``seg_off`` (int64, length n_seg + 1): anchor i is token
    ``seg_off[i]``, body i is the open interval (seg_off[i], seg_off[i+1]), and
    the full-resolution tail starts at ``seg_off[n_seg]``.
    """
    s = np.asarray(s)
    T = s.shape[0]
    a, e = n_sink, T - n_recent
    if e - a < 2:
        return np.array([a], dtype=np.int64)
    heads = [a]
    h = a
    for t in range(a + 1, e):
        body = t - h - 1
        if body == hi:
            heads.append(t)
            h = t
        elif s[t] > thr and body >= lo and (e - t - 1) >= lo:
            heads.append(t)
            h = t
    if h == e - 1:
        heads.pop()
        tail = h
    else:
        tail = e
    return np.array(heads + [tail], dtype=np.int64)


def sealed_segment(s, thr: float, n_sink: int, n_recent: int, lo: int, hi: int) -> np.ndarray:
    """Span offsets of a context during decode: only the sealed spans.

    [de-1]/[zh-1] define the segmentation at prefill; during decode tokens
    keep arriving and leave the recent window.  Reading (when a span seals):
    the rule of ``segment`` decides token t for good once t <= e - 1 - lo,
    e = T - n_recent: from then on the data-head condition's room before the
    recent window (e - t - 1 >= lo) holds at every longer context, and the
    forced-head condition never depended on e.  A span seals when its closing
    head is decided.  The cache of a context holds the sealed spans; every
    token from the last sealed head on (that head is the anchor of the span
    still open) stays at full resolution.

    Returns ``seg_off`` in the format of ``segment``: the decided heads
    h_0 .. h_k, the last of which is the tail start (n_seg = k).
    """
    s = np.asarray(s)
    e = s.shape[0] - n_recent
    heads = [int(h) for h in segment(s, thr, n_sink, n_recent, lo, hi)[:-1] if h <= e - 1 - lo]
    if not heads:
        heads = [n_sink]
    return np.array(heads, dtype=np.int64)


def seal_next(seg_off, s, thr: float, n_sink: int, n_recent: int, lo: int, hi: int) -> np.ndarray:
    """One decode step of online sealing: ``seg_off`` is the sealed layout of
    the context of len(s) - 1 tokens, s the surprisal of len(s) tokens (the
    last one new).  With the new token one more token becomes decided,
    t = len(s) - n_recent - 1 - lo; it is a head if its body (tokens since the
    last sealed head) has reached ``hi``, or if s[t] > thr and the body holds
    at least ``lo`` tokens.  A new head closes (seals) the span after the last
    sealed head.  Returns the sealed layout of the longer context."""
    so = [int(x) for x in seg_off]
    t = len(s) - n_recent - 1 - lo
    if t >= n_sink + 1:
        h = so[-1]
        body = t - h - 1
        if body == hi or (s[t] > thr and body >= lo):
            so.append(t)
    return np.array(so, dtype=np.int64)


def full_res_tokens(seg_off: np.ndarray, n_sink: int, T: int) -> np.ndarray:
    """Token indices kept at full resolution, in this order: sink, anchors, tail."""
    seg_off = np.asarray(seg_off, dtype=np.int64)
    return np.concatenate([np.arange(n_sink), seg_off[:-1], np.arange(seg_off[-1], T)]).astype(np.int64)


# --------------------------------------------------------------------------
# [de-2] / [zh-2]: per-span summary and routing key
# --------------------------------------------------------------------------
def span_summary(k_body, v_body, s_body):
    """Surprisal-weighted mean key and value of one span body (fp64).

    [de-2]/[zh-2]: the GPU keeps a light summary per span, a normalised,
    surprisal-weighted average.  Reading: weights w_t = s_t / sum(s) (uniform if
    the sum is 0); the value summary uses the same weights.
    """
    k_body = np.asarray(k_body, np.float64)
    v_body = np.asarray(v_body, np.float64)
    s_body = np.asarray(s_body, np.float64)
    tot = s_body.sum()
    if tot > 0:
        w = s_body / tot
    else:
        w = np.full(s_body.shape, 1.0 / s_body.shape[0])
    return (w[:, None] * k_body).sum(axis=0), (w[:, None] * v_body).sum(axis=0)


def span_summaries(k, v, s, seg_off):
    """``span_summary`` for every span of one (sequence, kv head): [n_seg][d] x2."""
    n_seg = len(seg_off) - 1
    d = k.shape[1]
    kb = np.zeros((n_seg, d))
    vb = np.zeros((n_seg, d))
    for i in range(n_seg):
        lo, hi = int(seg_off[i]) + 1, int(seg_off[i + 1])
        kb[i], vb[i] = span_summary(k[lo:hi], v[lo:hi], s[lo:hi])
    return kb, vb


def routing_keys(kbar, P):
    """Routing key per span (fp64), [n][d].

    [de-2]/[zh-2]: the summary is a normalised average of *projected* keys;
    [de-3]/[zh-3]: the query is projected into the same routing space and a
    sigmoid gate scores relevance.  Readings: one d x d projection P per KV head
    for both sides; r = P kbar, r_hat = r / |r| (0 if |r| = 0); the stored key
    is rho = P^T r_hat so that (P q) . r_hat = q . rho.
    """
    kbar = np.asarray(kbar, np.float64)
    P = np.asarray(P, np.float64)
    r = kbar @ P.T
    nrm = np.sqrt((r * r).sum(axis=1, keepdims=True))
    rhat = np.where(nrm > 0, r / np.where(nrm > 0, nrm, 1.0), 0.0)
    return rhat @ P


def span_factors(k_body, v_body, r: int):
    """Rank-r SVD factors of one span's joint key/value matrix (fp64).

    [abstract], [de-2]/[zh-2]: each span keeps a low-rank SVD basis for
    on-demand token-level reconstruction.  Reading: one basis for [K_S | V_S]
    (L x 2d); keep the r largest singular triplets; U is L x r, Vh is r x 2d
    (first d columns: key part, last d: value part).  Sign: each U column is
    flipped so its largest-magnitude entry (lowest index on ties) is positive.
    """
    M = np.concatenate([np.asarray(k_body, np.float64), np.asarray(v_body, np.float64)], axis=1)
    U, sig, Vh = np.linalg.svd(M, full_matrices=False)
    U, sig, Vh = U[:, :r].copy(), sig[:r].copy(), Vh[:r].copy()
    for j in range(r):
        i = int(np.argmax(np.abs(U[:, j])))
        if U[i, j] < 0:
            U[:, j] *= -1.0
            Vh[j] *= -1.0
    return U, sig, Vh


def span_factors_separate(k_body, v_body, r: int):
    """Reading variant: one rank-r basis for the keys and another for the
    values of a span (two SVDs of L x d matrices instead of one of L x 2d).

    [de-2]/[zh-2] speak of one low-rank SVD basis per span; this variant tests
    that reading.  Returns ((U_K, sigma_K, Vh_K [r][d]), (U_V, sigma_V,
    Vh_V [r][d])), each signed like ``span_factors``.
    """
    out = []
    for M in (np.asarray(k_body, np.float64), np.asarray(v_body, np.float64)):
        U, sig, Vh = np.linalg.svd(M, full_matrices=False)
        U, sig, Vh = U[:, :r].copy(), sig[:r].copy(), Vh[:r].copy()
        for j in range(r):
            i = int(np.argmax(np.abs(U[:, j])))
            if U[i, j] < 0:
                U[:, j] *= -1.0
                Vh[j] *= -1.0
        out.append((U, sig, Vh))
    return tuple(out)


def span_ranks(rank_req, L, d: int, rank_cap: str = "full", basis: str = "joint"):
    """Rank of each span: r = min(requested, cap(L), rank of the factored
    matrix).  Readings: cap(L) = L (default) or ceil(L / 2) (variant "half");
    the factored matrix is L x 2d (joint basis) or L x d (separate bases)."""
    L = np.asarray(L, np.int64)
    cap = L if rank_cap == "full" else (L + 1) // 2
    width = 2 * d if basis == "joint" else d
    return np.minimum(np.minimum(np.asarray(rank_req, np.int64), cap), width)


# --------------------------------------------------------------------------
# reading variant: routing folded onto the attention summary key
# --------------------------------------------------------------------------
def fold_matrix(P) -> np.ndarray:
    """M = P^T P (fp64), accumulated over the rows a of P in order:
    M += outer(P[a], P[a]), each product and sum rounded in fp64."""
    P = np.asarray(P, np.float64)
    M = np.zeros((P.shape[1], P.shape[1]))
    for a in range(P.shape[0]):
        M = M + np.multiply.outer(P[a], P[a])
    return M


def fold_query(M, q) -> np.ndarray:
    """Folded query q' = M q per head, as float32: for each output element a
    sequential fp64 sum over j of M[i][j] * q[j] (each product and sum rounded
    in fp64), then rounded to float32.  q: [G][d] stored values."""
    M = np.asarray(M, np.float64)
    q = np.asarray(q, np.float64)
    acc = np.zeros((q.shape[0], M.shape[0]))
    for j in range(M.shape[1]):
        acc = acc + np.multiply.outer(q[:, j], M[:, j])
    return acc.astype(np.float32)


def key_scales(kbar, P) -> np.ndarray:
    """Per-span scale 1 / |P kbar| (0 if the norm is 0), float32, from the
    unrounded fp64 summary key."""
    r = np.asarray(kbar, np.float64) @ np.asarray(P, np.float64).T
    nrm = np.sqrt((r * r).sum(axis=1))
    return np.where(nrm > 0, 1.0 / np.where(nrm > 0, nrm, 1.0), 0.0).astype(np.float32)


def route_scores_folded(qf, kbar, scale) -> np.ndarray:
    """Reading variant of the routing score: (P q) . normalize(P kbar) written
    as (P^T P q) . kbar / |P kbar|, so the route reads the stored attention
    summary key kbar instead of a separate routing key.  Canonical float32
    order: z = sequential float32 sum over i of fl32(q'_i * kbar_i), then
    z' = fl32(z * scale).  qf: folded queries [G][d] float32 (fold_query)."""
    z = route_scores(qf, kbar)
    return np.multiply(z, np.asarray(scale, np.float32)[None, :], dtype=np.float32)


# --------------------------------------------------------------------------
# cache build (prefill side)
# --------------------------------------------------------------------------
@dataclasses.dataclass
class OracleCache:
    """Everything the decode reads, per sequence b and KV head.

    Stored arrays hold values exactly representable in ``dtype`` (as fp64);
    ``sigma`` is float32-representable; ``gate`` is the float32 input.
    """
    dtype: str
    n_sink: int
    T: int
    d: int
    seg_off: List[np.ndarray]                 # [b] -> int64 [n_seg+1]
    full_idx: List[np.ndarray]                # [b] -> int64 [n_full]
    full_k: List[List[np.ndarray]]            # [b][kv] -> [n_full][d]
    full_v: List[List[np.ndarray]]
    sum_k: List[List[np.ndarray]]             # [b][kv] -> [n_seg][d]
    sum_v: List[List[np.ndarray]]
    rho: List[List[np.ndarray]]
    rank: List[np.ndarray]                    # [b] -> int64 [n_seg]
    U: List[List[List[np.ndarray]]]           # [b][kv][S] -> [L][r]
    sigma: List[List[List[np.ndarray]]]       # [b][kv][S] -> [r]
    gate: List[List[List[np.ndarray]]]        # [b][kv][S] -> [r]
    Vh: List[List[List[np.ndarray]]]          # [b][kv][S] -> [r][2d] (joint) or [r][d] (keys, separate)
    basis: str = "joint"
    U_V: List = None                          # separate bases: [b][kv][S] -> [L][r]
    sigma_V: List = None                      # [b][kv][S] -> [r]
    Vh_V: List = None                         # [b][kv][S] -> [r][d]
    key_scale: List = None                    # folded routing: [b][kv] -> [n_seg] float32
    fold: List = None                         # folded routing: [kv] -> [d][d] fp64

    def n_seg(self, b: int) -> int:
        return len(self.seg_off[b]) - 1

    def span_len(self, b: int) -> np.ndarray:
        so = self.seg_off[b]
        return (so[1:] - so[:-1] - 1).astype(np.int64)


def build_cache(k, v, s, thr, P, rank_req, gate, *, n_sink, n_recent, lo, hi, dtype,
                factor_spans=None, rank_cap="full", basis="joint", sealed=False) -> OracleCache:
    """Build the mixed-resolution cache from stored K/V [B][Hkv][T][d], surprisal
    [B][T], boundary thresholds [B], projections [Hkv][d][d], requested ranks
    [B][>=n_seg] and gates [B][Hkv][>=n_seg][>=r].

    Reading: rank r_S = min(requested, L_S, 2d) (``span_ranks``), shared by
    the span's KV heads; gates are applied at decode, not folded into the
    factors.  Variants: ``rank_cap="half"`` caps r_S at ceil(L_S / 2);
    ``basis="separate"`` factors keys and values separately (r_S <= d), with
    the same gate vector on both.  The folded-routing fields (fold matrix and
    per-span key scales) are always filled.

    ``factor_spans`` (optional): {(b, kv head): span indices}; only those spans
    get factors (the others hold None and must not be expanded).  This skips
    work only; every value computed is the same.

    ``sealed``: the layout of a context during decode (``sealed_segment``):
    only sealed spans, a longer full-resolution tail.
    """
    B, Hkv, T, d = k.shape
    sep = basis == "separate"
    seg_offs, full_idx, fk, fv, sk, sv, rh, ranks, Us, sigs, gts, Vhs = ([] for _ in range(12))
    UVs, sVs, VVs, kss = [], [], [], []
    for b in range(B):
        seg = sealed_segment if sealed else segment
        so = seg(s[b], float(thr[b]), n_sink, n_recent, lo, hi)
        n_seg = len(so) - 1
        L = (so[1:] - so[:-1] - 1).astype(np.int64)
        r = span_ranks(rank_req[b][:n_seg], L, d, rank_cap, basis)
        fi = full_res_tokens(so, n_sink, T)
        seg_offs.append(so)
        full_idx.append(fi)
        ranks.append(r)
        fk_b, fv_b, sk_b, sv_b, rh_b, U_b, sg_b, g_b, Vh_b, UV_b, sV_b, VV_b, ks_b = ([] for _ in range(13))
        for h in range(Hkv):
            kk = np.asarray(k[b, h], np.float64)
            vv = np.asarray(v[b, h], np.float64)
            fk_b.append(kk[fi].copy())
            fv_b.append(vv[fi].copy())
            kbar, vbar = span_summaries(kk, vv, np.asarray(s[b], np.float64), so)
            sk_b.append(storage_round(kbar, dtype))
            sv_b.append(storage_round(vbar, dtype))
            rh_b.append(storage_round(routing_keys(kbar, P[h]), dtype))
            ks_b.append(key_scales(kbar, P[h]))
            Uh, sgh, gh, Vhh, UVh, sVh, VVh = [], [], [], [], [], [], []
            want = None if factor_spans is None else set(int(i) for i in factor_spans.get((b, h), ()))
            for i in range(n_seg):
                if want is not None and i not in want:
                    for lst in (Uh, sgh, gh, Vhh, UVh, sVh, VVh):
                        lst.append(None)
                    continue
                lo_t, hi_t = int(so[i]) + 1, int(so[i + 1])
                ri = int(r[i])
                if sep:
                    (Ui, si, Vi), (Uv, sv_, Vv) = span_factors_separate(kk[lo_t:hi_t], vv[lo_t:hi_t], ri)
                    UVh.append(storage_round(Uv, dtype))
                    sVh.append(sv_.copy() if dtype == "f64" else sv_.astype(np.float32).astype(np.float64))
                    VVh.append(storage_round(Vv, dtype))
                else:
                    Ui, si, Vi = span_factors(kk[lo_t:hi_t], vv[lo_t:hi_t], ri)
                    UVh.append(None); sVh.append(None); VVh.append(None)
                Uh.append(storage_round(Ui, dtype))
                sgh.append(si.copy() if dtype == "f64" else si.astype(np.float32).astype(np.float64))
                gh.append(np.asarray(gate[b][h][i][:ri], np.float32).astype(np.float64))
                Vhh.append(storage_round(Vi, dtype))
            U_b.append(Uh); sg_b.append(sgh); g_b.append(gh); Vh_b.append(Vhh)
            UV_b.append(UVh); sV_b.append(sVh); VV_b.append(VVh)
        fk.append(fk_b); fv.append(fv_b); sk.append(sk_b); sv.append(sv_b); rh.append(rh_b)
        Us.append(U_b); sigs.append(sg_b); gts.append(g_b); Vhs.append(Vh_b)
        UVs.append(UV_b); sVs.append(sV_b); VVs.append(VV_b); kss.append(ks_b)
    folds = [fold_matrix(P[h]) for h in range(Hkv)]
    return OracleCache(dtype, n_sink, T, d, seg_offs, full_idx, fk, fv, sk, sv, rh, ranks, Us, sigs, gts, Vhs,
                       basis=basis, U_V=UVs, sigma_V=sVs, Vh_V=VVs, key_scale=kss, fold=folds)


# --------------------------------------------------------------------------
# [de-3] / [zh-3]: routing and expansion decision
# --------------------------------------------------------------------------
def route_scores(q, rho) -> np.ndarray:
    """Canonical float32 routing score z[h][S] = sum_i q[h][i] * rho[S][i].

    Evaluated in float32 from the stored values, sequentially over i = 0..d-1,
    each product and each sum rounded to float32 separately (no fused
    multiply-add).  This fixes one evaluation order so the decision below is a
    function of the stored bits alone.
    """
    qf = np.asarray(q, dtype=np.float32)
    rf = np.asarray(rho, dtype=np.float32)
    z = np.zeros((qf.shape[0], rf.shape[0]), dtype=np.float32)
    for i in range(qf.shape[1]):
        prod = np.multiply.outer(qf[:, i], rf[:, i])      # float32 products
        z = np.add(z, prod, dtype=np.float32)               # float32 sums
    return z


def route(q, rho, theta) -> np.ndarray:
    """Expansion decisions e[h][S] = (z[h][S] > theta[h]).

    [de-3]/[zh-3]: a sigmoid relevance gate gives the probability that a span
    matters; a learned per-head (and per-layer) threshold decides expansion.
    Reading: sigma(z) > tau  <=>  z > logit(tau) = theta, compared strictly in
    float32; theta = +/-inf is allowed.
    """
    z = route_scores(q, rho)
    th = np.asarray(theta, dtype=np.float32)[:, None]
    return z > th


def compact(decisions: np.ndarray, group: int):
    """Per KV head: ascending list of spans that any query head of the group
    expands, a group-bit head mask per list entry, and the count.

    ``decisions``: [Hq][n_seg] bool.  Returns (lists, masks) as python lists
    over KV heads of int64 / int64 arrays.  Reading: decisions are per query
    head; rebuild happens once per KV head for the union of its group.
    """
    Hq, n = decisions.shape
    lists, masks = [], []
    for kv in range(Hq // group):
        dk = decisions[kv * group:(kv + 1) * group]
        bits = np.zeros(n, dtype=np.int64)
        for g in range(group):
            bits |= dk[g].astype(np.int64) << g
        idx = np.nonzero(bits)[0].astype(np.int64)
        lists.append(idx)
        masks.append(bits[idx])
    return lists, masks


def reconstruct(U, sigma, gate, Vh, d: int):
    """Token-level K/V of one expanded span: U diag(sigma * gate) Vh, split into
    the key part (first d columns) and the value part (last d).

    [de-2]/[zh-2]: soft gates on the singular values set the span's effective
    rank; [de-3]/[zh-3]: selected spans are rebuilt at token level.
    """
    scaled = np.asarray(sigma, np.float64) * np.asarray(gate, np.float64)
    M = np.asarray(U, np.float64) @ (scaled[:, None] * np.asarray(Vh, np.float64))
    return M[:, :d], M[:, d:]


def reconstruct_span(cache: "OracleCache", b: int, kv: int, S: int):
    """Token-level (K, V) of span S from the cache's factors: one joint basis
    (``reconstruct``), or separate key and value bases U_K diag(sigma_K * g)
    Vh_K and U_V diag(sigma_V * g) Vh_V."""
    d = cache.d
    if cache.basis != "separate":
        return reconstruct(cache.U[b][kv][S], cache.sigma[b][kv][S], cache.gate[b][kv][S], cache.Vh[b][kv][S], d)
    g = np.asarray(cache.gate[b][kv][S], np.float64)
    K = np.asarray(cache.U[b][kv][S]) @ ((np.asarray(cache.sigma[b][kv][S]) * g)[:, None] * np.asarray(cache.Vh[b][kv][S]))
    V = np.asarray(cache.U_V[b][kv][S]) @ ((np.asarray(cache.sigma_V[b][kv][S]) * g)[:, None]
                                           * np.asarray(cache.Vh_V[b][kv][S]))
    return K, V


def _softmax_pool(logits: np.ndarray, values: np.ndarray) -> np.ndarray:
    m = logits.max()
    p = np.exp(logits - m)
    return (p[:, None] * values).sum(axis=0) / p.sum()


def mixed_attention(cache: OracleCache, b: int, q_b, decisions_b, group: int) -> np.ndarray:
    """Decode attention of sequence b over its mixed-resolution memory.

    [de-3]/[zh-3]: anchors contribute full key/value pairs, unexpanded spans
    their coarse summary with a size correction, expanded spans their
    reconstructed token-level pairs.  Readings: the sink and the recent window
    are full resolution too; each query head uses its own decisions (a span
    expanded for a group sibling but not for this head contributes its summary
    here); logits are q.k / sqrt(d), plus ln|S| on summary entries; one fp64
    softmax over all entries.

    ``q_b``: [Hq][d] stored query; ``decisions_b``: [Hq][n_seg] bool.
    Returns [Hq][d] float32.
    """
    q_b = np.asarray(q_b, np.float64)
    Hq, d = q_b.shape
    c = 1.0 / math.sqrt(d)
    n_seg = cache.n_seg(b)
    L = cache.span_len(b)
    out = np.zeros((Hq, d), np.float32)
    for kv in range(Hq // group):
        heads = range(kv * group, (kv + 1) * group)
        union = np.zeros(n_seg, dtype=bool)
        for h in heads:
            union |= decisions_b[h]
        rebuilt = {}
        for S in np.nonzero(union)[0].tolist():
            rebuilt[S] = reconstruct_span(cache, b, kv, S)
        for h in heads:
            qh = q_b[h]
            keys = [cache.full_k[b][kv]]
            vals = [cache.full_v[b][kv]]
            extra = [np.zeros(cache.full_k[b][kv].shape[0])]
            summ = ~decisions_b[h]
            if summ.any():
                keys.append(cache.sum_k[b][kv][summ])
                vals.append(cache.sum_v[b][kv][summ])
                extra.append(np.log(L[summ].astype(np.float64)) if SIZE_CORRECTION else np.zeros(int(summ.sum())))
            for S in np.nonzero(decisions_b[h])[0].tolist():
                kh, vh = rebuilt[S]
                keys.append(kh)
                vals.append(vh)
                extra.append(np.zeros(kh.shape[0]))
            K = np.concatenate(keys, axis=0)
            V = np.concatenate(vals, axis=0)
            logits = c * (K @ qh) + np.concatenate(extra)
            out[h] = _softmax_pool(logits, V).astype(np.float32)
    return out


def mixed_attention_all(cache: OracleCache, q, decisions, group: int) -> np.ndarray:
    """``mixed_attention`` for every sequence: q [B][Hq][d], decisions
    [b] -> [Hq][n_seg_b]; returns [B][Hq][d] float32."""
    return np.stack([mixed_attention(cache, b, q[b], decisions[b], group) for b in range(len(decisions))])


def dense_attention(q, K, V, group: int) -> np.ndarray:
    """Plain softmax attention of one sequence over all T stored tokens (fp64).

    q [Hq][d], K/V [Hkv][T][d] -> [Hq][d] float32.  Textbook definition, used
    as the special case the method reduces to when every span is expanded at
    full rank with unit gates.
    """
    q = np.asarray(q, np.float64)
    Hq, d = q.shape
    out = np.zeros((Hq, d), np.float32)
    for h in range(Hq):
        kv = h // group
        Kh = np.asarray(K[kv], np.float64)
        Vh = np.asarray(V[kv], np.float64)
        out[h] = _softmax_pool((Kh @ q[h]) / math.sqrt(d), Vh).astype(np.float32)
    return out
