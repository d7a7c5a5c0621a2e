"""Pins of the oracle's reading variants (the rank cap 1/2 L, separate key and
value bases, routing folded onto the attention summary key) against things
other than the oracle itself: hand-worked values, Eckart-Young, the
optimality of per-part truncation over the joint one, fp64 brute force off
the rounding band, and the dense-attention special case."""
import math

import numpy as np

import oracle as O


def test_span_ranks_hand_values():
    L = np.array([1, 2, 3, 17, 128, 100])
    req = np.array([5, 5, 5, 64, 200, 7])
    assert O.span_ranks(req, L, 128).tolist() == [1, 2, 3, 17, 128, 7]
    assert O.span_ranks(req, L, 128, rank_cap="half").tolist() == [1, 1, 2, 9, 64, 7]
    assert O.span_ranks(req, L, 64, basis="separate").tolist() == [1, 2, 3, 17, 64, 7]
    assert O.span_ranks(req, L, 64, rank_cap="half", basis="separate").tolist() == [1, 1, 2, 9, 64, 7]


def test_separate_factors_eckart_young_and_no_swap():
    rng = np.random.default_rng(21)
    for L, d, r in [(9, 8, 3), (17, 16, 5), (6, 16, 6), (30, 8, 8)]:
        K = rng.standard_normal((L, d))
        V = 3.0 * rng.standard_normal((L, d)) + 1.0       # distinct from K
        (Uk, sk, Vk), (Uv, sv, Vv) = O.span_factors_separate(K, V, r)
        for M, U, sg, Vh in ((K, Uk, sk, Vk), (V, Uv, sv, Vv)):
            ev = np.sort(np.linalg.eigvalsh(M.T @ M))[::-1]      # squared singular values, another routine
            tail = ev[r:].clip(min=0).sum()
            err = np.linalg.norm(M - (U * sg) @ Vh) ** 2
            assert abs(err - tail) <= 1e-9 * max(1.0, (M * M).sum())
            assert np.allclose(U.T @ U, np.eye(r), atol=1e-10) and np.allclose(Vh @ Vh.T, np.eye(r), atol=1e-10)
        # per-part truncation is never worse than truncating the joint matrix at the same rank
        Uj, sj, Vj = O.span_factors(K, V, r)
        joint = np.linalg.norm(np.concatenate([K, V], 1) - (Uj * sj) @ Vj) ** 2
        sep = np.linalg.norm(K - (Uk * sk) @ Vk) ** 2 + np.linalg.norm(V - (Uv * sv) @ Vv) ** 2
        assert sep <= joint * (1 + 1e-12) + 1e-12


def test_separate_bases_full_rank_all_expanded_is_dense_attention():
    rng = np.random.default_rng(22)
    B, Hkv, T, d, G = 1, 2, 48, 8, 2
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    s = rng.lognormal(0, 1, (B, T))
    P = rng.standard_normal((Hkv, d, d)) / math.sqrt(d)
    cap = T
    c = O.build_cache(k, v, s, np.array([np.quantile(s[0], 0.7)]), P, np.full((B, cap), 64),
                      np.ones((B, Hkv, cap, 64)), n_sink=2, n_recent=4, lo=1, hi=8, dtype="f64", basis="separate")
    assert c.n_seg(0) > 3
    L = c.span_len(0)
    assert np.all(c.rank[0] == np.minimum(L, d))
    q = rng.standard_normal((Hkv * G, d))
    dec = np.ones((Hkv * G, c.n_seg(0)), bool)
    out = O.mixed_attention(c, 0, q, dec, G)
    ref = O.dense_attention(q, k[0], v[0], G)
    assert np.abs(out - ref).max() <= 1e-6
    # and the rebuilt spans are the stored K and V themselves (not swapped)
    for S in range(c.n_seg(0)):
        Kh, Vh = O.reconstruct_span(c, 0, 1, S)
        t0, t1 = int(c.seg_off[0][S]) + 1, int(c.seg_off[0][S + 1])
        assert np.allclose(Kh, k[0, 1, t0:t1], atol=1e-10) and np.allclose(Vh, v[0, 1, t0:t1], atol=1e-10)


def test_rank_cap_half_stays_within_cap_and_eckart_young():
    rng = np.random.default_rng(23)
    B, Hkv, T, d = 1, 1, 200, 8
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    s = rng.lognormal(0, 1, (B, T))
    c = O.build_cache(k, v, s, np.array([np.quantile(s[0], 0.85)]), rng.standard_normal((Hkv, d, d)),
                      np.full((B, T), 64), np.ones((B, Hkv, T, 64)), n_sink=2, n_recent=4, lo=2, hi=20,
                      dtype="f64", rank_cap="half")
    L = c.span_len(0)
    assert np.all(c.rank[0] == (L + 1) // 2)
    for S in range(c.n_seg(0)):
        t0, t1 = int(c.seg_off[0][S]) + 1, int(c.seg_off[0][S + 1])
        M = np.concatenate([k[0, 0, t0:t1], v[0, 0, t0:t1]], 1)
        ev = np.sort(np.linalg.eigvalsh(M @ M.T))[::-1]
        Kh, Vh = O.reconstruct_span(c, 0, 0, S)
        err = np.linalg.norm(M - np.concatenate([Kh, Vh], 1)) ** 2
        assert abs(err - ev[int(c.rank[0][S]):].clip(min=0).sum()) <= 1e-9 * (M * M).sum()


def test_fold_matrix_and_query_match_library_products():
    rng = np.random.default_rng(24)
    P = rng.standard_normal((16, 16)) / 4
    M = O.fold_matrix(P)
    assert np.allclose(M, P.T @ P, rtol=1e-13, atol=1e-14)
    assert np.array_equal(M, M.T)                        # same products, same order: bitwise symmetric
    q = rng.standard_normal((3, 16)).astype(np.float32).astype(np.float64)
    qf = O.fold_query(M, q)
    ref = q @ M.T
    assert qf.dtype == np.float32
    assert np.all(np.abs(qf.astype(np.float64) - ref) <= 2.0 ** -23 * np.abs(ref) + 1e-30)


def test_key_scales_are_inverse_projected_norms():
    rng = np.random.default_rng(25)
    P = rng.standard_normal((8, 8))
    kb = rng.standard_normal((5, 8))
    kb[2] = 0.0
    sc = O.key_scales(kb, P)
    nrm = np.linalg.norm(kb @ P.T, axis=1)
    want = 1.0 / np.where(nrm > 0, nrm, 1.0)
    assert sc[2] == 0.0
    assert np.allclose(np.delete(sc, 2), np.delete(want, 2).astype(np.float32), rtol=2e-7)


def test_folded_route_order_golden():
    # z = fl32(1 + 2^-24) = 1 (ties to even), then fl32(1 * 3) = 3; evaluating
    # z * scale in higher precision would give 3 + 2^-22 instead
    qf = np.array([[1.0, 2.0 ** -24]], np.float32)
    kb = np.array([[1.0, 1.0]])
    z = O.route_scores_folded(qf, kb, np.array([3.0], np.float32))
    assert z.dtype == np.float32 and z[0, 0] == np.float32(3.0)
    assert np.float32((1.0 + 2.0 ** -24) * 3.0) != np.float32(3.0)


def test_folded_route_agrees_with_rho_route_and_fp64_off_band():
    rng = np.random.default_rng(26)
    d, G, n = 64, 4, 400
    P = rng.standard_normal((d, d)) / math.sqrt(d)
    kbar = rng.standard_normal((n, d))
    kbar_s = O.storage_round(kbar, "bf16")
    rho = O.storage_round(O.routing_keys(kbar, P), "bf16")
    sc = O.key_scales(kbar, P)
    M = O.fold_matrix(P)
    q = O.storage_round(rng.standard_normal((G, d)), "bf16")
    qf = O.fold_query(M, q)
    zf = O.route_scores_folded(qf, kbar_s, sc).astype(np.float64)
    zr = O.route_scores(q, rho).astype(np.float64)
    # both evaluate (P q) . normalize(P kbar); they differ by the storage roundings only
    assert np.abs(zf - zr).max() <= 0.05 * np.abs(zr).max()
    # fp64 brute force of the canonical definition, decisions off the rounding band
    exact = (qf.astype(np.float64) @ kbar_s.T) * sc.astype(np.float64)[None, :]
    u = 2.0 ** -24
    gam = d * u / (1 - d * u)
    band = (gam * (np.abs(qf.astype(np.float64)) @ np.abs(kbar_s).T) + u * np.abs(exact)) * sc[None, :] + 1e-30
    for th in np.quantile(exact, [0.1, 0.5, 0.9]):
        off = np.abs(exact - th) > band
        assert off.mean() > 0.99
        assert np.array_equal((zf > np.float32(th))[off], (exact > np.float32(th))[off])
