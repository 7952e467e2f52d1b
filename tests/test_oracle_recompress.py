"""Pins of the oracle's compression during decoding ([InfoKV] Technical detail:
compression at prefill and again every 1024 generated tokens).

  * Slot fusion against scipy's softmax row by row, and against the prefill
    fusion when every head's slots hold the same tokens (the two definitions
    then coincide: a dropped or misplaced head index, or a softmax over the
    wrong axis, breaks it).
  * A period whose kept slots are the whole previous cache is the prefill path
    over the longer sequence (the slot bookkeeping of E: old tokens keep D * H,
    new tokens get theirs appended, in position order).
  * Brute force: the kept slots are the top of S by a plain sort, and the
    gathered E / K / V are the kept slots' own values.
"""
import numpy as np
import pytest
import scipy.special

from oracle import infokv

rng = np.random.default_rng(1234)


def test_slot_softmax_rows_match_scipy():
    A = rng.random((3, 50))
    E = rng.normal(size=(3, 50)) * 3
    S, Ebar, sigma = infokv.fuse_scores_slots(A, E, 0.9)
    for g in range(3):
        np.testing.assert_allclose(sigma[g], scipy.special.softmax(E[g]), rtol=1e-13)
    np.testing.assert_allclose(S, 0.9 * A + 0.1 * sigma, rtol=1e-14)
    assert Ebar == pytest.approx(E.mean(), rel=1e-14)


def test_slot_softmax_is_per_head_under_far_apart_rows():
    # head 1's scores sit 2000 below head 0's: each head's softmax is its own,
    # so both rows still sum to one (a shared shift would underflow head 1)
    E = np.stack([rng.normal(size=40), rng.normal(size=40) - 2000.0])
    _, _, sigma = infokv.fuse_scores_slots(np.zeros((2, 40)), E, 0.5)
    np.testing.assert_allclose(sigma.sum(axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(sigma[1], scipy.special.softmax(E[1]), rtol=1e-12)


def test_slot_fusion_equals_prefill_fusion_for_shared_slots():
    n = 64
    A = rng.random((4, n))
    A /= A.sum(axis=1, keepdims=True)
    D = 1.0 + rng.random(n)
    H = rng.random(n) * 5
    S_pre, Ebar_pre, _, _ = infokv.fuse_scores(A, D, H, 0.9)
    S_slot, Ebar_slot, _ = infokv.fuse_scores_slots(A, np.tile(D * H, (4, 1)), 0.9)
    np.testing.assert_allclose(S_slot, S_pre, rtol=1e-13)
    assert Ebar_slot == pytest.approx(Ebar_pre, rel=1e-13)
    np.testing.assert_allclose(S_slot.sum(axis=1), 1.0, atol=1e-12)


def test_period_over_the_whole_cache_is_the_prefill_path():
    Hq, Hkv, d, w = 4, 2, 8, 4
    n_old, t = 30, 10
    n = n_old + t
    q = rng.normal(size=(Hq, w, d))
    K = rng.normal(size=(Hkv, n, d))
    V = rng.normal(size=(Hkv, n, d))
    D = 1.0 + rng.random(n)
    H = rng.random(n) * 4
    k_keep = 15
    # no compaction yet: the kept slots are tokens 0..n_old-1 of every head
    E_kept = np.tile(D[:n_old] * H[:n_old], (Hkv, 1))
    out = infokv.recompress_period(q, K, V, E_kept, D[n_old:], H[n_old:], 0.9, k_keep, w)
    A, S, S32, _, idx = infokv.infokv_layer(q, K, D, H, 0.9, k_keep, w)
    np.testing.assert_allclose(out["S"], S, rtol=1e-13)
    assert (out["idx"] == idx).all()
    Kc, Vc = infokv.compact(K, V, idx)
    assert (out["Kc"] == Kc).all() and (out["Vc"] == Vc).all()
    np.testing.assert_array_equal(out["E_next"], np.take_along_axis(np.tile(D * H, (Hkv, 1)),
                                                                    idx.astype(np.int64), axis=1))


def test_period_with_per_head_slots_brute_force():
    Hq, Hkv, d, w = 6, 3, 4, 3
    k_old, t, k_keep = 12, 5, 9
    n = k_old + t
    q = rng.normal(size=(Hq, w, d))
    K = rng.normal(size=(Hkv, n, d))
    V = rng.normal(size=(Hkv, n, d))
    E_kept = rng.normal(size=(Hkv, k_old))          # different per head
    D_new, H_new = 1.0 + rng.random(t), rng.random(t) * 3
    out = infokv.recompress_period(q, K, V, E_kept, D_new, H_new, 0.8, k_keep, w)
    for g in range(Hkv):
        E = list(E_kept[g]) + list(D_new * H_new)
        assert np.allclose(out["E"][g], E, rtol=0, atol=0)
        m = max(E)
        z = sum(np.exp(e - m) for e in E)
        S = [0.8 * out["A"][g, j] + 0.2 * np.exp(E[j] - m) / z for j in range(n)]
        np.testing.assert_allclose(out["S"][g], S, rtol=1e-13)
        S32 = np.float32(S)
        body = sorted(range(n - w), key=lambda j: (-float(S32[j]), j))[: k_keep - w]
        kept = sorted(body + list(range(n - w, n)))
        assert list(out["idx"][g]) == kept
        assert list(out["E_next"][g]) == [E[j] for j in kept]
        assert (out["Kc"][g] == K[g][kept]).all() and (out["Vc"][g] == V[g][kept]).all()
