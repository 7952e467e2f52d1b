"""Pins of the oracle's top-k entropy (O1) and representation distance (O2).

Each test compares against something other than the oracle's own formula: a
closed form derived from the definition, a library routine (scipy), or a
brute-force pure-Python evaluation on tiny rows with a different selection
method (full sort instead of partition).
"""
import math

import numpy as np
import pytest
import scipy.spatial.distance
import scipy.stats

from oracle import infokv

rng = np.random.default_rng(1234)


@pytest.mark.parametrize("k", [64, 256])
def test_flat_row_is_log_k(golden, k):
    row = np.full((3, 1000), 0.75)
    H = infokv.topk_entropy(row, k)
    np.testing.assert_allclose(H, golden[f"entropy_flat_k{k}"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("k", [64, 256])
def test_two_level_closed_form_with_junk_below(golden, k):
    # top k: k/2 at x, k/2 at x - ln 3; everything else just below (must be ignored,
    # which catches a missing top-k restriction or a missing renormalisation)
    V = 4 * k + 17
    row = rng.uniform(-1.0, 0.85, size=V)   # just below the lower level 2 - ln 3
    cols = rng.permutation(V)[:k]
    row[cols[: k // 2]] = 2.0
    row[cols[k // 2:]] = 2.0 - math.log(3.0)
    H = infokv.topk_entropy(row[None, :], k)[0]
    assert abs(H - golden[f"entropy_two_level_k{k}"]) < 1e-12


def test_dominant_logit_gives_zero():
    row = rng.normal(size=(2, 5000))
    row[:, 7] = 200.0
    H = infokv.topk_entropy(row, 256)
    assert np.all(H >= 0) and np.all(H < 1e-60)


def test_ties_straddling_threshold(golden):
    # 10 values above, then 500 equal values across the k-th place: the multiset
    # is 10 high + 54 ties, whichever ties are picked.
    k = 64
    row = np.full(600, 1.0)
    row[:10] = 1.0 + math.log(3.0)
    row[560:] = -5.0
    H = infokv.topk_entropy(row[None, :], k)[0]
    w_hi, w_lo = 3.0, 1.0
    Z = 10 * w_hi + 54 * w_lo
    expect = -(10 * (w_hi / Z) * math.log(w_hi / Z) + 54 * (w_lo / Z) * math.log(w_lo / Z))
    assert abs(H - expect) < 1e-12


def test_bounds_and_shift_invariance():
    z = 4.0 * rng.normal(size=(20, 3000))
    for k in (1, 64, 256, 3000):
        H = infokv.topk_entropy(z, k)
        assert np.all(H >= -1e-12) and np.all(H <= math.log(k) + 1e-12)
        np.testing.assert_allclose(infokv.topk_entropy(z + 37.5, k), H, atol=1e-10)
    assert np.all(infokv.topk_entropy(z, 1) == 0.0)


def test_matches_scipy_entropy_of_sorted_topk():
    z = 4.0 * rng.normal(size=(16, 4096))
    z[:, :5] += 12.0
    for k in (64, 256):
        H = infokv.topk_entropy(z, k)
        for i in range(z.shape[0]):
            top = np.sort(z[i])[-k:]
            p = np.exp(top - top.max())
            assert abs(H[i] - scipy.stats.entropy(p)) < 1e-10


def test_masked_logits_fewer_than_k_finite():
    """-inf logits (a masked vocabulary): with fewer than k finite values the
    zero-probability entries contribute 0 (the limit of p ln p), so H is the
    entropy of the finite part (scipy.stats.entropy, which uses the same
    convention).  A row with no finite logit has no entropy."""
    z = 4.0 * rng.normal(size=(6, 500))
    z[:, 40:] = -np.inf                          # 40 finite values per row
    z[5, :] = -np.inf
    H = infokv.topk_entropy(z, 200)
    for i in range(5):
        fin = z[i][np.isfinite(z[i])]
        assert abs(H[i] - scipy.stats.entropy(np.exp(fin - fin.max()))) < 1e-10
    assert np.isnan(H[5])
    # the same rows with the masked entries simply absent
    np.testing.assert_allclose(H[:5], infokv.topk_entropy(z[:5, :40], 40), atol=1e-12)


def test_brute_force_python():
    z = rng.normal(size=(4, 40))
    k = 7
    H = infokv.topk_entropy(z, k)
    for i in range(4):
        top = sorted(z[i].tolist(), reverse=True)[:k]
        Z = sum(math.exp(t) for t in top)
        expect = -sum(math.exp(t) / Z * math.log(math.exp(t) / Z) for t in top)
        assert abs(H[i] - expect) < 1e-12


def test_distance_closed_forms(golden):
    a = rng.normal(size=(5, 300))
    D = infokv.repr_distance(a, a, tau=1.0)
    np.testing.assert_allclose(D, golden["distance_identical"], atol=1e-14)
    D = infokv.repr_distance(-a, a, tau=1.0)
    np.testing.assert_allclose(D, golden["distance_opposite"], atol=1e-14)
    b = np.zeros_like(a)
    b[:, :150] = a[:, :150]
    c = np.zeros_like(a)
    c[:, 150:] = a[:, 150:]
    D = infokv.repr_distance(b, c, tau=1.0)
    np.testing.assert_allclose(D, golden["distance_orthogonal"], atol=1e-14)


def test_distance_matches_scipy_cosine_and_scale_invariance():
    a = rng.normal(size=(30, 256))
    b = 0.6 * a + 0.8 * rng.normal(size=(30, 256))
    D = infokv.repr_distance(a, b, tau=0.5)
    for i in range(30):
        assert abs(D[i] - (scipy.spatial.distance.cosine(a[i], b[i]) + 0.5)) < 1e-12
    np.testing.assert_allclose(infokv.repr_distance(3.0 * a, 0.25 * b, 0.5), D, atol=1e-12)
    # argument order does not matter for a cosine
    np.testing.assert_allclose(infokv.repr_distance(b, a, 0.5), D, atol=1e-14)


def test_distance_zero_vector_reading():
    a = np.zeros((1, 16))
    b = np.ones((1, 16))
    assert infokv.repr_distance(a, b, 1.0)[0] == 2.0
