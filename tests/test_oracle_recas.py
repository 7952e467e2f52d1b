"""Pins of the oracle's active-set decoding ([RECAS] sections 2.B and 2.C).

  * Scores against per-head brute force (Python loops over the group's heads):
    a wrong head-to-group map or a mean instead of a max fails it.
  * The active set against a plain sort on (-score, index).
  * With every entry active the step is plain decode attention over the cache.
  * The formal bound of section 2.B, ||o - o_active|| <= 2 * V_max * delta,
    where delta is the attention mass outside the active set, on random sets.
  * A large utility on chosen entries puts exactly them into the active set.
  * Decode attention itself (the function the active step calls): lse by a
    closed form and by scipy's logsumexp, o by torch's SDPA with the bias as
    an additive mask.
"""
import math

import numpy as np
import pytest

from oracle import infokv, recas

rng = np.random.default_rng(4321)


def test_scores_brute_force():
    Hq, Hkv, n, d = 6, 2, 40, 8
    q, K = rng.normal(size=(Hq, d)), rng.normal(size=(Hkv, n, d))
    u = rng.normal(size=(Hkv, n))
    s = recas.active_scores(q, K, u, 0.5)
    G = Hq // Hkv
    for g in range(Hkv):
        for j in range(n):
            best = max(sum(q[h, e] * K[g, j, e] for e in range(d)) / math.sqrt(d)
                       for h in range(g * G, (g + 1) * G))
            assert abs(s[g, j] - (best + 0.5 * u[g, j])) < 1e-12


def test_active_set_brute_force():
    s = rng.normal(size=(3, 50)).astype(np.float32)
    s[1, 10] = s[1, 20] = s[1, 30] = 5.0                    # ties: lower index first
    a = recas.active_set(s, 2)
    for g in range(3):
        order = sorted(range(50), key=lambda j: (-float(s[g, j]), j))[:2]
        assert a[g].tolist() == sorted(order)
    assert a[1].tolist() == [10, 20]


def test_all_active_is_plain_decode():
    Hq, Hkv, n, d = 8, 2, 70, 16
    q, K, V = rng.normal(size=(Hq, d)), rng.normal(size=(Hkv, n, d)), rng.normal(size=(Hkv, n, d))
    lr = rng.random((Hkv, n))
    allrows = np.tile(np.arange(n), (Hkv, 1))
    o1, l1 = recas.active_decode(q, K, V, allrows, lr, 0.7)
    o2, l2 = infokv.decode_attention(q, K, V, lr, 0.7)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)


def test_formal_bound_on_active_sets():
    Hq, Hkv, n, d = 4, 2, 200, 16
    for trial in range(20):
        q = rng.normal(size=(Hq, d)) * 2
        K, V = rng.normal(size=(Hkv, n, d)), rng.normal(size=(Hkv, n, d))
        k = int(rng.integers(1, n + 1))
        act = recas.active_set(recas.active_scores(q, K).astype(np.float32), k)
        o_act, _ = recas.active_decode(q, K, V, act)
        o, o2, delta, vmax = infokv.dropped_mass_bound(q, K, V, act)
        np.testing.assert_allclose(o2, o_act, rtol=1e-12, atol=1e-14)
        assert np.all(np.linalg.norm(o - o_act, axis=1) <= 2 * vmax * delta + 1e-12)


def test_utility_selects_its_entries():
    Hq, Hkv, n, d = 4, 1, 64, 8
    q, K = rng.normal(size=(Hq, d)), rng.normal(size=(Hkv, n, d))
    u = np.zeros((Hkv, n))
    u[0, [3, 17, 40]] = 1e6
    a = recas.active_set(recas.active_scores(q, K, u, 1.0).astype(np.float32), 3)
    assert a[0].tolist() == [3, 17, 40]


def test_decode_lse_closed_form(golden):
    # two keys with the logit 10; ln R = (0, ln 3) adds ln 3 to the second
    q = np.array([[2.0, 0.0, 0.0, 0.0]])
    K = np.array([[[10.0, 0.0, 0.0, 0.0], [10.0, 0.0, 0.0, 0.0]]])
    V = np.array([[[4.0, 0.0, 0.0, 0.0], [0.0, 8.0, 0.0, 0.0]]])
    lnR = np.array([[0.0, math.log(3.0)]])
    o, lse = infokv.decode_attention(q, K, V, lnR, 1.0, scale=0.5)
    assert abs(lse[0] - golden["decode_lse_two_keys_bias_ln3"]) < 1e-13
    np.testing.assert_allclose(o[0], [1.0, 6.0, 0.0, 0.0], rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_decode_matches_library_logsumexp_and_sdpa(seed):
    """lse against scipy's logsumexp of the biased logits, o against torch's
    scaled_dot_product_attention (float64, CPU) with alpha * ln R as an additive
    mask; both are library routines, not the oracle's own steps."""
    import scipy.special
    import torch
    r = np.random.default_rng(seed)
    Hq, Hkv, n, d = 8, 2, 90, 16
    q = r.normal(size=(Hq, d)) * 3.0 + 2.0          # large logits: lse far from 0
    K, V = r.normal(size=(Hkv, n, d)), r.normal(size=(Hkv, n, d))
    lnR = r.random((Hkv, n)) * 2.0
    alpha = 0.7
    o, lse = infokv.decode_attention(q, K, V, lnR, alpha)
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(d)
    for h in range(Hq):
        g = h // G
        logits = (K[g] @ q[h]) * sc + alpha * lnR[g]
        assert abs(lse[h] - scipy.special.logsumexp(logits)) <= 1e-12 * max(1.0, abs(lse[h]))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[h])[None, None], torch.from_numpy(K[g])[None],
            torch.from_numpy(V[g])[None], attn_mask=torch.from_numpy(alpha * lnR[g])[None, None])
        np.testing.assert_allclose(o[h], ref[0, 0].numpy(), rtol=1e-12, atol=1e-13)
    assert np.abs(lse).min() > 1.0
