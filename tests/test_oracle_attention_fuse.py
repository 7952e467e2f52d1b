"""Pins of the oracle's window attention (O3), fusion (O4) and budgets (O5).

Window attention is checked against torch's scaled_dot_product_attention in
float64 on the CPU (a library routine: with V = identity it returns the
attention matrix itself) and against the equal-keys closed form, which fixes
the causal mask's orientation.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import infokv

rng = np.random.default_rng(99)


def sdpa_window_attention(q, k):
    """Per-head window attention from torch SDPA (float64 CPU), V = identity."""
    Hq, w, d = q.shape
    Hkv, n, _ = k.shape
    G = Hq // Hkv
    pos = n - w + np.arange(w)
    mask = torch.from_numpy(np.arange(n)[None, :] <= pos[:, None])
    eye = torch.eye(n, dtype=torch.float64)
    out = []
    for h in range(Hq):
        P = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[h])[None], torch.from_numpy(k[h // G])[None],
            eye[None], attn_mask=mask[None])[0]
        out.append(P.numpy().mean(axis=0))
    return np.stack(out)


@pytest.mark.parametrize("Hq,Hkv,n,w,d", [(4, 2, 40, 8, 16), (6, 2, 33, 33, 8), (2, 2, 70, 1, 4)])
def test_window_attention_matches_sdpa(Hq, Hkv, n, w, d):
    q = rng.normal(size=(Hq, w, d))
    k = rng.normal(size=(Hkv, n, d))
    A_h = infokv.window_attention(q, k, per_query_head=True)
    ref = sdpa_window_attention(q, k)
    np.testing.assert_allclose(A_h, ref, rtol=1e-12, atol=1e-15)
    A_g = infokv.window_attention(q, k)
    G = Hq // Hkv
    np.testing.assert_allclose(A_g, ref.reshape(Hkv, G, n).mean(axis=1), rtol=1e-12, atol=1e-15)


def test_window_attention_sums_to_one():
    q = rng.normal(size=(8, 16, 32))
    k = rng.normal(size=(2, 300, 32))
    np.testing.assert_allclose(infokv.window_attention(q, k).sum(axis=1), 1.0, atol=1e-12)
    np.testing.assert_allclose(infokv.window_attention(q, k, per_query_head=True).sum(axis=1),
                               1.0, atol=1e-12)


def test_equal_keys_closed_form_and_grouping(golden):
    # group 1 has equal keys (closed form); group 0 is random.  A wrong head ->
    # group map (h % Hkv instead of h // G) would mix group 0 into group 1.
    n, w, d = 8, 4, 5
    q = rng.normal(size=(4, w, d))
    k = rng.normal(size=(2, n, d))
    k[1] = rng.normal(size=d)[None, :]
    A = infokv.window_attention(q, k)
    np.testing.assert_allclose(A[1], golden["window_attention_equal_keys_n8_w4"], atol=1e-15)
    assert np.abs(A[0] - A[1]).max() > 1e-3


def test_scale_argument():
    q = rng.normal(size=(2, 4, 8))
    k = rng.normal(size=(1, 20, 8))
    a1 = infokv.window_attention(q, k, scale=1 / math.sqrt(8))
    a2 = infokv.window_attention(q * 2.0, k, scale=0.5 / math.sqrt(8))
    np.testing.assert_allclose(a1, a2, atol=1e-15)


def test_fuse_sums_to_one_and_special_cases():
    Hkv, n = 3, 200
    A = rng.random((Hkv, n))
    A /= A.sum(axis=1, keepdims=True)
    D = 1.0 + 2.0 * rng.random(n)
    H = 5.0 * rng.random(n)
    S, Ebar, E, sigma = infokv.fuse_scores(A, D, H, 0.9)
    np.testing.assert_allclose(S.sum(axis=1), 1.0, atol=1e-12)
    np.testing.assert_allclose(sigma, scipy.special.softmax(D * H), atol=1e-15)
    assert abs(Ebar - np.mean(D * H)) < 1e-12
    S1, *_ = infokv.fuse_scores(A, D, H, 1.0)
    np.testing.assert_array_equal(S1, A)                       # attention only
    S0, *_ = infokv.fuse_scores(A, D, H, 0.0)
    np.testing.assert_allclose(S0, np.broadcast_to(S0[0], S0.shape), atol=0)
    Sc, *_ = infokv.fuse_scores(A, np.full(n, 2.0), np.full(n, 1.5), 0.0)
    np.testing.assert_allclose(Sc, 1.0 / n, atol=1e-15)        # constant E


def test_uniform_budget():
    assert infokv.uniform_budget(0.25, 512) == 128
    assert infokv.uniform_budget(0.4, 16384) == 6553
    assert infokv.uniform_budget(0.2, 32768) == 6553
    assert infokv.uniform_budget(0.25, 102400) == 25600


def test_adaptive_budget(golden):
    k = infokv.adaptive_budget([1.0, 2.0, 3.0], 100, 0, 1000)
    assert k.tolist() == golden["adaptive_budget_123_B100"]
    k = infokv.adaptive_budget([5.0, 5.0, 5.0], 10, 0, 1000)
    assert k.tolist() == golden["adaptive_budget_equal_L3_B10"]
    e = rng.random(32).astype(np.float32) + 0.5
    k = infokv.adaptive_budget(e, 262144, 32, 65536)
    assert k.sum() == 262144
    assert np.all(np.diff(k[np.argsort(e, kind="stable")]) >= -1)   # monotone up to the +1
    k = infokv.adaptive_budget(np.ones(32), 262144, 32, 65536)
    assert np.all(k == 8192)
