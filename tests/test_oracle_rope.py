"""Pins of the oracle's RoPE re-positioning ([SelKV] section 2, pipeline step 6).

  * d = 2: the single pair turns by (new - old) radians (frequency base^0 = 1),
    so (1, 0) goes to (cos, sin) of that angle.
  * Re-positioning a key embedded at position p to position p' equals embedding
    the raw key at p' (rotations compose): a wrong sign, a swapped pair half or
    a wrong frequency exponent fails it.
  * Zero shift is the identity; every pair keeps its norm.
"""
import math

import numpy as np

from oracle import selkv

rng = np.random.default_rng(77)


def test_two_dims_closed_form():
    K = np.array([[[1.0, 0.0], [0.0, 2.0]]])             # [1, 2, 2]
    out = selkv.rope_reposition(K, np.array([[5, 9]]), 2, 10000.0)
    # slot 0: 2 - 5 = -3 rad; slot 1: 3 - 9 = -6 rad
    np.testing.assert_allclose(out[0, 0], [math.cos(-3), math.sin(-3)], rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[0, 1], [-2 * math.sin(-6), 2 * math.cos(-6)], rtol=0, atol=1e-15)


def test_reposition_equals_embedding_at_the_new_position():
    Hkv, m, d, base = 3, 40, 64, 500000.0
    raw = rng.normal(size=(Hkv, m, d))
    old = np.sort(rng.choice(100000, size=(Hkv, m), replace=True), axis=1)
    emb = selkv.rope_apply(raw, old, base)
    out = selkv.rope_reposition(emb, old, 7, base)
    want = selkv.rope_apply(raw, np.tile(7 + np.arange(m), (Hkv, 1)), base)
    np.testing.assert_allclose(out, want, rtol=1e-9, atol=1e-9)


def test_identity_and_norms():
    K = rng.normal(size=(2, 30, 16))
    pos = np.tile(np.arange(30), (2, 1))
    np.testing.assert_allclose(selkv.rope_reposition(K, pos, 0, 10000.0), K, rtol=0, atol=0)
    out = selkv.rope_reposition(K, pos + 1000, 0, 10000.0)
    h = 8
    np.testing.assert_allclose(out[..., :h] ** 2 + out[..., h:] ** 2, K[..., :h] ** 2 + K[..., h:] ** 2,
                               rtol=1e-12)
