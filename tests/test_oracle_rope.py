"""Pins of the oracle's RoPE re-positioning ([SelKV] section 2, pipeline step 6).

  * d = 2: the single pair turns by (new - old) radians (frequency base^0 = 1),
    so (1, 0) goes to (cos, sin) of that angle.
  * d = 4: pair 1 (elements 1 and 3) turns by (new - old) * base^(-1/2), a
    closed form that fixes the frequency schedule base^(-2i/d) (a wrong
    exponent such as base^(-i/d) turns it by another angle).
  * Re-positioning a key embedded at position p to position p' equals embedding
    the raw key at p' (rotations compose): a wrong sign or a swapped pair half
    fails it.  It holds for any frequency family, so it does not fix the
    schedule; the d = 4 closed form does.
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


def test_four_dims_pair_one_frequency(golden):
    # row 0 holds (0, 1, 0, 0): pair 1 is (element 1, element 3) = (1, 0);
    # row 1 holds (1, 0, 0, 0): pair 0 turns by the whole shift (base^0 = 1)
    K = np.array([[[0.0, 1.0, 0.0, 0.0], [1.0, 0.0, 0.0, 0.0]]])
    out = selkv.rope_reposition(K, np.array([[3, 4]]), 10, 10000.0)     # shifts 7 and 7
    ang = golden["rope_d4_pair1_angle_base1e4_delta7"]
    np.testing.assert_allclose(out[0, 0], [0.0, math.cos(ang), 0.0, math.sin(ang)], rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[0, 1], [math.cos(7.0), 0.0, math.sin(7.0), 0.0], rtol=0, atol=1e-15)


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
