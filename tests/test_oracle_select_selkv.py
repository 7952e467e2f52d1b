"""Pins of the oracle's selection and gather (O6, O7), the dropped-mass bound
(O8) and SelKV's merge path (O9).

Selection is checked against a brute-force Python sort of (-S, index) tuples
(a different method from the oracle's lexsort).  SelKV is pinned by the gate's
closed forms, special cases, and the duplicate-key construction, under which
compensated decode over the compacted cache equals full-cache attention.
"""
import math

import numpy as np
import pytest

from oracle import infokv, precision, selkv

rng = np.random.default_rng(7)


def brute_select(S, k, w):
    Hkv, n = S.shape
    out = []
    for g in range(Hkv):
        if k <= w:
            out.append(list(range(n - k, n)))
            continue
        ranked = sorted(range(n - w), key=lambda i: (-float(S[g, i]), i))
        out.append(sorted(ranked[: k - w] + list(range(n - w, n))))
    return np.array(out, dtype=np.int32)


@pytest.mark.parametrize("n,k,w,levels", [(50, 20, 5, 0), (64, 64, 8, 0), (40, 8, 8, 0),
                                          (100, 30, 4, 3), (37, 5, 8, 0), (90, 45, 0, 2)])
def test_select_matches_brute_force(n, k, w, levels):
    if levels:
        S = ((rng.integers(0, levels, size=(3, n)) + 1) / levels).astype(np.float32)
    else:
        S = rng.random((3, n)).astype(np.float32)
    idx = infokv.select_topk(S, k, w)
    np.testing.assert_array_equal(idx, brute_select(S, k, w))
    assert np.all(np.diff(idx, axis=1) > 0)


def test_select_special_cases():
    S = rng.random((2, 30)).astype(np.float32)
    np.testing.assert_array_equal(infokv.select_topk(S, 30, 4), np.tile(np.arange(30), (2, 1)))
    np.testing.assert_array_equal(infokv.select_topk(S, 4, 4), np.tile(np.arange(26, 30), (2, 1)))
    flat = np.ones((1, 20), dtype=np.float32)          # all tied -> lowest indices
    assert infokv.select_topk(flat, 7, 2).tolist() == [[0, 1, 2, 3, 4, 18, 19]]


def test_compact_is_bit_gather():
    K = rng.integers(0, 65535, size=(2, 10, 4), dtype=np.uint16)
    V = rng.integers(0, 65535, size=(2, 10, 4), dtype=np.uint16)
    idx = np.array([[0, 3, 9], [1, 2, 8]], dtype=np.int32)
    Kc, Vc = infokv.compact(K, V, idx)
    for g in range(2):
        for j in range(3):
            assert (Kc[g, j] == K[g, idx[g, j]]).all() and (Vc[g, j] == V[g, idx[g, j]]).all()
    Kc, Vc = infokv.compact(K, V, np.tile(np.arange(10, dtype=np.int32), (2, 1)))
    assert (Kc == K).all() and (Vc == V).all()


@pytest.mark.parametrize("seed", range(5))
def test_dropped_mass_bound_and_renormalised_output(seed):
    r = np.random.default_rng(seed)
    Hq, Hkv, n, d = 4, 2, 120, 16
    q = r.normal(size=(Hq, d)) * 2.0
    K = r.normal(size=(Hkv, n, d))
    V = r.normal(size=(Hkv, n, d)) * r.random((Hkv, n, 1)) * 3
    S = r.random((Hkv, n)).astype(np.float32)
    idx = infokv.select_topk(S, 40, 8)
    o, o2, delta, vmax = infokv.dropped_mass_bound(q, K, V, idx)
    assert np.all(np.linalg.norm(o - o2, axis=1) <= 2 * vmax * delta + 1e-12)
    assert np.all((delta > 0) & (delta < 1))
    # o' is exactly decode attention over the compacted cache
    Kc, Vc = infokv.compact(K, V, idx)
    oc, _ = infokv.decode_attention(q, Kc, Vc)
    np.testing.assert_allclose(o2, oc, atol=1e-12)
    # and the full output is decode attention over the full cache
    of, _ = infokv.decode_attention(q, K, V)
    np.testing.assert_allclose(o, of, atol=1e-12)


def test_dropped_mass_closed_form():
    # two keys with equal logits (q orthogonal to both): p = (1/2, 1/2); token 1
    # is evicted, so delta = 1/2.  Values (3, 4) and (0, 1): V_max = 5, o is
    # their mean, o' = v0, and ||o - o'|| = ||(v1 - v0) / 2|| = sqrt(9 + 9) / 2.
    q = np.array([[0.0, 0.0, 1.0]])
    K = np.array([[[1.0, 0.0, 0.0], [0.0, 1.0, 0.0]]])
    V = np.array([[[3.0, 4.0, 0.0], [0.0, 1.0, 0.0]]])
    o, o2, delta, vmax = infokv.dropped_mass_bound(q, K, V, np.array([[0]]))
    assert delta[0] == 0.5 and vmax[0] == 5.0
    np.testing.assert_allclose(o[0], [1.5, 2.5, 0.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o2[0], [3.0, 4.0, 0.0], rtol=0, atol=1e-15)
    assert abs(np.linalg.norm(o - o2) - math.sqrt(18.0) / 2) < 1e-14
    assert np.linalg.norm(o - o2) <= 2 * vmax[0] * delta[0]


def test_selkv_group_attention_is_the_group_mean_of_sdpa():
    """A_g (routing target and merge weight) is the mean over the group's heads
    of window attention, here rebuilt from torch's SDPA (float64, V = I); the
    route and merge of ``selkv_layer`` are re-run on that A_g."""
    import torch
    Hq, Hkv, n, d, w, m, bucket = 6, 2, 96, 8, 8, 30, 16
    q_win = rng.normal(size=(Hq, w, d)) * 2.0
    K = rng.normal(size=(Hkv, n, d))
    V = rng.normal(size=(Hkv, n, d))
    out = selkv.selkv_layer(q_win, K, V, m, w, bucket)
    G = Hq // Hkv
    pos = n - w + np.arange(w)
    mask = torch.from_numpy(np.arange(n)[None, :] <= pos[:, None])
    eye = torch.eye(n, dtype=torch.float64)
    A_h = np.stack([torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q_win[h])[None], torch.from_numpy(K[h // G])[None], eye[None],
        attn_mask=mask[None])[0].numpy().mean(axis=0) for h in range(Hq)])
    A_g = A_h.reshape(Hkv, G, n).mean(axis=1)
    np.testing.assert_allclose(out["A_g"], A_g, rtol=1e-12, atol=1e-15)
    assert np.abs(A_h.reshape(Hkv, G, n).max(axis=1) - A_g).max() > 1e-3   # mean != max here
    for g in range(Hkv):
        t = selkv.route(out["idx"][g], A_g[g], n, bucket)
        np.testing.assert_array_equal(out["target"][g], t)
        Vp, lnR, _ = selkv.merge_group(V[g], A_g[g], out["idx"][g], t)
        np.testing.assert_allclose(out["Vp"][g], Vp, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(out["lnR"][g], lnR, rtol=1e-12, atol=1e-14)


def test_gate_closed_forms(golden):
    a = np.array([1.0, 0.0, 2.0, 0.0])
    b = np.array([0.0, 3.0, 0.0, -1.0])
    assert selkv.gate(a, b) == golden["gate_orthogonal"]
    assert abs(selkv.gate(a, 2.5 * a) - golden["gate_parallel"]) < 1e-15
    assert selkv.gate(a, -a) == golden["gate_antiparallel"]
    assert selkv.gate(a, np.zeros(4)) == 0.0


def test_merge_ratio_closed_form(golden):
    V = np.array([[1.0, 0.0], [2.0, 0.0], [4.0, 0.0], [0.0, 1.0]])
    A = np.array([0.5, 0.25, 0.25, 0.1])
    kept = np.array([0, 3])
    target = np.array([-1, 0, 0, -1])
    Vp, lnR, gates = selkv.merge_group(V, A, kept, target)
    assert abs(lnR[0] - golden["ratio_two_parallel_routed"]) < 1e-15
    np.testing.assert_allclose(Vp[0], [(0.5 * 1 + 0.25 * 2 + 0.25 * 4) / 1.0, 0.0], atol=1e-15)
    assert lnR[1] == 0.0 and (Vp[1] == V[3]).all()
    assert gates[1] == 1.0 and np.isnan(gates[0])


def test_orthogonal_routed_tokens_are_dropped():
    V = np.array([[1.0, 0.0], [0.0, 5.0], [0.0, -2.0]])
    A = np.array([0.2, 0.5, 0.3])
    Vp, lnR, gates = selkv.merge_group(V, A, np.array([0]), np.array([-1, 0, 0]))
    assert (Vp[0] == V[0]).all() and lnR[0] == 0.0 and gates[1] == 0 and gates[2] == 0


def test_route_picks_highest_attention_lowest_index():
    A = np.array([0.1, 0.3, 0.3, 0.2, 0.9, 0.1, 0.0, 0.4])
    kept = np.array([1, 2, 3, 7])
    t = selkv.route(kept, A, 8, 4)
    # bucket 0 (0..3): kept 1, 2, 3 -> highest A is tie 1/2 -> 1
    assert t.tolist() == [1, -1, -1, -1, 7, 7, 7, -1]
    t = selkv.route(np.array([5]), A, 8, 4)     # bucket 0 has no kept token
    assert t.tolist() == [-1, -1, -1, -1, 5, -1, 5, 5]


def test_vatp_union_closed_form(golden):
    # token 0: group 0 value (3, 4, 0, 0), group 1 value (5, 12, 0, 0); token 1
    # is a zero vector (norm 0, so VATP 0 whatever the attention)
    V = np.zeros((2, 2, 4))
    V[0, 0, :2] = [3.0, 4.0]
    V[1, 0, :2] = [5.0, 12.0]
    A_hq = np.array([[0.1, 0.9], [0.2, 0.8], [0.3, 0.7], [0.4, 0.6]])
    vatp, U = selkv.vatp_union(A_hq, V)
    want = golden["vatp_norms_5_13_A_1234"]
    np.testing.assert_allclose(vatp[:, 0], want["vatp"], rtol=1e-15)
    np.testing.assert_allclose(U[:, 0], want["U"], rtol=1e-15)
    assert (vatp[:, 1] == 0).all() and (U[:, 1] == 0).all()


def test_vatp_union_brute_force():
    Hq, Hkv, n, d = 6, 3, 25, 5
    A_hq = rng.random((Hq, n))
    V = rng.normal(size=(Hkv, n, d)) * rng.random((Hkv, 1, 1)) * 4
    vatp, U = selkv.vatp_union(A_hq, V)
    G = Hq // Hkv
    for g in range(Hkv):
        for j in range(n):
            norm = math.sqrt(sum(float(x) ** 2 for x in V[g, j]))
            heads = [A_hq[h, j] * norm for h in range(g * G, (g + 1) * G)]
            for h, val in zip(range(g * G, (g + 1) * G), heads):
                assert abs(vatp[h, j] - val) <= 1e-14 * max(1.0, val)
            assert abs(U[g, j] - max(heads)) <= 1e-14 * max(1.0, max(heads))


def test_union_is_shared_threshold_superlevel_union():
    Hq, Hkv, n, d, w, m = 8, 2, 300, 8, 8, 80
    A_hq = rng.random((Hq, n))
    V = rng.normal(size=(Hkv, n, d))
    vatp, U = selkv.vatp_union(A_hq, V)
    idx = infokv.select_topk(U.astype(np.float32), m, w)
    G = Hq // Hkv
    for g in range(Hkv):
        body = [i for i in idx[g] if i < n - w]
        t = min(U[g, i] for i in body)
        union = set()
        for h in range(g * G, (g + 1) * G):
            union |= {j for j in range(n - w) if vatp[h, j] >= t}
        assert union == set(body)


def duplicate_key_instance(seed, Hq=4, Hkv=2, n=512, d=16, w=32, bucket=64):
    r = np.random.default_rng(seed)
    nb = n // bucket
    K = np.empty((Hkv, n, d))
    V = np.empty((Hkv, n, d))
    for g in range(Hkv):
        for b in range(nb):
            K[g, b * bucket:(b + 1) * bucket] = 0.05 * r.normal(size=d)
            u = r.normal(size=d)
            s = r.uniform(0.5, 1.0, size=bucket)
            s[r.integers(0, bucket - w if b == nb - 1 else bucket)] *= 5000.0
            V[g, b * bucket:(b + 1) * bucket] = s[:, None] * u[None, :]
    q_win = r.normal(size=(Hq, w, d))
    q = r.normal(size=(Hq, d))
    return q_win, K, V, q


@pytest.mark.parametrize("seed", range(3))
def test_duplicate_key_construction_recovers_full_attention(seed):
    q_win, K, V, q = duplicate_key_instance(seed)
    out = selkv.selkv_layer(q_win, K, V, m_keep=128, w=32, bucket=64)
    g = out["gates"][~np.isnan(out["gates"])]
    np.testing.assert_allclose(g, 1.0, atol=1e-12)
    Kc, _ = infokv.compact(K, V, out["idx"])
    o_full, _ = infokv.decode_attention(q, K, V)
    o_comp, _ = selkv.compensated_decode(q, Kc, out["Vp"], out["lnR"], 1.0)
    np.testing.assert_allclose(o_comp, o_full, rtol=1e-9, atol=1e-9)
    # without compensation the merged entries are under-weighted
    o_nobias, _ = selkv.compensated_decode(q, Kc, out["Vp"], out["lnR"], 0.0)
    assert np.abs(o_nobias - o_full).max() > 1e-3
    assert np.all(out["lnR"] >= 0)


def test_bf16_encoding_matches_torch_on_float32_values():
    import torch
    x = (rng.normal(size=20000) * 10.0 ** rng.integers(-30, 30, size=20000)).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, 1.0, 3.0e38, -3.3e38, 1e-40])])
    mine = precision.f64_to_bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)
    np.testing.assert_array_equal(precision.bf16_bits_to_f64(ref),
                                  torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16)
                                  .to(torch.float64).numpy())


def test_bf16_ties_round_to_even():
    # 1 + 2^-8 lies halfway between bf16 1.0 and 1 + 2^-7 -> even (1.0)
    assert precision.f64_to_bf16_bits(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    assert precision.f64_to_bf16_bits(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82
    assert precision.f64_to_bf16_bits(np.array([1.0 + 2.0 ** -8 + 2.0 ** -30]))[0] == 0x3F81
