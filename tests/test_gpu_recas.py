"""GPU parity of RECAS's active-set decoding ([RECAS] section 2.C) against the
oracle.

  * Sparse scores element by element (matrix-core path: bf16, d 64/128, G <= 4;
    general path otherwise), with and without a utility row.
  * Decode over seeded random active lists (unsorted, repeated rows, one row, all
    rows) against the oracle's attention over the same rows.
  * The chain scores -> select -> decode: the active set is the exact top K_t
    of the GPU's own scores, equal to the oracle's outside the 1e-3 band, and
    where equal the step's output matches the oracle's.
"""
import math

import numpy as np
import pytest
import torch

from oracle import recas
from tests.gpu_util import announce, assert_rel, host_f64, kept_sets_match, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = need_gpu()
    from kv_cache_compression_softmax_amd import binding
    binding.lib()
    return d


def B():
    from kv_cache_compression_softmax_amd import binding
    return binding


def gen(shape, seed, dev, dtype):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(dtype)


CASES = [(32, 8, 3000, 128, torch.bfloat16, True), (8, 2, 700, 64, torch.bfloat16, False),
         (4, 4, 17, 128, torch.bfloat16, True), (6, 2, 1025, 128, torch.bfloat16, False),
         (16, 2, 500, 128, torch.bfloat16, True), (8, 2, 300, 64, torch.float32, True)]


@pytest.mark.parametrize("Hq,Hkv,n,d,dtype,util", CASES, ids=str)
def test_active_scores(dev, Hq, Hkv, n, d, dtype, util, L=2):
    announce("active scores", Hq, Hkv, n, d, dtype, util, L)
    q = [gen((Hq, d), 500 + l, dev, dtype) for l in range(L)]
    K = [gen((Hkv, n, d), 520 + l, dev, dtype) for l in range(L)]
    u = [gen((Hkv, n), 540 + l, dev, torch.float32) for l in range(L)] if util else None
    sc = torch.empty(L, Hkv, n, device=dev)
    B().kvc_active_scores(q, K, 1 / math.sqrt(d), sc, u, 0.3)
    torch.cuda.synchronize()
    for l in range(L):
        ref = recas.active_scores(host_f64(q[l]), host_f64(K[l]), host_f64(u[l]) if util else None, 0.3)
        # a score is a logit: relative 1e-3, absolute 1e-3 where it is below 1
        assert_rel(sc[l].cpu().numpy(), ref, 1e-3, floor=1.0, what="score")


DEC_CASES = [(32, 8, 2000, 128, torch.bfloat16, 600, True), (8, 2, 700, 64, torch.bfloat16, 1, False),
             (4, 1, 513, 128, torch.bfloat16, 513, True), (12, 4, 1000, 128, torch.bfloat16, 77, False),
             (16, 2, 400, 128, torch.bfloat16, 150, True), (8, 2, 300, 64, torch.float32, 90, True)]


@pytest.mark.parametrize("Hq,Hkv,n,d,dtype,k,bias", DEC_CASES, ids=str)
def test_decode_over_random_active_lists(dev, Hq, Hkv, n, d, dtype, k, bias, L=2):
    announce("decode active", Hq, Hkv, n, d, dtype, k, bias, L)
    q = [gen((Hq, d), 600 + l, dev, dtype) for l in range(L)]
    K = [gen((Hkv, n, d), 620 + l, dev, dtype) for l in range(L)]
    V = [gen((Hkv, n, d), 640 + l, dev, dtype) for l in range(L)]
    gl = torch.Generator(device=dev)
    gl.manual_seed(660 + n)
    lr = [torch.rand(Hkv, n, generator=gl, device=dev) for _ in range(L)] if bias else None
    r = np.random.default_rng(n + k)
    act = [torch.from_numpy(r.integers(0, n, size=(Hkv, k)).astype(np.int32)).to(dev) for _ in range(L)]
    o = torch.empty(L, Hq, d, device=dev)
    lse = torch.empty(L, Hq, device=dev)
    B().kvc_decode_attn_active(q, K, V, lr, 0.9, act, 1 / math.sqrt(d), o, lse)
    torch.cuda.synchronize()
    for l in range(L):
        ro, rl = recas.active_decode(host_f64(q[l]), host_f64(K[l]), host_f64(V[l]), act[l].cpu().numpy(),
                                     host_f64(lr[l]) if bias else None, 0.9 if bias else 0.0)
        assert np.max(np.abs(o[l].cpu().numpy() - ro)) <= 1e-3
        assert_rel(lse[l].cpu().numpy(), rl, 1e-4, floor=1.0, what="lse")


def test_layer_groups(dev):
    """34 layers: two launches of at most 32 layers' pointers each."""
    test_active_scores(dev, 4, 2, 200, 64, torch.bfloat16, True, L=34)
    test_decode_over_random_active_lists(dev, 4, 2, 200, 64, torch.bfloat16, 50, True, L=34)


@pytest.mark.parametrize("Hq,Hkv,n,d,frac", [(32, 8, 6400, 128, 0.293), (8, 2, 1000, 64, 0.5)], ids=str)
def test_active_step_end_to_end(dev, Hq, Hkv, n, d, frac):
    announce("active step", Hq, Hkv, n, d, frac)
    L, dtype = 2, torch.bfloat16
    q = [gen((Hq, d), 700 + l, dev, dtype) for l in range(L)]
    K = [gen((Hkv, n, d), 720 + l, dev, dtype) for l in range(L)]
    V = [gen((Hkv, n, d), 740 + l, dev, dtype) for l in range(L)]
    k = int(frac * n)
    sc = torch.empty(L, Hkv, n, device=dev)
    act = [torch.empty(Hkv, k, dtype=torch.int32, device=dev) for _ in range(L)]
    o = torch.empty(L, Hq, d, device=dev)
    B().kvc_active_scores(q, K, 1 / math.sqrt(d), sc)
    B().kvc_select_topk(sc, [k] * L, 0, act)
    B().kvc_decode_attn_active(q, K, V, None, 0.0, act, 1 / math.sqrt(d), o)
    torch.cuda.synchronize()
    compared = 0
    G = Hq // Hkv
    for l in range(L):
        ref_s = recas.active_scores(host_f64(q[l]), host_f64(K[l]))
        ref_a = recas.active_set(ref_s.astype(np.float32), k)
        gs, ga = sc[l].cpu().numpy(), act[l].cpu().numpy()
        for g in range(Hkv):                               # exact top-k of the GPU's own scores
            kept = np.zeros(n, dtype=bool)
            kept[ga[g]] = True
            assert np.all(np.diff(ga[g]) > 0) and kept.sum() == k
            if k < n:
                assert gs[g][kept].min() >= gs[g][~kept].max()
        kept_sets_match(ga, ref_s, k, 0)
        Kf, Vf = host_f64(K[l]), host_f64(V[l])
        for g in range(Hkv):
            if not np.array_equal(ga[g], ref_a[g]):
                continue
            ro, _ = recas.active_decode(host_f64(q[l][g * G:(g + 1) * G]), Kf[g:g + 1], Vf[g:g + 1], ref_a[g:g + 1])
            assert np.max(np.abs(o[l, g * G:(g + 1) * G].cpu().numpy() - ro)) <= 1e-3
            compared += 1
    assert compared >= (L * Hkv + 1) // 2
