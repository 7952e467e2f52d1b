"""GPU parity of the dropped-attention-mass monitor ([RECAS] section 2.B).

kvc_dropped_mass takes the log normalisers of a decode query over the kept rows
and over the full cache and returns delta (the evicted share of the full
softmax), V_max (the largest value norm of the full cache) and 2 * V_max *
delta.  The oracle's ``dropped_mass_bound`` computes delta as the sum of the
evicted tokens' probabilities and V_max as the largest norm, so the two meet
only on the inputs.
"""
import math

import numpy as np
import pytest
import torch

from kv_cache_compression_softmax_amd import configs, synth
from oracle import infokv
from tests.gpu_util import announce, assert_rel, host_f64, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = need_gpu()
    from kv_cache_compression_softmax_amd import binding
    binding.lib()
    return d


@pytest.mark.parametrize("w", [configs.TINY, configs.reduced(configs.LLAMA8B_32K, layers=3, n=3000),
                               configs.reduced(configs.LLAMA3B_16K, layers=2, n=1111)],
                         ids=lambda w: w.name)
def test_probe_matches_oracle(dev, w):
    from kv_cache_compression_softmax_amd import pipeline
    announce("dropped mass probe", w.name)
    inp = synth.make_inputs(w, dev)
    plan = pipeline.InfoKVPlan(w, dev).run(inp)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q = [synth.normal((w.heads_q, w.head_dim), dev, 55, "q_dec", l, dtype=dt) for l in range(w.layers)]
    p = plan.probe(inp, q)
    torch.cuda.synchronize()
    G = w.group
    for l in range(w.layers):
        o, o2, delta, vmax = infokv.dropped_mass_bound(host_f64(q[l]), host_f64(inp["k"][l]),
                                                       host_f64(inp["v"][l]), plan.idx[l].cpu().numpy())
        # delta from two float32 normalisers: absolute error ~1e-6
        got = p["delta"][l].cpu().numpy()
        assert np.max(np.abs(got - delta)) <= 1e-4 + 1e-3 * np.abs(delta).max(), (got, delta)
        assert_rel(p["vmax"][l].cpu().numpy(), vmax[::G], 1e-3, what="V_max")
        assert_rel(p["bound"][l].cpu().numpy(), 2 * vmax * delta, 1e-3, floor=1e-3, what="bound")
        # the page's bound holds for the GPU's own outputs
        err = torch.linalg.vector_norm(p["o_kept"][l] - p["o_full"][l], dim=1)
        assert torch.all(err <= p["bound"][l] + 1e-4)
        np.testing.assert_allclose(p["o_full"][l].cpu().numpy(), o, atol=1e-3)
        np.testing.assert_allclose(p["o_kept"][l].cpu().numpy(), o2, atol=1e-3)


@pytest.mark.parametrize("dtype,d,Hq,Hkv,n", [("f32", 100, 4, 2, 300), ("f32", 512, 2, 1, 77),
                                              ("bf16", 64, 8, 2, 5000), ("f32", 128, 6, 3, 1),
                                              ("bf16", 24, 4, 4, 999), ("f32", 4, 2, 1, 4097),
                                              ("f32", 8, 4, 2, 700), ("bf16", 32, 4, 1, 2049),
                                              ("bf16", 512, 2, 2, 1000)])
def test_dropped_mass_row_shapes(dev, dtype, d, Hq, Hkv, n):
    """Every row-size path of the V_max pass (16-byte lanes per row from 1 to
    64, and the general one), with the oracle's own normalisers as inputs."""
    from kv_cache_compression_softmax_amd import binding as B
    announce("dropped mass shapes", dtype, d, Hq, Hkv, n)
    L = 2
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    r = np.random.default_rng(d * 7 + n)
    V = [synth.normal((Hkv, n, d), dev, 9, "v", l, dtype=tdt, scale=1.5) for l in range(L)]
    for l in range(L):          # one long row per head, at a varying place
        for g in range(Hkv):
            V[l][g, int(r.integers(0, n))] *= 3
    lk, lf, dref, vref = [], [], [], []
    for l in range(L):
        Vf = host_f64(V[l])
        K = r.normal(size=(Hkv, n, d))
        q = r.normal(size=(Hq, d))
        keep = np.sort(np.stack([r.choice(n, max(1, n // 3), replace=False) for _ in range(Hkv)]), axis=1)
        _, _, delta, vmax = infokv.dropped_mass_bound(q, K, Vf, keep)
        Kc = np.take_along_axis(K, keep[:, :, None], axis=1)
        Vc = np.take_along_axis(Vf, keep[:, :, None], axis=1)
        _, lse_kept = infokv.decode_attention(q, Kc, Vc)
        _, lse_full = infokv.decode_attention(q, K, Vf)
        lk.append(lse_kept); lf.append(lse_full); dref.append(delta); vref.append(vmax[::Hq // Hkv])
    t = lambda a: torch.tensor(np.array(a), dtype=torch.float32, device=dev)
    delta, vmax, bound = (torch.empty(L, Hq, device=dev), torch.empty(L, Hkv, device=dev),
                          torch.empty(L, Hq, device=dev))
    B.kvc_dropped_mass(t(lk), t(lf), V, delta, vmax, bound)
    torch.cuda.synchronize()
    assert np.max(np.abs(delta.cpu().numpy() - np.array(dref))) <= 1e-5
    assert_rel(vmax.cpu().numpy(), np.array(vref), 1e-5, what="V_max")
    assert_rel(bound.cpu().numpy(), 2 * np.repeat(np.array(vref), Hq // Hkv, axis=1) * np.array(dref),
               1e-4, floor=1e-6, what="bound")
