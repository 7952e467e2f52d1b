"""GPU parity of SelKV's RoPE re-positioning ([SelKV] section 2, step 6)
against the oracle: random keys at sorted original positions (as kept indices
are), re-embedded at contiguous positions, bf16 and float32, several head
dimensions and bases.  bf16 results may differ from the oracle's exact value by
its rounding (half a bf16 ulp) plus the float32 rotation."""
import numpy as np
import pytest
import torch

from oracle import selkv
from tests.gpu_util import announce, host_f64, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = need_gpu()
    from kv_cache_compression_softmax_amd import binding
    binding.lib()
    return d


@pytest.mark.parametrize("Hkv,m,d,dtype,base,new0", [
    (8, 3000, 128, torch.bfloat16, 500000.0, 0), (2, 700, 64, torch.bfloat16, 10000.0, 17),
    (4, 129, 2, torch.float32, 10000.0, 3), (3, 1000, 128, torch.float32, 1e6, 0),
    (1, 1, 128, torch.bfloat16, 10000.0, 0), (2, 333, 4, torch.bfloat16, 10000.0, 5),
    (2, 200, 6, torch.float32, 10000.0, 0), (1, 50, 512, torch.bfloat16, 10000.0, 1)], ids=str)
def test_rope_reposition(dev, Hkv, m, d, dtype, base, new0, L=2):
    from kv_cache_compression_softmax_amd import binding as B
    announce("rope", Hkv, m, d, dtype, base, new0, L)
    g = torch.Generator(device=dev)
    g.manual_seed(m + d)
    K = [torch.randn(Hkv, m, d, generator=g, device=dev).to(dtype) for _ in range(L)]
    r = np.random.default_rng(m)
    pos = [torch.from_numpy(np.stack([np.sort(r.choice(100000, size=m, replace=False))
                                      for _ in range(Hkv)]).astype(np.int32)).to(dev) for _ in range(L)]
    K0 = [host_f64(k) for k in K]
    B.kvc_rope_reposition(K, pos, new0, base)
    torch.cuda.synchronize()
    for l in range(L):
        ref = selkv.rope_reposition(K0[l], pos[l].cpu().numpy(), new0, base)
        got = host_f64(K[l])
        h = d // 2
        scale = np.concatenate([np.abs(K0[l][..., :h]) + np.abs(K0[l][..., h:])] * 2, axis=-1)
        tol = (2.0 ** -8) * np.abs(ref) + 1e-5 * scale + 1e-6 if dtype == torch.bfloat16 else \
            1e-5 * scale + 1e-6
        assert np.all(np.abs(got - ref) <= tol), float(np.max(np.abs(got - ref) - tol))


def test_rope_layer_groups(dev):
    """34 layers: two launches of at most 32 layers' pointers each."""
    test_rope_reposition(dev, 2, 100, 128, torch.bfloat16, 500000.0, 3, L=34)
