"""The no-alloc window attention (kvc_score_window_attn_noalloc) against the
entry point it mirrors (kvc_score_window_attn with a caller workspace), through
the C ABI: two calls in a row, the second smaller, each equal bit for bit to
the workspace call on the same inputs (the same kernels run; only where the
partial results live differs).  The outputs are first filled with NaN, so an
unwritten element fails."""
import ctypes
import math

import numpy as np
import pytest
import torch

from kv_cache_compression_softmax_amd import synth
from tests.gpu_util import announce, need_gpu

pytestmark = pytest.mark.gpu


def _call_noalloc(lib, q, k, scale, per_head, A):
    L = len(k)
    Hq, w, d = q[0].shape
    Hkv, n, _ = k[0].shape
    qa = (ctypes.c_void_p * L)(*[t.data_ptr() for t in q])
    ka = (ctypes.c_void_p * L)(*[t.data_ptr() for t in k])
    dt = 1 if k[0].dtype == torch.bfloat16 else 0
    st = lib.kvc_score_window_attn_noalloc(
        ctypes.cast(qa, ctypes.c_void_p), ctypes.cast(ka, ctypes.c_void_p), dt, L, Hq, Hkv, n, w, d,
        ctypes.c_float(scale), int(per_head), ctypes.c_void_p(A.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.kvc_last_error()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_workspace_call_twice(dtype):
    from kv_cache_compression_softmax_amd import binding as B
    dev = need_gpu()
    lib = B.lib()
    shapes = [(6, 32, 8, 20000, 32, 128, True), (3, 24, 8, 5000, 32, 128, False)] if dtype == torch.bfloat16 \
        else [(2, 8, 2, 3000, 16, 64, True), (1, 4, 2, 700, 16, 64, False)]
    for i, (L, Hq, Hkv, n, w, d, per_head) in enumerate(shapes):
        announce("window attention no-alloc", i, L, Hq, Hkv, n, w, d, per_head, dtype)
        q = [synth.normal((Hq, w, d), dev, 31 + i, "q_win", l, dtype) for l in range(L)]
        k = [synth.normal((Hkv, n, d), dev, 31 + i, "k", l, dtype) for l in range(L)]
        rows = Hq if per_head else Hkv
        A_ref = torch.full((L, rows, n), float("nan"), device=dev)
        A_new = torch.full((L, rows, n), float("nan"), device=dev)
        scale = 1.0 / math.sqrt(d)
        B.kvc_score_window_attn(q, k, scale, per_head, A_ref)
        _call_noalloc(lib, q, k, scale, per_head, A_new)
        torch.cuda.synchronize()
        assert torch.isfinite(A_ref).all()
        assert torch.equal(A_new, A_ref), float((A_new - A_ref).abs().max())
        np.testing.assert_allclose(A_new.sum(dim=2).cpu().numpy(), 1.0, atol=1e-3)
