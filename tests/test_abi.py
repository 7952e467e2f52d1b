"""C-ABI checks that need no GPU: the library loads, exports every function that
include/kvc.h declares, rejects bad arguments before launching anything, and
its host-only budget calls agree with the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "kvc.h")
LIB = os.path.join(ROOT, "kv_cache_compression_softmax_amd", "libkvc.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libkvc.so not built")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_path():
    names = declared()
    for n in ["kvc_topk_entropy", "kvc_repr_distance", "kvc_score_window_attn", "kvc_fuse_scores",
              "kvc_adaptive_budget", "kvc_uniform_budget", "kvc_select_topk", "kvc_compact",
              "kvc_vatp_union", "kvc_merge_gated", "kvc_decode_attn"]:
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_entry_point():
    from kv_cache_compression_softmax_amd import binding
    for n in declared():
        if n in ("kvc_status_string", "kvc_last_error"):
            continue
        assert hasattr(binding, n), n


@pytest.fixture(scope="module")
def lib():
    from kv_cache_compression_softmax_amd import binding
    return binding.lib()


def err(lib):
    return lib.kvc_last_error().decode()


def test_status_strings(lib):
    assert lib.kvc_version() >= 100
    assert lib.kvc_status_string(0) == b"ok"
    assert lib.kvc_status_string(-3).startswith(b"workspace")


def test_validation_before_launch(lib):
    fake = ctypes.c_void_p(0x1000)     # never dereferenced: every call below fails validation
    # bad dtype
    assert lib.kvc_topk_entropy(fake, 7, 4, 100, 100, 8, fake, None) == -2
    # topk > vocab
    assert lib.kvc_topk_entropy(fake, 1, 4, 100, 100, 101, fake, None) == -1
    assert "topk" in err(lib)
    # topk above the maximum
    assert lib.kvc_topk_entropy(fake, 1, 4, 5000, 5000, 1025, fake, None) == -1
    # row_stride < vocab
    assert lib.kvc_topk_entropy(fake, 1, 4, 100, 99, 8, fake, None) == -1
    # null logits
    assert lib.kvc_topk_entropy(None, 1, 4, 100, 100, 8, fake, None) == -1
    # zero rows is a no-op success
    assert lib.kvc_topk_entropy(None, 1, 0, 100, 100, 8, None, None) == 0
    # window attention: Hq not a multiple of Hkv, w > n, missing workspace, bad d for bf16
    arr = (ctypes.c_void_p * 1)(0x1000)
    pa = ctypes.cast(arr, ctypes.c_void_p)
    assert lib.kvc_score_window_attn(pa, pa, 1, 1, 6, 4, 64, 8, 128, ctypes.c_float(0.1), 0, fake, fake, 1 << 30, None) == -1
    assert lib.kvc_score_window_attn(pa, pa, 1, 1, 4, 2, 64, 65, 128, ctypes.c_float(0.1), 0, fake, fake, 1 << 30, None) == -1
    assert lib.kvc_score_window_attn(pa, pa, 1, 1, 4, 2, 64, 8, 128, ctypes.c_float(0.1), 0, fake, None, 0, None) == -3
    assert lib.kvc_score_window_attn(pa, pa, 1, 1, 4, 2, 64, 8, 96, ctypes.c_float(0.1), 0, fake, fake, 1 << 30, None) == -1
    # window attention: the scale must be finite and positive
    for bad in (0.0, -0.1, float("inf"), float("nan")):
        assert lib.kvc_score_window_attn(pa, pa, 1, 1, 4, 2, 64, 8, 128, ctypes.c_float(bad), 0, fake, fake, 1 << 30, None) == -1
        assert "scale" in err(lib)
    # window attention, per_query_head: only 0, 1, 2; form 2 in bf16 needs one tile
    # per head (w <= 32) and at most 4 heads per group
    assert lib.kvc_score_window_attn(pa, pa, 1, 1, 4, 2, 64, 8, 128, ctypes.c_float(0.1), 3, fake, fake, 1 << 30, None) == -1
    assert lib.kvc_score_window_attn(pa, pa, 1, 1, 4, 2, 64, 48, 128, ctypes.c_float(0.1), 2, fake, fake, 1 << 30, None) == -1
    assert "per_query_head 2" in err(lib)
    assert lib.kvc_score_window_attn(pa, pa, 1, 1, 16, 2, 64, 8, 128, ctypes.c_float(0.1), 2, fake, fake, 1 << 30, None) == -1
    # VATP from the group max: bad d * element size, null output
    assert lib.kvc_vatp_union_gmax(fake, pa, 1, 1, 2, 64, 100, fake, None) == -1
    assert lib.kvc_vatp_union_gmax(fake, pa, 1, 1, 2, 64, 128, None, None) == -1
    # select: k_keep outside [1, n]
    kk = (ctypes.c_int64 * 1)(65)
    assert lib.kvc_select_topk(fake, 1, 2, 64, kk, 8, pa, None) == -1
    kk = (ctypes.c_int64 * 1)(0)
    assert lib.kvc_select_topk(fake, 1, 2, 64, kk, 8, pa, None) == -1
    # compact: V without V_out
    kk = (ctypes.c_int64 * 1)(8)
    assert lib.kvc_compact(pa, pa, 1, 1, 2, 64, 128, pa, kk, pa, None, None) == -1
    # fuse: alpha outside [0, 1]
    assert lib.kvc_fuse_scores(fake, fake, fake, 1, 2, 64, ctypes.c_float(1.5), fake, None, fake, 1 << 20, None) == -1
    # merge: bucket 0
    assert lib.kvc_merge_gated(pa, pa, 1, fake, 1, 2, 64, 128, pa, kk, 0, pa, pa, pa, None) == -1
    # decode: too many query heads per KV head
    assert lib.kvc_decode_attn(pa, pa, pa, 1, None, ctypes.c_float(0), 1, 16, 1, 64, 128, ctypes.c_float(0.1), fake, None, fake, 1 << 20, None) == -1


def test_validation_before_launch_decode_side(lib):
    fake = ctypes.c_void_p(0x1000)     # never dereferenced: every call below fails validation
    arr = (ctypes.c_void_p * 1)(0x1000)
    pa = ctypes.cast(arr, ctypes.c_void_p)
    kk = (ctypes.c_int64 * 1)(8)
    # compact into a head stride: out_rows below k_keep, or below 1
    assert lib.kvc_compact_into(pa, None, 1, 1, 2, 64, 128, pa, kk, 7, pa, None, None) == -1
    assert "out_rows" in err(lib)
    assert lib.kvc_compact_into(pa, None, 1, 1, 2, 64, 128, pa, kk, 0, pa, None, None) == -1
    # slot fusion: alpha outside [0, 1]; workspace missing
    assert lib.kvc_fuse_scores_slots(fake, fake, 1, 2, 64, 1.5, fake, None, fake, 1 << 20, None) == -1
    assert lib.kvc_fuse_scores_slots(fake, fake, 1, 2, 64, 0.9, fake, None, None, 0, None) == -3
    # entropy-score append past the slot capacity
    assert lib.kvc_append_entropy_scores(fake, fake, 1, 2, 100, fake, 150, 51, None) == -1
    # active scores: Hq not a multiple of Hkv
    assert lib.kvc_active_scores(pa, pa, 1, None, 0.0, 1, 6, 4, 64, 128, 0.1, fake, None) == -1
    # active scores: the scale must be finite and positive
    assert lib.kvc_active_scores(pa, pa, 1, None, 0.0, 1, 8, 2, 64, 128, -0.1, fake, None) == -1
    assert "scale" in err(lib)
    # decode: a non-finite scale or bias
    assert lib.kvc_decode_attn(pa, pa, pa, 1, None, ctypes.c_float(float("nan")), 1, 8, 2, 64, 128,
                               ctypes.c_float(0.1), fake, None, fake, 1 << 20, None) == -1
    assert lib.kvc_decode_attn(pa, pa, pa, 1, None, ctypes.c_float(0), 1, 8, 2, 64, 128,
                               ctypes.c_float(float("inf")), fake, None, fake, 1 << 20, None) == -1
    # active decode: no list, or more positions than rows
    assert lib.kvc_decode_attn_active(pa, pa, pa, 1, None, 0.0, None, 8, 1, 8, 2, 64, 128, 0.1,
                                      fake, None, fake, 1 << 20, None) == -1
    assert lib.kvc_decode_attn_active(pa, pa, pa, 1, None, 0.0, pa, 65, 1, 8, 2, 64, 128, 0.1,
                                      fake, None, fake, 1 << 20, None) == -1
    # RoPE re-positioning: odd d, base <= 1
    assert lib.kvc_rope_reposition(pa, 1, pa, 0, 10000.0, 1, 2, 64, 127, None) == -1
    assert lib.kvc_rope_reposition(pa, 1, pa, 0, 1.0, 1, 2, 64, 128, None) == -1


def test_uniform_budget_matches_oracle():
    from kv_cache_compression_softmax_amd import binding
    from oracle import infokv
    for f, n, w in [(0.25, 512, 16), (0.4, 16384, 32), (0.2, 32768, 32), (0.25, 102400, 32)]:
        assert binding.kvc_uniform_budget(f, n, w) == infokv.uniform_budget(f, n)
    assert binding.kvc_uniform_budget(0.01, 100, 8) == 8          # clamped to the window


@pytest.mark.parametrize("seed", range(20))
def test_adaptive_budget_matches_oracle(seed):
    from kv_cache_compression_softmax_amd import binding
    from oracle import infokv
    r = np.random.default_rng(seed)
    L = int(r.integers(1, 64))
    e = (r.random(L) * 10 + 0.1).astype(np.float32)
    n = 65536
    B = int(r.integers(L * 32, L * 20000))
    got = binding.kvc_adaptive_budget(e, B, 32, n)
    ref = infokv.adaptive_budget(e, B, 32, n)
    assert got == ref.tolist()


def test_adaptive_budget_rejects_nonpositive():
    from kv_cache_compression_softmax_amd import binding
    with pytest.raises(binding.KvcError):
        binding.kvc_adaptive_budget([1.0, 0.0], 100, 0, 1000)


def test_noalloc_window_attention_rejects_oversize_before_launch(lib):
    """The no-alloc window attention checks its workspace need against the fixed
    scratch before it touches the device."""
    arr = (ctypes.c_void_p * 1)(0x1000)
    pa = ctypes.cast(arr, ctypes.c_void_p)
    cap = lib.kvc_score_window_attn_noalloc_max_workspace()
    assert cap == 32 << 20
    # 32 layers of 32/8 heads at 2^23 tokens need far more than the scratch
    need = lib.kvc_score_window_attn_workspace_size(32, 32, 8, 1 << 23, 32, 128, 1)
    assert need > cap
    assert lib.kvc_score_window_attn_noalloc(pa, pa, 1, 32, 32, 8, 1 << 23, 32, 128, ctypes.c_float(0.1), 0,
                                             ctypes.c_void_p(0x1000), None) == -3
    assert "scratch" in err(lib)
    # the Llama-shaped workloads fit
    for L, Hq, n in [(28, 24, 16384), (32, 32, 32768), (32, 32, 65536), (32, 32, 102400)]:
        assert lib.kvc_score_window_attn_workspace_size(L, Hq, 8, n, 32, 128, 1) <= cap
