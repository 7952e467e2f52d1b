"""Helpers shared by the GPU parity tests (not a test module)."""
import sys

import numpy as np
import pytest
import torch

from oracle import precision


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def announce(*parts):
    """Print what the next GPU step is about to run (flushed, so a fault still
    leaves the case name in the log)."""
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


def host_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a device tensor's values (bf16 via its bit pattern)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return precision.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.numpy().astype(np.float64)


def host_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy().view(np.uint32)


def max_rel(got, ref, floor=0.0):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.maximum(np.abs(ref), floor)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(got - ref) / den)) if got.size else 0.0


def assert_rel(got, ref, tol=1e-3, floor=0.0, what=""):
    r = max_rel(got, ref, floor)
    assert r <= tol, f"{what}: max relative error {r:.3e} > {tol:g}"


def kept_sets_match(idx_gpu, S_ref, k, w, band=1e-3):
    """Kept sets equal except tokens whose reference score is within `band`
    (relative) of the reference threshold.  Returns the number of band tokens."""
    Hkv, n = S_ref.shape
    nb = n - w
    flexible = 0
    for g in range(Hkv):
        got = set(np.asarray(idx_gpu[g]).tolist())
        assert set(range(nb, n)) <= got, "window not kept"
        if k <= w or k - w >= nb:
            continue
        body = S_ref[g, :nb]
        thr = np.sort(body)[::-1][k - w - 1]
        near = np.abs(body - thr) <= band * abs(thr)
        must = set(np.nonzero((body > thr) & ~near)[0].tolist())
        never = set(np.nonzero((body < thr) & ~near)[0].tolist())
        assert must <= got, f"group {g}: {len(must - got)} clear winners missing"
        assert not (never & got), f"group {g}: {len(never & got)} clear losers kept"
        flexible += int(near.sum())
    return flexible
