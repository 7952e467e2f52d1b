"""Workload definitions: shapes, hyperparameters and input distributions.

Shapes follow the Llama-family models the InfoKV and SelKV pages evaluate on
(Llama-3.2-3B: 28 layers, 24 query / 8 KV heads, head dim 128, hidden 3072;
Llama-3.1-8B: 32 layers, 32 / 8 heads, head dim 128, hidden 4096; vocabulary
128256).  The defaults alpha_fuse = 0.9, tau = 1 and entropy top-k = 256 are
the InfoKV page's (Contributions; Method).  Every input is synthetic.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    method: str                 # "infokv" or "selkv"
    layers: int
    heads_q: int
    heads_kv: int
    head_dim: int
    n: int                      # prefill tokens
    window: int                 # observation window w
    dtype: str                  # "f32" or "bf16"
    seed: int
    hidden: int = 0
    vocab: int = 0
    topk_entropy: int = 256
    alpha_fuse: float = 0.9
    tau: float = 1.0
    keep_fraction: float = 0.0          # uniform budget per layer / KV head
    adaptive_fraction: float = 0.0      # adaptive: B = floor(f*n) * layers
    logits_scale: float = 4.0
    logits_spikes: bool = True          # 1..8 distinct columns per row get +12
    hidden_c: tuple = ()                # per-layer correlation with h^(L)
    logits_chunk_rows: int = 0          # 0: one call over all rows
    bucket: int = 64                    # SelKV positional bucket
    alpha_bias: float = 1.0             # SelKV logit-bias strength

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv

    def budgets(self):
        """Uniform k per layer (floor(f*n)), or None for the adaptive budget."""
        if self.adaptive_fraction:
            return None
        return [int(math.floor(self.keep_fraction * self.n))] * self.layers

    def adaptive_total(self) -> int:
        return int(math.floor(self.adaptive_fraction * self.n)) * self.layers

    def input_bytes(self) -> int:
        e = 4 if self.dtype == "f32" else 2
        b = 2 * self.layers * self.heads_kv * self.n * self.head_dim * e
        b += self.layers * self.heads_q * self.window * self.head_dim * e
        if self.method == "infokv":
            b += (self.layers + 1) * self.n * self.hidden * e
            b += self.n * self.vocab * e
        return b


def linear_c(layers: int, lo: float = 0.2, hi: float = 1.0) -> tuple:
    """c_l rising linearly from lo at layer 0 to hi at layer L-1 (hi exactly)."""
    if layers == 1:
        return (hi,)
    return tuple(hi if l == layers - 1 else lo + (hi - lo) * l / (layers - 1)
                 for l in range(layers))


TINY = Workload(
    name="tiny-infokv-n512-f32", method="infokv", layers=1, heads_q=4, heads_kv=2,
    head_dim=64, n=512, window=16, dtype="f32", seed=0, hidden=256, vocab=2048,
    topk_entropy=64, keep_fraction=0.25, logits_scale=3.0, logits_spikes=False,
    hidden_c=(0.6,))

LLAMA3B_16K = Workload(
    name="llama3.2-3b-n16384-keep40-bf16", method="infokv", layers=28, heads_q=24,
    heads_kv=8, head_dim=128, n=16384, window=32, dtype="bf16", seed=1,
    hidden=3072, vocab=128256, keep_fraction=0.4, hidden_c=linear_c(28))

LLAMA8B_32K = Workload(
    name="llama3.1-8b-n32768-keep20-bf16", method="infokv", layers=32, heads_q=32,
    heads_kv=8, head_dim=128, n=32768, window=32, dtype="bf16", seed=2,
    hidden=4096, vocab=128256, keep_fraction=0.2, hidden_c=linear_c(32))

LLAMA8B_64K_ADAPTIVE = Workload(
    name="llama3.1-8b-n65536-adaptive12.5-bf16", method="infokv", layers=32,
    heads_q=32, heads_kv=8, head_dim=128, n=65536, window=32, dtype="bf16", seed=3,
    hidden=4096, vocab=128256, adaptive_fraction=0.125, hidden_c=linear_c(32),
    logits_chunk_rows=8192)

LLAMA8B_SELKV_100K = Workload(
    name="llama3.1-8b-selkv-n102400-keep25-bf16", method="selkv", layers=32,
    heads_q=32, heads_kv=8, head_dim=128, n=102400, window=32, dtype="bf16", seed=4,
    keep_fraction=0.25, bucket=64, alpha_bias=1.0)

ALL = (TINY, LLAMA3B_16K, LLAMA8B_32K, LLAMA8B_64K_ADAPTIVE, LLAMA8B_SELKV_100K)
BY_NAME = {w.name: w for w in ALL}


def reduced(w: Workload, **changes) -> Workload:
    """A smaller copy of a workload (same generators) for parity tests.
    Adjusts hidden_c when the layer count changes."""
    if "layers" in changes and "hidden_c" not in changes and w.hidden_c:
        changes["hidden_c"] = linear_c(changes["layers"]) if len(w.hidden_c) > 1 \
            else w.hidden_c * changes["layers"]
    changes.setdefault("name", w.name + "-reduced")
    return dataclasses.replace(w, **changes)
