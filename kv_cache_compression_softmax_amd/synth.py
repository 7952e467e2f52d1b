"""Seeded synthetic inputs shared by the GPU path's tests, the bench and the
oracle's parity checks.

This module holds only random-number plumbing (torch generators); none of the
scoring or compaction arithmetic.  The GPU and the oracle see the same bytes:
inputs are generated once on the target device and the oracle receives a
device-to-host copy.

Recipe (per tensor an independent ``torch.Generator`` seeded from
(workload seed, tensor tag, layer); draws in float32, then rounded to the
workload dtype with round-to-nearest-even):
  * window queries q_win[l] [Hq, w, d], keys k[l] and values v[l] [Hkv, n, d]:
    N(0, 1);
  * final hidden state h^(L) [n, hidden]: N(0, 1); layer hidden states
    h^(l) = c_l * h^(L) + sqrt(1 - c_l^2) * N(0, 1), computed in float32 from
    the unrounded h^(L) draw (so c_l = 1 reproduces h^(L) bit for bit);
  * final-layer logits [n, vocab]: scale * N(0, 1); with spikes, each row gets
    m ~ U{1..8} distinct uniformly drawn columns raised by +12 before rounding;
  * decode queries q_dec [L, Hq, d]: N(0, 1) (SelKV check).
"""
from __future__ import annotations

import math

import torch

from .configs import Workload

_TAGS = {"q_win": 1, "k": 2, "v": 3, "h_final": 4, "h_noise": 5, "logits": 6,
         "spike_count": 7, "spike_cols": 8, "q_dec": 9, "scores": 10}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def generator(device, seed: int, tag: str, layer: int = 0, chunk: int = 0):
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + _TAGS[tag] * 10_007 + layer * 101 + chunk)
                  % (2 ** 63))
    return g


def normal(shape, device, seed, tag, layer=0, dtype=torch.bfloat16, scale=1.0):
    g = generator(device, seed, tag, layer)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype)


def hidden_states(w: Workload, device):
    """(h_layers list of L tensors [n, hidden], h_final [n, hidden])."""
    dt = TORCH_DTYPE[w.dtype]
    g = generator(device, w.seed, "h_final")
    hL = torch.randn((w.n, w.hidden), generator=g, device=device, dtype=torch.float32)
    layers = []
    for l in range(w.layers):
        c = float(w.hidden_c[l])
        gn = generator(device, w.seed, "h_noise", l)
        noise = torch.randn((w.n, w.hidden), generator=gn, device=device,
                            dtype=torch.float32)
        layers.append((c * hL + math.sqrt(max(0.0, 1.0 - c * c)) * noise).to(dt))
        del noise
    return layers, hL.to(dt)


def logits(w: Workload, device, rows: int | None = None, chunk_rows: int = 4096):
    """Final-layer logits [rows, vocab] (rows defaults to n), generated in
    row chunks, each chunk from its own generator stream."""
    rows = w.n if rows is None else rows
    dt = TORCH_DTYPE[w.dtype]
    out = torch.empty((rows, w.vocab), device=device, dtype=dt)
    for ci, r0 in enumerate(range(0, rows, chunk_rows)):
        r1 = min(rows, r0 + chunk_rows)
        g = generator(device, w.seed, "logits", 0, ci)
        x = torch.randn((r1 - r0, w.vocab), generator=g, device=device,
                        dtype=torch.float32)
        x.mul_(w.logits_scale)
        if w.logits_spikes:
            gc = generator(device, w.seed, "spike_count", 0, ci)
            count = torch.randint(1, 9, (r1 - r0,), generator=gc, device=device)
            gs = generator(device, w.seed, "spike_cols", 0, ci)
            cols = torch.randint(0, w.vocab, (r1 - r0, 8), generator=gs, device=device)
            for _ in range(64):                       # redraw rows with repeats
                s, _ = cols.sort(dim=1)
                dup = (s[:, 1:] == s[:, :-1]).any(dim=1)
                nd = int(dup.sum())
                if nd == 0:
                    break
                cols[dup] = torch.randint(0, w.vocab, (nd, 8), generator=gs,
                                          device=device)
            use = (torch.arange(8, device=device)[None, :] < count[:, None])
            x.scatter_add_(1, cols, use.to(torch.float32) * 12.0)
        out[r0:r1] = x.to(dt)
        del x
    return out


def make_inputs(w: Workload, device, with_logits: bool = True,
                with_values: bool = True) -> dict:
    """All inputs of one workload, resident on ``device``."""
    dt = TORCH_DTYPE[w.dtype]
    inp = {
        "q_win": [normal((w.heads_q, w.window, w.head_dim), device, w.seed, "q_win", l, dt)
                  for l in range(w.layers)],
        "k": [normal((w.heads_kv, w.n, w.head_dim), device, w.seed, "k", l, dt)
              for l in range(w.layers)],
    }
    if with_values:
        inp["v"] = [normal((w.heads_kv, w.n, w.head_dim), device, w.seed, "v", l, dt)
                    for l in range(w.layers)]
    if w.method == "infokv":
        inp["h"], inp["h_final"] = hidden_states(w, device)
        if with_logits:
            inp["logits"] = logits(w, device)
    else:
        inp["q_dec"] = normal((w.layers, w.heads_q, w.head_dim), device, w.seed,
                              "q_dec", 0, dt)
    return inp


def random_scores(shape, device, seed: int, tie_levels: int = 0):
    """Synthetic float32 scores for selection tests.  With ``tie_levels`` > 0 the
    values are drawn from that many distinct levels, so ties are common."""
    g = generator(device, seed, "scores")
    if tie_levels:
        lv = torch.randint(0, tie_levels, shape, generator=g, device=device)
        return (lv.to(torch.float32) + 1.0) / tie_levels
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32)
