"""The oracle over whole full-size workloads, for the GPU parity tests (not a
test module).

Inputs are host copies of the bytes the GPU consumed (bf16 as uint16 bit
patterns, decoded to float64 piece by piece, so host memory holds the bf16
copy plus one float64 piece per thread).  Every piece is a call of the oracle
function itself on a slice the definition makes independent (a chunk of logits
rows for H, a chunk of token rows for D, a layer for A, S and the selection);
``oracle.parallel`` runs the pieces on host threads and puts them back in
order.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import infokv, parallel, precision, selkv


def bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a device tensor: bf16 as uint16 bits, float32 as float32."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f64(a: np.ndarray) -> np.ndarray:
    return precision.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def entropy(logits: np.ndarray, k: int, rows: int = 256) -> np.ndarray:
    """H of every logits row ([InfoKV] Glossary), by chunks of rows."""
    parts = parallel.map_pieces(lambda c: infokv.topk_entropy(f64(logits[c[0]:c[1]]), k),
                                parallel.row_chunks(logits.shape[0], rows))
    return np.concatenate(parts)


def distance(h_layers, h_final: np.ndarray, tau: float, rows: int = 512) -> np.ndarray:
    """D [L, n] ([InfoKV] Method), by chunks of token rows over every layer."""
    def piece(c):
        b = f64(h_final[c[0]:c[1]])
        return np.stack([infokv.repr_distance(f64(h[c[0]:c[1]]), b, tau) for h in h_layers])
    return np.concatenate(parallel.map_pieces(piece, parallel.row_chunks(h_final.shape[0], rows)),
                          axis=1)


def infokv_layers(q_win, k, D: np.ndarray, H: np.ndarray, alpha: float):
    """Per layer: A (group mean), S, S rounded to float32 and Ebar."""
    def piece(l):
        A = infokv.window_attention(f64(q_win[l]), f64(k[l]))
        S, Ebar, _, _ = infokv.fuse_scores(A, D[l], H, alpha)
        return A, S, S.astype(np.float32), Ebar
    out = parallel.map_pieces(piece, range(len(k)))
    return ([o[0] for o in out], [o[1] for o in out], [o[2] for o in out],
            np.array([o[3] for o in out]))


def select_layers(S32, k_list, w: int):
    """The oracle's kept indices of every layer (int32 [Hkv, k_l])."""
    return parallel.map_pieces(lambda l: infokv.select_topk(S32[l], int(k_list[l]), w),
                               range(len(S32)))


def selkv_group_merge(V: np.ndarray, A_g: np.ndarray, idx: np.ndarray, bucket: int):
    """Route and gated merge of every KV head of one layer ([SelKV] section 2,
    steps 3-5) for given kept indices and group attention: (V' [Hkv, m, d],
    ln R [Hkv, m])."""
    Vf = f64(V)
    Hkv, n, d = Vf.shape

    def piece(g):
        tgt = selkv.route(idx[g], A_g[g], n, bucket)
        Vp, lnR, _ = selkv.merge_group(Vf[g], A_g[g], idx[g], tgt)
        return Vp, lnR
    out = parallel.map_pieces(piece, range(Hkv))
    return np.stack([o[0] for o in out]), np.stack([o[1] for o in out])
