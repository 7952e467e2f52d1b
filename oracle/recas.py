"""Plain float64 oracle of RECAS's active-set decoding over a retained cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Page cited as [RECAS]: gist.science technical summary of reasoning-aware,
error-bounded KV-cache compression and sparse attention (rs-10952127);
section 2.B (error-bounded compression: the dropped-attention-mass bound) and
section 2.C (dynamic sparse decoding attention: a query-aware sparse score over
the retained cache, the top K_t entries form the active set, and only they take
part in the step's attention).

Readings taken where the page is silent:
  * The sparse score of a cached entry is the query-key compatibility, scaled
    by 1/sqrt(d), plus a utility term.  The page fuses three utility signals
    without fixing their inputs, so the utility row is an input (zero by
    default).
  * Under GQA the active set is chosen per KV head, shared by the group's query
    heads, by the largest compatibility over the group's heads.
  * The top K_t scores form the active set, ties to the lower index; the
    decision is taken on float32 scores.
  * The attention of the step is the plain softmax attention over the active
    rows (with an optional log-ratio bias, as over any compacted cache).
"""
from __future__ import annotations

import math

import numpy as np

from .infokv import decode_attention, select_topk


def active_scores(q: np.ndarray, K: np.ndarray, utility: np.ndarray | None = None,
                  beta: float = 0.0, scale: float | None = None) -> np.ndarray:
    """Sparse score of every cached entry ([RECAS] 2.C): for KV head g and row
    j, the largest scale * <q_h, k_j> over the group's query heads h, plus
    beta * utility[g, j].  q [Hq, d], K [Hkv, len, d] -> [Hkv, len]."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    Hq, d = q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.empty(K.shape[:2])
    for g in range(Hkv):
        comp = (K[g] @ q[g * G:(g + 1) * G].T) * scale         # [len, G]
        out[g] = comp.max(axis=1)
        if utility is not None:
            out[g] += beta * np.asarray(utility, dtype=np.float64)[g]
    return out


def active_set(scores32: np.ndarray, k_active: int) -> np.ndarray:
    """The K_t entries with the largest float32 score per KV head ([RECAS]
    2.C), ties to the lower index, ascending: int32 [Hkv, k_active]."""
    return select_topk(np.asarray(scores32, dtype=np.float32), k_active, 0)


def active_decode(q, K, V, active: np.ndarray, logR=None, alpha_bias: float = 0.0,
                  scale: float | None = None):
    """Attention of one decode step over the active rows only ([RECAS] 2.C):
    decode attention over K[g, active[g]], V[g, active[g]] (and ln R there).
    Returns (o [Hq, d], lse [Hq])."""
    ii = np.asarray(active, dtype=np.int64)
    Ka = np.take_along_axis(np.asarray(K, dtype=np.float64), ii[:, :, None], axis=1)
    Va = np.take_along_axis(np.asarray(V, dtype=np.float64), ii[:, :, None], axis=1)
    La = None if logR is None else np.take_along_axis(np.asarray(logR, dtype=np.float64), ii, axis=1)
    return decode_attention(q, Ka, Va, La, alpha_bias, scale)
