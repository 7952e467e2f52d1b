"""Plain float64 oracle of SelKV's selective merge with attention compensation.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Page cited as [SelKV]: "SelKV: Selective KV Cache Merging with Per-Token
Merge-or-Drop and Attention Compensation", gist.science paper 2607.16213;
section 2 (방법론 / Method): "Soft cosine gate", "Attention compensation" and
the six-step "Pipeline overview".

Readings taken where the page is silent or ambiguous:
  * The importance score is VATP: window-averaged attention of a query head
    times the l2 norm of the token's value vector.
  * GQA union: U[g, j] = max over the group's query heads of VATP[h, j]; keep
    the top (m - w) of U over [0, n - w), ties to the lower index, plus the
    last w tokens.  This is the union of the heads' superlevel sets at the one
    threshold that keeps exactly m tokens.
  * "Prefill attention" of a token is A_g, the window- and group-averaged
    attention (the InfoKV A); the window tokens are valid merge targets.
  * Each evicted token goes to the kept token of its positional bucket
    (floor(index / bucket)) with the largest A_g, ties to the lower index; a
    bucket without a kept token drops its evicted tokens.
  * Keys are not merged; the target itself enters its merge with gate 1 and
    weight A_t.
  * The compensation ratio is gated: R_t = (A_t + sum g_e A_e) / A_t, one per
    KV head, shared by the group's query heads.
  * RoPE re-positioning (step 6, off for long contexts on the page) turns each
    kept key from its original position to its slot's position, with the
    half-split pairing (element i with element i + d/2) and a caller-given
    base; the page names neither.
"""
from __future__ import annotations

import numpy as np

from .infokv import decode_attention, select_topk, window_attention_per_head


def vatp_union(A_hq: np.ndarray, V: np.ndarray):
    """Step 1-2 of the [SelKV] pipeline: VATP[h, j] = A[h, j] * ||v_{g(h), j}||_2
    and U[g, j] = max over h in group g of VATP[h, j].
    A_hq: [Hq, n]; V: [Hkv, n, d].  Returns (VATP [Hq, n], U [Hkv, n])."""
    A_hq = np.asarray(A_hq, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq, n = A_hq.shape
    Hkv = V.shape[0]
    G = Hq // Hkv
    vnorm = np.sqrt((V * V).sum(axis=2))                 # [Hkv, n]
    vatp = A_hq * np.repeat(vnorm, G, axis=0)
    U = vatp.reshape(Hkv, G, n).max(axis=1)
    return vatp, U


def route(kept_idx: np.ndarray, A_g: np.ndarray, n: int, bucket: int) -> np.ndarray:
    """Step 3 of the [SelKV] pipeline for one KV group: merge target of every
    token.  Returns target [n] int64: -1 for kept tokens and for evicted tokens
    whose bucket holds no kept token (those are dropped), otherwise the index of
    the bucket's kept token with the largest A_g (ties to the lower index)."""
    A_g = np.asarray(A_g, dtype=np.float64)
    kept = np.zeros(n, dtype=bool)
    kept[np.asarray(kept_idx)] = True
    target = np.full(n, -1, dtype=np.int64)
    for start in range(0, n, bucket):
        members = np.arange(start, min(start + bucket, n))
        cands = members[kept[members]]
        if cands.size == 0:
            continue
        best = cands[0]
        for j in cands[1:]:
            if A_g[j] > A_g[best]:
                best = j
        for e in members[~kept[members]]:
            target[e] = best
    return target


def gate(v_e: np.ndarray, v_t: np.ndarray) -> float:
    """Soft cosine gate g = max(cos(v_e, v_t), 0) ([SelKV] section 2, soft cosine
    gate); cos := 0 when either vector is zero."""
    a = np.asarray(v_e, dtype=np.float64)
    b = np.asarray(v_t, dtype=np.float64)
    den = np.sqrt((a * a).sum()) * np.sqrt((b * b).sum())
    c = float((a * b).sum() / den) if den > 0 else 0.0
    return max(c, 0.0)


def merge_group(V_g: np.ndarray, A_g: np.ndarray, kept_idx: np.ndarray,
                target: np.ndarray):
    """Steps 4-5 of the [SelKV] pipeline for one KV group.

    For each kept token t with routed tokens e:
        v'_t = (A_t v_t + sum_e g_e A_e v_e) / (A_t + sum_e g_e A_e)
        R_t  = (A_t + sum_e g_e A_e) / A_t
    Kept tokens with nothing routed keep v_t and R = 1.  Returns
    (V' [m, d] float64, lnR [m], gates [n] with NaN for non-routed tokens).
    """
    V_g = np.asarray(V_g, dtype=np.float64)
    A_g = np.asarray(A_g, dtype=np.float64)
    kept_idx = np.asarray(kept_idx, dtype=np.int64)
    n = V_g.shape[0]
    slot = {int(t): s for s, t in enumerate(kept_idx)}
    num = V_g[kept_idx] * A_g[kept_idx][:, None]
    den = A_g[kept_idx].copy()
    gates = np.full(n, np.nan)
    for e in range(n):
        t = int(target[e])
        if t < 0:
            continue
        g = gate(V_g[e], V_g[t])
        gates[e] = g
        s = slot[t]
        num[s] += g * A_g[e] * V_g[e]
        den[s] += g * A_g[e]
    Vp = np.empty_like(num)
    lnR = np.zeros(len(kept_idx))
    for s, t in enumerate(kept_idx):
        if den[s] > 0:
            Vp[s] = num[s] / den[s]
            lnR[s] = np.log(den[s] / A_g[t])
        else:                     # A_t underflowed to 0 with nothing merged
            Vp[s] = V_g[t]
    return Vp, lnR, gates


def selkv_layer(q_win: np.ndarray, K: np.ndarray, V: np.ndarray, m_keep: int,
                w: int, bucket: int, scale: float | None = None) -> dict:
    """The [SelKV] pipeline (steps 1-5; RoPE re-positioning off) for one layer.

    q_win: [Hq, w, d]; K, V: [Hkv, n, d] float64 values.  Returns a dict with
    A_hq, A_g, VATP, U, U32, idx (int32 [Hkv, m]), target [Hkv, n],
    gates [Hkv, n], Vp [Hkv, m, d] float64 and lnR [Hkv, m].
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hkv, n, d = K.shape
    A_hq = window_attention_per_head(q_win, K, scale)
    Hq = A_hq.shape[0]
    G = Hq // Hkv
    A_g = A_hq.reshape(Hkv, G, n).mean(axis=1)
    vatp, U = vatp_union(A_hq, V)
    U32 = U.astype(np.float32)
    idx = select_topk(U32, m_keep, w)
    target = np.empty((Hkv, n), dtype=np.int64)
    gates = np.empty((Hkv, n))
    Vp = np.empty((Hkv, m_keep, d))
    lnR = np.empty((Hkv, m_keep))
    for g in range(Hkv):
        target[g] = route(idx[g], A_g[g], n, bucket)
        Vp[g], lnR[g], gates[g] = merge_group(V[g], A_g[g], idx[g], target[g])
    return dict(A_hq=A_hq, A_g=A_g, VATP=vatp, U=U, U32=U32, idx=idx,
                target=target, gates=gates, Vp=Vp, lnR=lnR)


def compensated_decode(q: np.ndarray, K_c: np.ndarray, Vp: np.ndarray,
                       lnR: np.ndarray, alpha_bias: float,
                       scale: float | None = None):
    """Decode over the compacted cache with the alpha * ln R logit bias
    ([SelKV] section 2, attention compensation).  Returns (o', lse)."""
    return decode_attention(q, K_c, Vp, lnR, alpha_bias, scale)


def rope_apply(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotary position embedding of rows x [..., n, d] at positions pos [..., n]
    (the half-split pairing: element i turns with element i + d/2 by the angle
    pos * base^(-2i/d)).  float64."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    inv = base ** (-2.0 * np.arange(h) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def rope_reposition(K_c: np.ndarray, pos_old: np.ndarray, new_pos0: int, base: float) -> np.ndarray:
    """[SelKV] section 2, pipeline step 6 (RoPE re-positioning): the kept keys,
    embedded at their original positions pos_old [Hkv, m], are re-embedded at
    the contiguous positions new_pos0, new_pos0 + 1, ...: each row turns by
    (new - old) times the pair's frequency.  float64 [Hkv, m, d]."""
    m = np.asarray(pos_old).shape[-1]
    delta = (new_pos0 + np.arange(m))[None, :] - np.asarray(pos_old, dtype=np.int64)
    return rope_apply(K_c, delta, base)
