"""Plain float64 oracle of InfoKV's prefill scoring and compaction.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Page cited as [InfoKV]: "긴 추론을 위한 정보 인지형 KV 캐시 압축(InfoKV)"
(information-aware KV-cache compression for long reasoning), aitrends.kr article
68510; sections 핵심 기여 (Contributions), 방법론 (Method), 기술 상세 (Technical
detail) and 용어 해설 (Glossary).

Every function takes float64 arrays (convert bf16 inputs with
``oracle.precision.bf16_bits_to_f64`` first), computes in float64 with numpy,
and returns float64 unless stated otherwise.  Each step is the plain definition;
library primitives (sort, partition, matmul) are used as steps, nothing is
blocked, fused or reordered.

Readings taken where the page is silent or garbled:
  * A comes from layer l's own window queries and keys (the Technical-detail
    section speaks of each layer; the Method section's "last layer" is read as
    a garble).
  * Attention scale 1/sqrt(d); causal mask inside the window; no pooling of A.
  * GQA: query head h belongs to KV group floor(h / G), G = Hq / Hkv; A of a
    group is the mean over its G query heads.
  * Top-k entropy renormalises over the k largest logits; natural log.
  * D = 1 - cos + tau (the Technical-detail section adds tau); a zero-norm
    vector has cos := 0.
  * The token softmax of E runs over all n tokens of the layer, window included.
  * The window is always kept and counted inside k_l; the rest of the budget
    goes to the highest S, ties to the lower index; output indices ascend.
  * Budgets round down; the adaptive budget gives the remainder to the lowest
    layer indices.
  * Compression during decoding (the Technical-detail section applies it at
    prefill and again every 1024 generated tokens): each period re-scores the
    cache as it stands -- the kept slots of every (layer, KV head) followed by
    the new tokens -- with the same S, a fresh window (the last w new tokens)
    and the same budget.  A kept slot reuses the E = D * H its token had; a new
    token's E comes from its own logits row and hidden states.  Kept sets differ
    per KV head, so the softmax of E runs over each head's own slots.
"""
from __future__ import annotations

import math

import numpy as np


def topk_entropy(logits: np.ndarray, k: int) -> np.ndarray:
    """Top-k restricted entropy H_i of each row ([InfoKV] Method; Glossary).

    For row i take the multiset T of its k largest logits, form the softmax
    over T only (p_t = e^(t - m) / Z with m = max T, Z = sum over T of e^(t - m))
    and return H_i = -sum_t p_t ln p_t.  A term with p_t = 0 (a -inf logit
    taken because fewer than k logits are finite, or one that underflows)
    contributes 0, the limit of p ln p; a row with no finite logit has no
    entropy and gives NaN.  Which of several equal logits at the k-th place are
    taken does not matter: the multiset of values is the same.
    """
    z = np.asarray(logits, dtype=np.float64)
    rows, vocab = z.shape
    if not 1 <= k <= vocab:
        raise ValueError("need 1 <= k <= vocab")
    top = np.partition(z, vocab - k, axis=1)[:, vocab - k:]        # [rows, k]
    m = top.max(axis=1, keepdims=True)
    with np.errstate(invalid="ignore"):          # -inf - -inf in a row with no finite logit
        e = np.exp(top - m)
        Z = e.sum(axis=1, keepdims=True)
        p = e / Z
        logp = (top - m) - np.log(Z)
        terms = np.where(p > 0, p * logp, 0.0)
    H = -terms.sum(axis=1)
    H[~np.isfinite(m[:, 0])] = np.nan            # no finite logit in the row
    return H


def repr_distance(h_l: np.ndarray, h_final: np.ndarray, tau: float) -> np.ndarray:
    """D_i^(l) = 1 - cos(h_i^(l), h_i^(L)) + tau for every token i ([InfoKV] Method,
    Technical detail; Glossary: layer-wise representation evolution).

    h_l, h_final: [n, hidden].  Returns D: [n].
    """
    a = np.asarray(h_l, dtype=np.float64)
    b = np.asarray(h_final, dtype=np.float64)
    dot = (a * b).sum(axis=1)
    na = np.sqrt((a * a).sum(axis=1))
    nb = np.sqrt((b * b).sum(axis=1))
    denom = na * nb
    cos = np.divide(dot, denom, out=np.zeros_like(dot), where=denom > 0)
    return 1.0 - cos + tau


def window_attention_per_head(q_win: np.ndarray, k: np.ndarray,
                              scale: float | None = None) -> np.ndarray:
    """Observation-window attention of every query head ([InfoKV] Method,
    Technical detail).

    q_win: [Hq, w, d], the queries of the last w positions; k: [Hkv, n, d].
    Window row r sits at position p_r = n - w + r and sees keys j <= p_r.
    For head h (group g = floor(h / G)):
        s[r, j] = <q[h, r], k[g, j]> * scale   (scale = 1/sqrt(d) by default)
        P[r, :] = softmax over the visible j, 0 elsewhere
        A[h, j] = (1/w) * sum_r P[r, j]
    Returns A: [Hq, n].
    """
    q = np.asarray(q_win, dtype=np.float64)
    kk = np.asarray(k, dtype=np.float64)
    Hq, w, d = q.shape
    Hkv, n, d2 = kk.shape
    if d != d2 or Hq % Hkv != 0 or not 1 <= w <= n:
        raise ValueError("bad shapes")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    pos = n - w + np.arange(w)                       # position of each window row
    visible = np.arange(n)[None, :] <= pos[:, None]  # [w, n]
    A = np.zeros((Hq, n))
    for h in range(Hq):
        g = h // G
        s = (q[h] @ kk[g].T) * scale                 # [w, n]
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        P = e / e.sum(axis=1, keepdims=True)
        A[h] = P.mean(axis=0)
    return A


def window_attention(q_win: np.ndarray, k: np.ndarray, scale: float | None = None,
                     per_query_head: bool = False) -> np.ndarray:
    """A per KV group: the mean of ``window_attention_per_head`` over the G query
    heads of each group (the GQA reading).  Returns [Hkv, n], or [Hq, n] when
    ``per_query_head``.
    """
    A_h = window_attention_per_head(q_win, k, scale)
    if per_query_head:
        return A_h
    Hq = A_h.shape[0]
    Hkv = np.asarray(k).shape[0]
    G = Hq // Hkv
    return A_h.reshape(Hkv, G, -1).mean(axis=1)


def fuse_scores(A: np.ndarray, D_l: np.ndarray, H: np.ndarray, alpha: float):
    """Importance fusion of one layer ([InfoKV] Contributions, Method, Technical
    detail).

    E_i = D_i^(l) * H_i; sigma = softmax of E over the n tokens of the layer;
    S[g, i] = alpha * A[g, i] + (1 - alpha) * sigma_i.  Ebar = mean_i E_i is the
    layer's entropy share used by the adaptive budget.
    Returns (S [Hkv, n], Ebar, E [n], sigma [n]).
    """
    A = np.asarray(A, dtype=np.float64)
    E = np.asarray(D_l, dtype=np.float64) * np.asarray(H, dtype=np.float64)
    e = np.exp(E - E.max())
    sigma = e / e.sum()
    S = alpha * A + (1.0 - alpha) * sigma[None, :]
    return S, float(E.mean()), E, sigma


def uniform_budget(keep_fraction: float, n: int) -> int:
    """The same k for every layer ([InfoKV] Contributions, Technical detail):
    floor(keep_fraction * n)."""
    return int(math.floor(keep_fraction * n))


def adaptive_budget(Ebar, B: int, w: int, n: int) -> np.ndarray:
    """k_l = (Ebar_l / sum_m Ebar_m) * B ([InfoKV] Method, Technical detail;
    Glossary: adaptive budget allocation), rounded down, the B - sum k_l
    leftover tokens given one each to the lowest layer indices, then clamped
    to [w, n].  ``Ebar`` is taken as given (the GPU rounds it to float32).
    """
    e = np.asarray(Ebar, dtype=np.float64)
    x = e / e.sum() * B
    k = np.floor(x).astype(np.int64)
    r = int(B - k.sum())
    k[:r] += 1
    return np.clip(k, w, n)


def select_topk(S32: np.ndarray, k_keep: int, w: int) -> np.ndarray:
    """Kept token indices of every KV group ([InfoKV] Method, Technical detail).

    S32: float32 scores [Hkv, n] -- selection works on the float32-rounded S.
    The last w tokens are always kept.  The other k_keep - w places go to the
    tokens of [0, n - w) with the largest S, ties to the lower index.  If
    k_keep <= w only the last k_keep tokens are kept.  Indices are returned in
    ascending order, int32 [Hkv, k_keep].
    """
    S32 = np.asarray(S32, dtype=np.float32)
    Hkv, n = S32.shape
    if not 1 <= k_keep <= n or not 0 <= w <= n:
        raise ValueError("need 1 <= k_keep <= n and 0 <= w <= n")
    out = np.empty((Hkv, k_keep), dtype=np.int32)
    for g in range(Hkv):
        if k_keep <= w:
            out[g] = np.arange(n - k_keep, n)
            continue
        body = np.arange(n - w)
        # lexsort: last key is primary -> descending S, then ascending index
        order = np.lexsort((body, -S32[g, : n - w].astype(np.float64)))
        kept = np.concatenate([order[: k_keep - w], np.arange(n - w, n)])
        out[g] = np.sort(kept)
    return out


def compact(K: np.ndarray, V: np.ndarray, idx: np.ndarray):
    """Order-preserving gather of the kept rows: K_c[g, j] = K[g, idx[g, j]] and
    likewise V.  Works on raw bit arrays (uint16 for bf16), so the copy is exact.
    """
    ii = np.asarray(idx, dtype=np.int64)[:, :, None]
    return (np.take_along_axis(np.asarray(K), ii, axis=1),
            np.take_along_axis(np.asarray(V), ii, axis=1))


def decode_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                     logR: np.ndarray | None = None, alpha_bias: float = 0.0,
                     scale: float | None = None):
    """One decode query per query head over a KV cache.

    q: [Hq, d]; K, V: [Hkv, len, d]; logR: [Hkv, len] or None.
    logits[h, t] = <q_h, k_{g(h), t}> * scale + alpha_bias * logR[g(h), t]
    (the logit bias of [SelKV] section 2, "Attention compensation"; with
    logR None it is plain attention).  Returns (o [Hq, d], lse [Hq]) where lse
    is the natural log of the softmax normaliser.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq, d = q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((Hq, V.shape[2]))
    lse = np.zeros(Hq)
    for h in range(Hq):
        g = h // G
        s = (K[g] @ q[h]) * scale
        if logR is not None:
            s = s + alpha_bias * np.asarray(logR, dtype=np.float64)[g]
        m = s.max()
        e = np.exp(s - m)
        Z = e.sum()
        o[h] = (e / Z) @ V[g]
        lse[h] = m + math.log(Z)
    return o, lse


def dropped_mass_bound(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                       kept: np.ndarray, scale: float | None = None):
    """Dropped-attention-mass bound of [RECAS] section 2.B ("formal bound").

    Page cited as [RECAS]: gist.science technical summary of reasoning-aware,
    error-bounded KV-cache compression and sparse attention (rs-10952127).

    For every query head h: p = softmax over the full cache, delta = total p of
    the evicted tokens, o = full-cache output, o' = output over the kept tokens
    only (the softmax renormalised over them), V_max = the largest value norm
    of the group.  Returns (o, o', delta [Hq], V_max [Hq]); the bound is
    ||o - o'||_2 <= 2 * V_max * delta.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq, d = q.shape
    Hkv, n, _ = K.shape
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((Hq, V.shape[2]))
    o2 = np.zeros_like(o)
    delta = np.zeros(Hq)
    vmax = np.zeros(Hq)
    for h in range(Hq):
        g = h // G
        s = (K[g] @ q[h]) * scale
        p = np.exp(s - s.max())
        p /= p.sum()
        keep = np.zeros(n, dtype=bool)
        keep[np.asarray(kept[g])] = True
        delta[h] = p[~keep].sum()
        o[h] = p @ V[g]
        pk = np.where(keep, p, 0.0)
        o2[h] = (pk / pk.sum()) @ V[g]
        vmax[h] = np.sqrt((V[g] ** 2).sum(axis=1)).max()
    return o, o2, delta, vmax


def infokv_layer(q_win, k, D_l, H, alpha: float, k_keep: int, w: int,
                 scale: float | None = None):
    """One layer of the InfoKV path: A, fuse, select ([InfoKV] Method).
    Returns (A [Hkv, n], S float64, S32 float32, Ebar, idx int32)."""
    A = window_attention(q_win, k, scale)
    S, Ebar, _, _ = fuse_scores(A, D_l, H, alpha)
    S32 = S.astype(np.float32)
    idx = select_topk(S32, k_keep, w)
    return A, S, S32, Ebar, idx


def fuse_scores_slots(A: np.ndarray, E: np.ndarray, alpha: float):
    """Importance fusion over the cache slots of one layer, one row per KV head
    ([InfoKV] Method: the fusion formula; Technical detail: compression during
    decoding).

    E[g, j] is the entropy score of the token held by slot j of head g;
    sigma[g] = softmax of E[g] over the head's slots;
    S[g, j] = alpha * A[g, j] + (1 - alpha) * sigma[g, j].  Ebar = mean of E.
    Returns (S [Hkv, n], Ebar, sigma [Hkv, n]).
    """
    A = np.asarray(A, dtype=np.float64)
    E = np.asarray(E, dtype=np.float64)
    sigma = np.empty_like(E)
    for g in range(E.shape[0]):
        e = np.exp(E[g] - E[g].max())
        sigma[g] = e / e.sum()
    S = alpha * A + (1.0 - alpha) * sigma
    return S, float(E.mean()), sigma


def recompress_period(q_win, K_cache, V_cache, E_kept, D_new, H_new, alpha: float,
                      k_keep: int, w: int, scale: float | None = None):
    """One period of compression during decoding, for one layer ([InfoKV]
    Technical detail: compression every 1024 generated tokens; Method).

    K_cache, V_cache [Hkv, k_old + t, d]: each head's kept slots (ascending
    positions) followed by the t new tokens.  E_kept [Hkv, k_old]: the entropy
    scores the kept slots carry.  D_new [t], H_new [t]: the new tokens'
    representation distance at this layer and top-k entropy.  q_win [Hq, w, d]:
    the fresh window, the queries of the last w new tokens.

    E = [E_kept | D_new * H_new] per head; A = window attention over the cache;
    S = fuse_scores_slots(A, E); the k_keep slots kept per head (the last w
    always); the kept slots' K, V and E are gathered in slot order.
    Returns a dict with A, E, S, S32, idx, Kc, Vc, E_next.
    """
    E_kept = np.asarray(E_kept, dtype=np.float64)
    e_new = np.asarray(D_new, dtype=np.float64) * np.asarray(H_new, dtype=np.float64)
    Hkv = E_kept.shape[0]
    E = np.concatenate([E_kept, np.repeat(e_new[None, :], Hkv, axis=0)], axis=1)
    A = window_attention(q_win, K_cache, scale)
    S, _, _ = fuse_scores_slots(A, E, alpha)
    S32 = S.astype(np.float32)
    idx = select_topk(S32, k_keep, w)
    Kc, Vc = compact(K_cache, V_cache, idx)
    E_next = np.take_along_axis(E, idx.astype(np.int64), axis=1)
    return {"A": A, "E": E, "S": S, "S32": S32, "idx": idx, "Kc": Kc, "Vc": Vc,
            "E_next": E_next}
