"""ctypes binding of libkvc (include/kvc.h): same names, argument marshalling only.

Tensors are torch tensors on the GPU (device memory); the current torch stream
is used unless ``stream`` is given.  Every function checks dtype, device and
contiguity, passes raw pointers and sizes, and raises ``KvcError`` on a
nonzero status.  All computation happens in the HIP library; if it is not
built, importing this module fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvc.so")

KVC_OK, KVC_ERR_ARG, KVC_ERR_DTYPE, KVC_ERR_WORKSPACE, KVC_ERR_HIP = 0, -1, -2, -3, -4
KVC_F32, KVC_BF16 = 0, 1

_c_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p
_i32, _i64, _f32, _f64, _sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_size_t

_SIGNATURES = {
    "kvc_version": ([], _i32),
    "kvc_status_string": ([_i32], ctypes.c_char_p),
    "kvc_last_error": ([], ctypes.c_char_p),
    "kvc_topk_entropy": ([_vp, _i32, _i64, _i64, _i64, _i32, _vp, _vp], _i32),
    "kvc_repr_distance": ([_vp, _vp, _i32, _i32, _i64, _i64, _f32, _vp, _vp], _i32),
    "kvc_score_window_attn_workspace_size": ([_i32, _i32, _i32, _i64, _i32, _i32, _i32], _sz),
    "kvc_score_window_attn": ([_vp, _vp, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _f32, _i32,
                               _vp, _vp, _sz, _vp], _i32),
    "kvc_score_window_attn_noalloc_max_workspace": ([], _sz),
    "kvc_score_window_attn_noalloc": ([_vp, _vp, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _f32,
                                       _i32, _vp, _vp], _i32),
    "kvc_fuse_scores_workspace_size": ([_i32, _i64], _sz),
    "kvc_fuse_scores": ([_vp, _vp, _vp, _i32, _i32, _i64, _f32, _vp, _vp, _vp, _sz, _vp], _i32),
    "kvc_uniform_budget": ([_f64, _i64, _i32, _c_i64p], _i32),
    "kvc_adaptive_budget": ([_vp, _i32, _i64, _i32, _i64, _c_i64p], _i32),
    "kvc_select_topk": ([_vp, _i32, _i32, _i64, _c_i64p, _i32, _vp, _vp], _i32),
    "kvc_compact": ([_vp, _vp, _i32, _i32, _i32, _i64, _i32, _vp, _c_i64p, _vp, _vp, _vp], _i32),
    "kvc_vatp_union": ([_vp, _vp, _i32, _i32, _i32, _i32, _i64, _i32, _vp, _vp, _vp], _i32),
    "kvc_vatp_union_gmax": ([_vp, _vp, _i32, _i32, _i32, _i64, _i32, _vp, _vp], _i32),
    "kvc_merge_gated": ([_vp, _vp, _i32, _vp, _i32, _i32, _i64, _i32, _vp, _c_i64p, _i32, _vp, _vp,
                         _vp, _vp], _i32),
    "kvc_compact_into": ([_vp, _vp, _i32, _i32, _i32, _i64, _i32, _vp, _c_i64p, _i64, _vp, _vp, _vp],
                         _i32),
    "kvc_fuse_scores_slots_workspace_size": ([_i32, _i32, _i64], _sz),
    "kvc_fuse_scores_slots": ([_vp, _vp, _i32, _i32, _i64, _f32, _vp, _vp, _vp, _sz, _vp], _i32),
    "kvc_append_entropy_scores": ([_vp, _vp, _i32, _i32, _i64, _vp, _i64, _i64, _vp], _i32),
    "kvc_active_scores": ([_vp, _vp, _i32, _vp, _f32, _i32, _i32, _i32, _i64, _i32, _f32, _vp, _vp],
                          _i32),
    "kvc_decode_attn_active": ([_vp, _vp, _vp, _i32, _vp, _f32, _vp, _i64, _i32, _i32, _i32, _i64,
                                _i32, _f32, _vp, _vp, _vp, _sz, _vp], _i32),
    "kvc_rope_reposition": ([_vp, _i32, _vp, _i64, _f64, _i32, _i32, _i64, _i32, _vp], _i32),
    "kvc_dropped_mass": ([_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _i32, _vp, _vp, _vp, _vp],
                         _i32),
    "kvc_decode_attn_workspace_size": ([_i32, _i32, _i64, _i32], _sz),
    "kvc_decode_attn": ([_vp, _vp, _vp, _i32, _vp, _f32, _i32, _i32, _i32, _i64, _i32, _f32, _vp,
                         _vp, _vp, _sz, _vp], _i32),
}


class KvcError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().kvc_last_error().decode() or lib().kvc_status_string(status).decode()
        super().__init__(f"{fn} failed ({status}): {msg}")


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded libkvc; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m kv_cache_compression_softmax_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes, f.restype = args, res
        _LIB = L
    return _LIB


def _check(fn: str, status: int):
    if status != KVC_OK:
        raise KvcError(fn, status)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KVC_BF16
    if t.dtype == torch.float32:
        return KVC_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _ptrs(ts, dtype=None):
    if ts is None:
        return None
    arr = (ctypes.c_void_p * len(ts))(*[_ptr(t, dtype) for t in ts])
    return ctypes.cast(arr, ctypes.c_void_p), arr      # keep arr alive with the call


def _i64s(vals):
    arr = (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])
    return arr


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(stream)


def _ws(nbytes: int, device, ws=None):
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError("workspace too small")
        return ws
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ entry points
def kvc_version() -> int:
    return lib().kvc_version()


def kvc_topk_entropy(logits: torch.Tensor, topk: int, H_out: torch.Tensor, vocab: int | None = None,
                     stream=None):
    """H_out[i] = top-k restricted entropy of row i of logits [rows, row_stride]."""
    rows, stride = logits.shape
    vocab = stride if vocab is None else vocab
    _check("kvc_topk_entropy", lib().kvc_topk_entropy(
        _ptr(logits), _dtype(logits), rows, vocab, stride, topk, _ptr(H_out, torch.float32),
        _stream(stream)))
    return H_out


def kvc_repr_distance(h_layers, h_final: torch.Tensor, tau: float, D_out: torch.Tensor, stream=None):
    """D_out[l, i] = 1 - cos(h_layers[l][i], h_final[i]) + tau."""
    n, hidden = h_final.shape
    hp, keep = _ptrs(h_layers, h_final.dtype)
    _check("kvc_repr_distance", lib().kvc_repr_distance(
        hp, _ptr(h_final), _dtype(h_final), len(h_layers), n, hidden, tau,
        _ptr(D_out, torch.float32), _stream(stream)))
    return D_out


def kvc_score_window_attn_workspace_size(L, Hq, Hkv, n, w, d, dtype) -> int:
    return lib().kvc_score_window_attn_workspace_size(L, Hq, Hkv, n, w, d, dtype)


def kvc_score_window_attn(q_win, k, scale: float, per_query_head, A_out: torch.Tensor,
                          ws: torch.Tensor | None = None, stream=None):
    """A_out from per-layer q_win [Hq, w, d] and k [Hkv, n, d]: [L, Hkv, n] for
    per_query_head 0 (or False), [L, Hq, n] for 1 (or True), [2, L, Hkv, n]
    (group mean, group max over heads) for 2."""
    L = len(k)
    Hq, w, d = q_win[0].shape
    Hkv, n, _ = k[0].shape
    dt = _dtype(k[0])
    need = kvc_score_window_attn_workspace_size(L, Hq, Hkv, n, w, d, dt)
    ws = _ws(need, k[0].device, ws)
    qp, kq = _ptrs(q_win, k[0].dtype)
    kp, kk = _ptrs(k, k[0].dtype)
    _check("kvc_score_window_attn", lib().kvc_score_window_attn(
        qp, kp, dt, L, Hq, Hkv, n, w, d, scale, int(per_query_head), _ptr(A_out, torch.float32),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return A_out


def kvc_score_window_attn_noalloc_max_workspace() -> int:
    return lib().kvc_score_window_attn_noalloc_max_workspace()


def kvc_score_window_attn_noalloc(q_win, k, scale: float, per_query_head: bool, A_out: torch.Tensor,
                                  stream=None):
    """kvc_score_window_attn with the library's fixed device scratch as its
    workspace: nothing is allocated (calls that overlap on one GPU race)."""
    L = len(k)
    Hq, w, d = q_win[0].shape
    Hkv, n, _ = k[0].shape
    qp, kq = _ptrs(q_win, k[0].dtype)
    kp, kk = _ptrs(k, k[0].dtype)
    _check("kvc_score_window_attn_noalloc", lib().kvc_score_window_attn_noalloc(
        qp, kp, _dtype(k[0]), L, Hq, Hkv, n, w, d, scale, int(per_query_head),
        _ptr(A_out, torch.float32), _stream(stream)))
    return A_out


def kvc_fuse_scores_workspace_size(L, n) -> int:
    return lib().kvc_fuse_scores_workspace_size(L, n)


def kvc_fuse_scores(A, D, H, alpha_fuse: float, S_out, Ebar_out=None, ws=None, stream=None):
    """S_out [L, Hkv, n] = alpha*A + (1-alpha)*softmax_tokens(D*H); Ebar_out [L]."""
    L, Hkv, n = A.shape
    ws = _ws(kvc_fuse_scores_workspace_size(L, n), A.device, ws)
    _check("kvc_fuse_scores", lib().kvc_fuse_scores(
        _ptr(A, torch.float32), _ptr(D, torch.float32), _ptr(H, torch.float32), L, Hkv, n,
        alpha_fuse, _ptr(S_out, torch.float32), _ptr(Ebar_out, torch.float32) if Ebar_out is not None else None,
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return S_out


def kvc_uniform_budget(keep_fraction: float, n: int, w: int) -> int:
    out = ctypes.c_int64()
    _check("kvc_uniform_budget", lib().kvc_uniform_budget(keep_fraction, n, w, ctypes.byref(out)))
    return out.value


def kvc_adaptive_budget(Ebar, B: int, w: int, n: int):
    """Host call: Ebar (sequence of float32) -> list of int k_l."""
    import numpy as np
    e = np.ascontiguousarray(np.asarray(Ebar, dtype=np.float32))
    L = e.size
    out = (ctypes.c_int64 * L)()
    _check("kvc_adaptive_budget", lib().kvc_adaptive_budget(
        e.ctypes.data_as(ctypes.c_void_p), L, B, w, n, out))
    return list(out)


def kvc_select_topk(S: torch.Tensor, k_keep, w: int, idx_out, stream=None):
    """idx_out[l] int32 [Hkv, k_keep[l]]: window plus top scores, ascending."""
    L, Hkv, n = S.shape
    kk = _i64s(k_keep)
    ip, keep = _ptrs(idx_out, torch.int32)
    _check("kvc_select_topk", lib().kvc_select_topk(
        _ptr(S, torch.float32), L, Hkv, n, kk, w, ip, _stream(stream)))
    return idx_out


def kvc_compact(K, V, idx, k_keep, K_out, V_out, stream=None):
    """K_out[l][g, j] = K[l][g, idx[l][g, j]] (and V); V/V_out may be None."""
    L = len(K)
    Hkv, n, d = K[0].shape
    dt = K[0].dtype
    kp, a1 = _ptrs(K, dt)
    vp = _ptrs(V, dt)
    ip, a2 = _ptrs(idx, torch.int32)
    kop, a3 = _ptrs(K_out, dt)
    vop = _ptrs(V_out, dt)
    _check("kvc_compact", lib().kvc_compact(
        kp, vp[0] if vp else None, _dtype(K[0]), L, Hkv, n, d, ip, _i64s(k_keep), kop,
        vop[0] if vop else None, _stream(stream)))
    return K_out, V_out


def kvc_compact_into(K, V, idx, k_keep, K_out, V_out, stream=None):
    """K_out[l][g, j] = K[l][g, idx[l][g, j]] for j < k_keep[l] (and V), where
    K_out[l] is [Hkv, out_rows, d]: rows past k_keep[l] are left as they are."""
    L = len(K)
    Hkv, n, d = K[0].shape
    out_rows = K_out[0].shape[1]
    dt = K[0].dtype
    for t in K_out + (V_out or []):
        if tuple(t.shape) != (Hkv, out_rows, d):
            raise ValueError("K_out / V_out must all be [Hkv, out_rows, d]")
    kp, a1 = _ptrs(K, dt)
    vp = _ptrs(V, dt)
    ip, a2 = _ptrs(idx, torch.int32)
    kop, a3 = _ptrs(K_out, dt)
    vop = _ptrs(V_out, dt)
    _check("kvc_compact_into", lib().kvc_compact_into(
        kp, vp[0] if vp else None, _dtype(K[0]), L, Hkv, n, d, ip, _i64s(k_keep), out_rows, kop,
        vop[0] if vop else None, _stream(stream)))
    return K_out, V_out


def kvc_fuse_scores_slots_workspace_size(L, Hkv, n) -> int:
    return lib().kvc_fuse_scores_slots_workspace_size(L, Hkv, n)


def kvc_fuse_scores_slots(A, E, alpha_fuse: float, S_out, Ebar_out=None, ws=None, stream=None):
    """S_out [L, Hkv, n] = alpha*A + (1-alpha)*softmax over each row of E [L, Hkv, n]."""
    L, Hkv, n = A.shape
    if tuple(E.shape) != (L, Hkv, n):
        raise ValueError("E must be shaped like A")
    ws = _ws(kvc_fuse_scores_slots_workspace_size(L, Hkv, n), A.device, ws)
    _check("kvc_fuse_scores_slots", lib().kvc_fuse_scores_slots(
        _ptr(A, torch.float32), _ptr(E, torch.float32), L, Hkv, n, alpha_fuse,
        _ptr(S_out, torch.float32), _ptr(Ebar_out, torch.float32) if Ebar_out is not None else None,
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return S_out


def kvc_append_entropy_scores(D, H, E, offset: int, stream=None):
    """E[l, g, offset + i] = D[l, i] * H[i] for every KV head g; E is [L, Hkv, cap]."""
    L, t = D.shape
    _, Hkv, cap = E.shape
    if H.shape[0] != t or E.shape[0] != L:
        raise ValueError("shape mismatch")
    _check("kvc_append_entropy_scores", lib().kvc_append_entropy_scores(
        _ptr(D, torch.float32), _ptr(H, torch.float32), L, Hkv, t, _ptr(E, torch.float32), cap,
        offset, _stream(stream)))
    return E


def kvc_vatp_union(A_hq: torch.Tensor, V, U_out: torch.Tensor, Ag_out: torch.Tensor, stream=None):
    """U_out = max over the group of A_hq * ||v||, Ag_out = group mean of A_hq."""
    L, Hq, n = A_hq.shape
    Hkv, _, d = V[0].shape
    vp, keep = _ptrs(V, V[0].dtype)
    _check("kvc_vatp_union", lib().kvc_vatp_union(
        _ptr(A_hq, torch.float32), vp, _dtype(V[0]), L, Hq, Hkv, n, d,
        _ptr(U_out, torch.float32), _ptr(Ag_out, torch.float32), _stream(stream)))
    return U_out, Ag_out


def kvc_vatp_union_gmax(A_gmax: torch.Tensor, V, U_out: torch.Tensor, stream=None):
    """U_out = A_gmax * ||v|| (A_gmax: the group max over heads, [L, Hkv, n])."""
    L, Hkv, n = A_gmax.shape
    d = V[0].shape[2]
    vp, keep = _ptrs(V, V[0].dtype)
    _check("kvc_vatp_union_gmax", lib().kvc_vatp_union_gmax(
        _ptr(A_gmax, torch.float32), vp, _dtype(V[0]), L, Hkv, n, d,
        _ptr(U_out, torch.float32), _stream(stream)))
    return U_out


def kvc_merge_gated(K, V, Ag: torch.Tensor, idx, m_keep, bucket: int, K_out, V_out, logR_out,
                    stream=None):
    """SelKV route + gate + merge + ln R, fused with the gather."""
    L = len(K)
    Hkv, n, d = K[0].shape
    dt = K[0].dtype
    kp, a1 = _ptrs(K, dt)
    vp, a2 = _ptrs(V, dt)
    ip, a3 = _ptrs(idx, torch.int32)
    kop, a4 = _ptrs(K_out, dt)
    vop, a5 = _ptrs(V_out, dt)
    lp, a6 = _ptrs(logR_out, torch.float32)
    _check("kvc_merge_gated", lib().kvc_merge_gated(
        kp, vp, _dtype(K[0]), _ptr(Ag, torch.float32), L, Hkv, n, d, ip, _i64s(m_keep), bucket,
        kop, vop, lp, _stream(stream)))
    return K_out, V_out, logR_out


def kvc_decode_attn_workspace_size(L, Hq, length, d) -> int:
    return lib().kvc_decode_attn_workspace_size(L, Hq, length, d)


def kvc_decode_attn(q, K, V, logR, alpha_bias: float, scale: float, o_out: torch.Tensor,
                    lse_out: torch.Tensor | None = None, ws=None, stream=None):
    """o_out [L, Hq, d] (and lse_out [L, Hq]) of one decode query per head."""
    L = len(K)
    Hq, d = q[0].shape
    Hkv, length, _ = K[0].shape
    dt = K[0].dtype
    ws = _ws(kvc_decode_attn_workspace_size(L, Hq, length, d), K[0].device, ws)
    qp, a1 = _ptrs(q, dt)
    kp, a2 = _ptrs(K, dt)
    vp, a3 = _ptrs(V, dt)
    lp = _ptrs(logR, torch.float32)
    _check("kvc_decode_attn", lib().kvc_decode_attn(
        qp, kp, vp, _dtype(K[0]), lp[0] if lp else None, alpha_bias, L, Hq, Hkv, length, d, scale,
        _ptr(o_out, torch.float32), _ptr(lse_out, torch.float32) if lse_out is not None else None,
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return o_out, lse_out


def kvc_active_scores(q, K, scale: float, score_out: torch.Tensor, utility=None, beta: float = 0.0,
                      stream=None):
    """score_out [L, Hkv, len] = max over each group's heads of scale*<q, k> (+ beta*utility)."""
    L = len(K)
    Hq, d = q[0].shape
    Hkv, length, _ = K[0].shape
    dt = K[0].dtype
    qp, a1 = _ptrs(q, dt)
    kp, a2 = _ptrs(K, dt)
    up = _ptrs(utility, torch.float32)
    _check("kvc_active_scores", lib().kvc_active_scores(
        qp, kp, _dtype(K[0]), up[0] if up else None, beta, L, Hq, Hkv, length, d, scale,
        _ptr(score_out, torch.float32), _stream(stream)))
    return score_out


def kvc_decode_attn_active(q, K, V, logR, alpha_bias: float, active, scale: float,
                           o_out: torch.Tensor, lse_out: torch.Tensor | None = None, ws=None,
                           stream=None):
    """Decode attention over the rows active[l][g, :] of each KV head's cache."""
    L = len(K)
    Hq, d = q[0].shape
    Hkv, length, _ = K[0].shape
    k_active = active[0].shape[1]
    for a in active:
        if tuple(a.shape) != (Hkv, k_active):
            raise ValueError("active index lists must all be [Hkv, k_active]")
    dt = K[0].dtype
    ws = _ws(kvc_decode_attn_workspace_size(L, Hq, length, d), K[0].device, ws)
    qp, a1 = _ptrs(q, dt)
    kp, a2 = _ptrs(K, dt)
    vp, a3 = _ptrs(V, dt)
    ip, a4 = _ptrs(active, torch.int32)
    lp = _ptrs(logR, torch.float32)
    _check("kvc_decode_attn_active", lib().kvc_decode_attn_active(
        qp, kp, vp, _dtype(K[0]), lp[0] if lp else None, alpha_bias, ip, k_active, L, Hq, Hkv,
        length, d, scale, _ptr(o_out, torch.float32),
        _ptr(lse_out, torch.float32) if lse_out is not None else None,
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return o_out, lse_out


def kvc_rope_reposition(K, pos_old, new_pos0: int, base: float, stream=None):
    """In place: row j of K[l][g] re-embedded from position pos_old[l][g, j] to new_pos0 + j."""
    L = len(K)
    Hkv, m, d = K[0].shape
    for p in pos_old:
        if tuple(p.shape) != (Hkv, m):
            raise ValueError("pos_old[l] must be [Hkv, m]")
    kp, a1 = _ptrs(K, K[0].dtype)
    pp, a2 = _ptrs(pos_old, torch.int32)
    _check("kvc_rope_reposition", lib().kvc_rope_reposition(
        kp, _dtype(K[0]), pp, new_pos0, base, L, Hkv, m, d, _stream(stream)))
    return K


def kvc_dropped_mass(lse_kept: torch.Tensor, lse_full: torch.Tensor, V, delta_out: torch.Tensor,
                     vmax_out: torch.Tensor, bound_out: torch.Tensor, stream=None):
    """delta_out [L, Hq] = 1 - exp(lse_kept - lse_full) (clamped at 0), vmax_out [L, Hkv] =
    largest value norm of the full cache V[l] [Hkv, n, d], bound_out = 2 * vmax * delta."""
    L, Hq = lse_full.shape
    Hkv, n, d = V[0].shape
    if tuple(lse_kept.shape) != (L, Hq) or len(V) != L:
        raise ValueError("lse_kept / lse_full must be [L, Hq] and V a list of L tensors")
    vp, keep = _ptrs(V, V[0].dtype)
    _check("kvc_dropped_mass", lib().kvc_dropped_mass(
        _ptr(lse_kept, torch.float32), _ptr(lse_full, torch.float32), vp, _dtype(V[0]), L, Hq, Hkv,
        n, d, _ptr(delta_out, torch.float32), _ptr(vmax_out, torch.float32),
        _ptr(bound_out, torch.float32), _stream(stream)))
    return delta_out, vmax_out, bound_out
