"""Host orchestration of the two compression paths over the C ABI.

InfoKV ([InfoKV] Method / Technical detail): H (top-k entropy of the final
logits), D (layer-wise distance), A (window attention), fuse -> S, budget,
select -> kept indices, compact -> K_c, V_c.

SelKV ([SelKV] section 2, pipeline steps 1-5): per-head window attention, VATP
union, select, then the fused route / gate / merge / ln R / gather.

A plan allocates every output and workspace once; ``run`` only enqueues HIP
work (plus, for the adaptive budget, one device-to-host copy of L floats and
the host budget call).  Nothing here computes on the CPU.
"""
from __future__ import annotations

import math

import torch

from . import binding as B
from .configs import Workload


def _carve(pool: torch.Tensor, sizes, shape_of):
    """Per-layer views into one flat buffer (no allocation)."""
    out, off = [], 0
    for s in sizes:
        shp = shape_of(s)
        num = math.prod(shp)
        out.append(pool[off:off + num].view(shp))
        off += num
    return out


class InfoKVPlan:
    def __init__(self, w: Workload, device="cuda"):
        assert w.method == "infokv"
        self.w = w
        self.device = device
        L, Hkv, n, d = w.layers, w.heads_kv, w.n, w.head_dim
        f32 = torch.float32
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.scale = 1.0 / math.sqrt(d)
        self.H = torch.empty(n, dtype=f32, device=device)
        self.D = torch.empty(L, n, dtype=f32, device=device)
        self.A = torch.empty(L, Hkv, n, dtype=f32, device=device)
        self.S = torch.empty(L, Hkv, n, dtype=f32, device=device)
        self.Ebar = torch.empty(L, dtype=f32, device=device)
        dtc = B.KVC_BF16 if w.dtype == "bf16" else B.KVC_F32
        self.ws_attn = torch.empty(max(1, B.kvc_score_window_attn_workspace_size(
            L, w.heads_q, Hkv, n, w.window, d, dtc)), dtype=torch.uint8, device=device)
        self.ws_fuse = torch.empty(max(1, B.kvc_fuse_scores_workspace_size(L, n)),
                                   dtype=torch.uint8, device=device)
        budgets = w.budgets()
        if budgets is not None:
            self.k = [B.kvc_uniform_budget(w.keep_fraction, n, w.window)] * L
            total = sum(self.k)
        else:
            self.k = None
            total = w.adaptive_total()
        self.total = total
        # logits processed in row chunks: consecutive chunks alternate between the
        # launch stream and this one, so one chunk's last round of rows overlaps
        # the next chunk's first (the chunks are independent)
        self.entropy_rows = w.logits_chunk_rows or n
        self.side = torch.cuda.Stream(device=device)
        self.ev = [torch.cuda.Event(), torch.cuda.Event()]
        self.idx_pool = torch.empty(Hkv * total, dtype=torch.int32, device=device)
        self.kc_pool = torch.empty(Hkv * total * d, dtype=dt, device=device)
        self.vc_pool = torch.empty(Hkv * total * d, dtype=dt, device=device)
        if self.k is not None:
            self._views(self.k)

    def _views(self, k):
        Hkv, d = self.w.heads_kv, self.w.head_dim
        self.idx = _carve(self.idx_pool, k, lambda s: (Hkv, s))
        self.Kc = _carve(self.kc_pool, k, lambda s: (Hkv, s, d))
        self.Vc = _carve(self.vc_pool, k, lambda s: (Hkv, s, d))

    def run(self, inp: dict, stream=None, mark=None):
        """Enqueue the whole path.  ``mark(name)``, if given, is called before
        the first step ("start") and after each step (for event timing)."""
        w = self.w
        mark = mark or (lambda name: None)
        mark("start")
        chunk = self.entropy_rows
        logits = inp["logits"]
        if chunk >= w.n:
            B.kvc_topk_entropy(logits, w.topk_entropy, self.H, stream=stream)
        else:
            s0 = stream if isinstance(stream, torch.cuda.Stream) else \
                (torch.cuda.ExternalStream(stream) if stream is not None else torch.cuda.current_stream())
            self.ev[0].record(s0)
            self.side.wait_event(self.ev[0])
            for ci, r0 in enumerate(range(0, w.n, chunk)):
                r1 = min(w.n, r0 + chunk)
                B.kvc_topk_entropy(logits[r0:r1], w.topk_entropy, self.H[r0:r1],
                                   stream=s0 if ci % 2 == 0 else self.side)
            self.ev[1].record(self.side)
            s0.wait_event(self.ev[1])
        mark("topk_entropy")
        B.kvc_repr_distance(inp["h"], inp["h_final"], w.tau, self.D, stream=stream)
        mark("repr_distance")
        B.kvc_score_window_attn(inp["q_win"], inp["k"], self.scale, False, self.A,
                                ws=self.ws_attn, stream=stream)
        mark("window_attn")
        B.kvc_fuse_scores(self.A, self.D, self.H, w.alpha_fuse, self.S, self.Ebar,
                          ws=self.ws_fuse, stream=stream)
        mark("fuse_scores")
        if w.adaptive_fraction:
            ebar = self.Ebar.cpu()                       # the one host sync of the path
            k = B.kvc_adaptive_budget(ebar.numpy(), self.total, w.window, w.n)
            if sum(k) != self.total:
                raise RuntimeError("adaptive budget clamp changed the total")
            self.k = k
            self._views(k)
        B.kvc_select_topk(self.S, self.k, w.window, self.idx, stream=stream)
        mark("select_topk")
        B.kvc_compact(inp["k"], inp["v"], self.idx, self.k, self.Kc, self.Vc, stream=stream)
        mark("compact")
        return self

    def probe(self, inp: dict, q, stream=None, mark=None):
        """A full-attention probe step of [RECAS] section 2.B over the compacted
        cache: decode one query per head (q[l] [Hq, d]) over the kept rows and
        over the full cache, then the exact dropped mass delta [L, Hq], the
        largest value norm V_max [L, Hkv] and the bound 2 * V_max * delta.
        Returns a dict of the plan's own buffers (allocated on the first call,
        overwritten by the next)."""
        w = self.w
        mark = mark or (lambda name: None)
        if getattr(self, "_probe", None) is None:
            L, Hq, Hkv, d, dev = w.layers, w.heads_q, w.heads_kv, w.head_dim, self.S.device
            f32 = torch.float32
            nbytes = B.kvc_decode_attn_workspace_size(L, Hq, w.n, d)
            self._probe = {"o_kept": torch.empty(L, Hq, d, dtype=f32, device=dev),
                           "lse_kept": torch.empty(L, Hq, dtype=f32, device=dev),
                           "o_full": torch.empty(L, Hq, d, dtype=f32, device=dev),
                           "lse_full": torch.empty(L, Hq, dtype=f32, device=dev),
                           "delta": torch.empty(L, Hq, dtype=f32, device=dev),
                           "vmax": torch.empty(L, Hkv, dtype=f32, device=dev),
                           "bound": torch.empty(L, Hq, dtype=f32, device=dev),
                           "ws": torch.empty(max(1, nbytes), dtype=torch.uint8, device=dev)}
        p = self._probe
        if len(set(self.k)) != 1:
            raise ValueError("probe() needs the same budget in every layer (one compacted length)")
        mark("start")
        B.kvc_decode_attn(q, self.Kc, self.Vc, None, 0.0, self.scale, p["o_kept"], p["lse_kept"],
                          ws=p["ws"], stream=stream)
        mark("decode_kept")
        B.kvc_decode_attn(q, inp["k"], inp["v"], None, 0.0, self.scale, p["o_full"], p["lse_full"],
                          ws=p["ws"], stream=stream)
        mark("decode_full")
        B.kvc_dropped_mass(p["lse_kept"], p["lse_full"], inp["v"], p["delta"], p["vmax"], p["bound"],
                           stream=stream)
        mark("dropped_mass")
        return p


class InfoKVDecodePlan:
    """Compression repeated during decoding ([InfoKV] Technical detail: at
    prefill and again every ``period`` generated tokens, e.g. 1024).

    After the prefill compaction every (layer, KV head) holds k kept slots.  The
    cache buffers hold cap = k + period rows per head: the kept slots first, then
    the tokens decoded since.  A period re-scores all cap slots -- window
    attention with the fresh window, E = D * H carried by the kept slots and
    computed for the new tokens only, the per-head slot softmax -- keeps k per
    head (the last w always) and gathers K, V and E into the other buffer, whose
    rows [k, cap) then take the next period's tokens.  Uniform budget only.
    """

    def __init__(self, w: Workload, period: int = 1024, device="cuda"):
        assert w.method == "infokv" and not w.adaptive_fraction
        self.w, self.period, self.device = w, period, device
        L, Hq, Hkv, d = w.layers, w.heads_q, w.heads_kv, w.head_dim
        f32 = torch.float32
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        dtc = B.KVC_BF16 if w.dtype == "bf16" else B.KVC_F32
        self.scale = 1.0 / math.sqrt(d)
        self.k = B.kvc_uniform_budget(w.keep_fraction, w.n, w.window)
        self.cap = cap = self.k + period
        self.K = [[torch.empty(Hkv, cap, d, dtype=dt, device=device) for _ in range(L)] for _ in range(2)]
        self.V = [[torch.empty(Hkv, cap, d, dtype=dt, device=device) for _ in range(L)] for _ in range(2)]
        self.E = [torch.empty(L, Hkv, cap, dtype=f32, device=device) for _ in range(2)]
        self.cur = 0
        self.H = torch.empty(period, dtype=f32, device=device)
        self.D = torch.empty(L, period, dtype=f32, device=device)
        self.A = torch.empty(L, Hkv, cap, dtype=f32, device=device)
        self.S = torch.empty(L, Hkv, cap, dtype=f32, device=device)
        self.idx = [torch.empty(Hkv, self.k, dtype=torch.int32, device=device) for _ in range(L)]
        self.ws_attn = torch.empty(max(1, B.kvc_score_window_attn_workspace_size(
            L, Hq, Hkv, cap, w.window, d, dtc)), dtype=torch.uint8, device=device)
        self.ws_fuse = torch.empty(max(1, B.kvc_fuse_scores_slots_workspace_size(L, Hkv, cap)),
                                   dtype=torch.uint8, device=device)

    def _e_rows(self, E):
        return [E[l].unsqueeze(-1) for l in range(self.w.layers)]      # [Hkv, rows, 1] views

    def start(self, prefill: "InfoKVPlan", inp: dict, stream=None):
        """The slots after the prefill compaction: the kept K and V rows and the
        E = D * H of their tokens (per head, gathered by the kept indices)."""
        w = self.w
        if list(prefill.k) != [self.k] * w.layers:
            raise ValueError("the prefill plan must use the same uniform budget")
        B.kvc_compact_into(inp["k"], inp["v"], prefill.idx, prefill.k, self.K[0], self.V[0],
                           stream=stream)
        E_full = torch.empty(w.layers, w.heads_kv, w.n, dtype=torch.float32, device=self.device)
        B.kvc_append_entropy_scores(prefill.D, prefill.H, E_full, 0, stream=stream)
        B.kvc_compact_into(self._e_rows(E_full), None, prefill.idx, prefill.k,
                           self._e_rows(self.E[0]), None, stream=stream)
        self.cur = 0
        return self

    def append(self, new: dict):
        """The decoder's own writes, outside the compression path: the new
        tokens' K and V rows go after the kept slots of the current buffer."""
        for l in range(self.w.layers):
            self.K[self.cur][l][:, self.k:].copy_(new["k"][l])
            self.V[self.cur][l][:, self.k:].copy_(new["v"][l])

    def run(self, new: dict, stream=None, mark=None):
        """One period over the current buffer.  ``new`` holds the period's
        logits [period, vocab], hidden states h (L x [period, hidden]) and
        h_final, and the fresh window queries q_win (L x [Hq, w, d])."""
        w = self.w
        L, k = w.layers, self.k
        cur, nxt = self.cur, 1 - self.cur
        mark = mark or (lambda name: None)
        mark("start")
        B.kvc_topk_entropy(new["logits"], w.topk_entropy, self.H, stream=stream)
        mark("topk_entropy")
        B.kvc_repr_distance(new["h"], new["h_final"], w.tau, self.D, stream=stream)
        mark("repr_distance")
        B.kvc_score_window_attn(new["q_win"], self.K[cur], self.scale, False, self.A,
                                ws=self.ws_attn, stream=stream)
        mark("window_attn")
        B.kvc_append_entropy_scores(self.D, self.H, self.E[cur], k, stream=stream)
        B.kvc_fuse_scores_slots(self.A, self.E[cur], w.alpha_fuse, self.S, ws=self.ws_fuse,
                                stream=stream)
        mark("fuse_scores")
        B.kvc_select_topk(self.S, [k] * L, w.window, self.idx, stream=stream)
        mark("select_topk")
        B.kvc_compact_into(self.K[cur], self.V[cur], self.idx, [k] * L, self.K[nxt], self.V[nxt],
                           stream=stream)
        B.kvc_compact_into(self._e_rows(self.E[cur]), None, self.idx, [k] * L,
                           self._e_rows(self.E[nxt]), None, stream=stream)
        mark("compact")
        self.cur = nxt
        return self


class SelKVPlan:
    def __init__(self, w: Workload, device="cuda"):
        assert w.method == "selkv"
        self.w = w
        L, Hq, Hkv, n, d = w.layers, w.heads_q, w.heads_kv, w.n, w.head_dim
        f32 = torch.float32
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        dtc = B.KVC_BF16 if w.dtype == "bf16" else B.KVC_F32
        self.scale = 1.0 / math.sqrt(d)
        # window attention's group mean (A_g) and group max over the query heads
        self.A2 = torch.empty(2, L, Hkv, n, dtype=f32, device=device)
        self.Ag, self.Amax = self.A2[0], self.A2[1]
        self.U = torch.empty(L, Hkv, n, dtype=f32, device=device)
        self.ws_attn = torch.empty(max(1, B.kvc_score_window_attn_workspace_size(
            L, Hq, Hkv, n, w.window, d, dtc)), dtype=torch.uint8, device=device)
        m = B.kvc_uniform_budget(w.keep_fraction, n, w.window)
        self.m = [m] * L
        self.idx = [torch.empty(Hkv, m, dtype=torch.int32, device=device) for _ in range(L)]
        self.Kc = [torch.empty(Hkv, m, d, dtype=dt, device=device) for _ in range(L)]
        self.Vc = [torch.empty(Hkv, m, d, dtype=dt, device=device) for _ in range(L)]
        self.logR = [torch.empty(Hkv, m, dtype=f32, device=device) for _ in range(L)]

    def run(self, inp: dict, stream=None, mark=None):
        w = self.w
        mark = mark or (lambda name: None)
        mark("start")
        B.kvc_score_window_attn(inp["q_win"], inp["k"], self.scale, 2, self.A2,
                                ws=self.ws_attn, stream=stream)
        mark("window_attn")
        B.kvc_vatp_union_gmax(self.Amax, inp["v"], self.U, stream=stream)
        mark("vatp_union")
        B.kvc_select_topk(self.U, self.m, w.window, self.idx, stream=stream)
        mark("select_topk")
        B.kvc_merge_gated(inp["k"], inp["v"], self.Ag, self.idx, self.m, w.bucket,
                          self.Kc, self.Vc, self.logR, stream=stream)
        mark("merge_gated")
        return self

    def _decode_buffers(self):
        if getattr(self, "_dec", None) is None:
            w = self.w
            L, Hq, d, dev = w.layers, w.heads_q, w.head_dim, self.U.device
            f32 = torch.float32
            nbytes = B.kvc_decode_attn_workspace_size(L, Hq, w.n, d)   # the full length bounds both
            self._dec = (torch.empty(L, Hq, d, dtype=f32, device=dev), torch.empty(L, Hq, dtype=f32, device=dev),
                         torch.empty(L, Hq, d, dtype=f32, device=dev), torch.empty(L, Hq, dtype=f32, device=dev),
                         torch.empty(max(1, nbytes), dtype=torch.uint8, device=dev))
        return self._dec

    def decode_check(self, inp: dict, stream=None, mark=None, active_fraction: float = 0.0):
        """Compensated decode over the compacted cache and plain decode over the
        full cache, one query per head and layer: (o', lse', o, lse).  The output
        buffers are the plan's own (allocated on the first call) and are
        overwritten by the next call.

        With ``active_fraction`` > 0 it also runs RECAS's active-set step over
        the compacted cache ([RECAS] section 2.C): sparse scores (the compensated
        logit, max over the group's heads: compatibility plus alpha * ln R as
        the utility), the top floor(fraction * m) entries per KV head, attention
        over them; the outputs go to ``self.o_active``, ``self.lse_active``."""
        w = self.w
        mark = mark or (lambda name: None)
        q = [inp["q_dec"][l] for l in range(w.layers)]
        o_c, l_c, o_f, l_f, ws = self._decode_buffers()
        mark("start")
        B.kvc_decode_attn(q, self.Kc, self.Vc, self.logR, w.alpha_bias, self.scale, o_c, l_c,
                          ws=ws, stream=stream)
        mark("decode_compacted")
        B.kvc_decode_attn(q, inp["k"], inp["v"], None, 0.0, self.scale, o_f, l_f, ws=ws, stream=stream)
        mark("decode_full")
        if active_fraction > 0:
            L, m = w.layers, self.m[0]
            kt = max(1, int(math.floor(active_fraction * m)))
            if getattr(self, "_act", None) is None or self._act[0] != kt:
                dev = self.U.device
                self._act = (kt, torch.empty(L, w.heads_kv, m, dtype=torch.float32, device=dev),
                             [torch.empty(w.heads_kv, kt, dtype=torch.int32, device=dev) for _ in range(L)])
                self.o_active = torch.empty_like(o_c)
                self.lse_active = torch.empty_like(l_c)
            _, sc, act = self._act
            B.kvc_active_scores(q, self.Kc, self.scale, sc, self.logR, w.alpha_bias, stream=stream)
            mark("active_scores")
            B.kvc_select_topk(sc, [kt] * L, 0, act, stream=stream)
            mark("active_select")
            B.kvc_decode_attn_active(q, self.Kc, self.Vc, self.logR, w.alpha_bias, act, self.scale,
                                     self.o_active, self.lse_active, ws=ws, stream=stream)
            mark("decode_active")
        return o_c, l_c, o_f, l_f
