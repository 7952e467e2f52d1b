/*
 * kvc.h -- C ABI of the MI355X (gfx950) KV-cache scoring and compaction library.
 *
 * Pages cited:
 *   [InfoKV] "긴 추론을 위한 정보 인지형 KV 캐시 압축(InfoKV)" (information-aware
 *            KV-cache compression for long reasoning), aitrends.kr article 68510;
 *            sections Contributions, Method, Technical detail, Glossary.
 *   [SelKV]  "SelKV: Selective KV Cache Merging with Per-Token Merge-or-Drop and
 *            Attention Compensation", gist.science paper 2607.16213; section 2
 *            (soft cosine gate, attention compensation, pipeline overview).
 *   [RECAS]  gist.science technical summary rs-10952127 (reasoning-aware,
 *            error-bounded KV-cache compression); section 2.B, formal bound.
 *
 * Conventions shared by every entry point
 *   - Batch 1.  Tensors are dense and row-major; shapes are given innermost last.
 *   - "device" pointers are HIP device memory owned by the caller; the library
 *     never allocates, frees or keeps them.  "host" arrays are read during the
 *     call only.  A per-layer tensor is passed as a host array of L device
 *     pointers (one tensor per layer, as a model holds its cache).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without waiting, except kvc_adaptive_budget and
 *     kvc_uniform_budget, which are host-only.
 *   - dtype: KVC_F32 (binary32) or KVC_BF16 (bfloat16 bits).  Scores are float32
 *     and indices int32 regardless of dtype; arithmetic accumulates in float32.
 *   - Arguments are checked before anything is launched.  On error nothing is
 *     enqueued and a negative status is returned; kvc_last_error() then holds a
 *     message for the calling thread.  NaN or Inf inputs are not supported and
 *     not checked.
 *   - Workspace: an entry point that needs scratch device memory takes `ws`,
 *     `ws_bytes`; kvc_*_workspace_size() with the same shape arguments gives the
 *     minimum size.  Workspace contents need not be initialised and are not
 *     preserved.  Two calls that share a workspace must be ordered (same stream).
 */
#ifndef KVC_H_
#define KVC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum kvc_status {
  KVC_OK = 0,
  KVC_ERR_ARG = -1,        /* null pointer, bad shape or out-of-range parameter */
  KVC_ERR_DTYPE = -2,      /* unsupported dtype for this entry point           */
  KVC_ERR_WORKSPACE = -3,  /* ws missing or smaller than *_workspace_size()     */
  KVC_ERR_HIP = -4         /* a HIP launch or device query failed              */
};

enum kvc_dtype { KVC_F32 = 0, KVC_BF16 = 1 };

/* Largest per-launch limits (checked; exceeding them is KVC_ERR_ARG). */
#define KVC_MAX_LAYERS 1024
#define KVC_MAX_TOPK_ENTROPY 1024

/* Library version (major * 10000 + minor * 100 + patch). */
int kvc_version(void);
/* Static text for a status code. */
const char* kvc_status_string(int status);
/* Message of the calling thread's last failed call ("" if none). */
const char* kvc_last_error(void);

/*
 * Top-k restricted entropy of each logits row ([InfoKV] Method; Glossary).
 * For row i: T = the k largest logits (as a multiset), p_t = softmax over T
 * only, H[i] = -sum_t p_t ln p_t (natural log).  0 <= H <= ln k.  Logits may
 * be -inf (a masked vocabulary): a term with p_t = 0 contributes 0, the limit
 * of p ln p; a row with no finite logit gives NaN.  NaN logits are unsupported.
 *   logits     device, [rows, row_stride] of dtype; the first `vocab` columns
 *              of each row are used.
 *   rows >= 0; 1 <= topk <= min(vocab, KVC_MAX_TOPK_ENTROPY); row_stride >= vocab.
 *   H_out      device float32 [rows].
 */
int kvc_topk_entropy(const void* logits, int dtype, int64_t rows, int64_t vocab,
                     int64_t row_stride, int topk, float* H_out, void* stream);

/*
 * Layer-wise representation distance ([InfoKV] Method, Technical detail):
 * D[l, i] = 1 - cos(h_l[i, :], h_final[i, :]) + tau, with cos := 0 when either
 * vector has zero norm.
 *   h_layers   host array of L device pointers, each [n, hidden] of dtype.
 *   h_final    device [n, hidden] of dtype (the last layer's hidden state).
 *   D_out      device float32 [L, n].
 *   1 <= L <= KVC_MAX_LAYERS, n >= 0, hidden >= 1.
 */
int kvc_repr_distance(const void* const* h_layers, const void* h_final, int dtype,
                      int L, int64_t n, int64_t hidden, float tau, float* D_out,
                      void* stream);

/*
 * Observation-window attention ([InfoKV] Method, Technical detail; the
 * attention factor of VATP in [SelKV] section 2, pipeline step 1).
 * For layer l, query head h of KV group g = h / (Hq/Hkv), window row r at
 * position p_r = n - w + r:
 *   P[h, r, j] = softmax over j <= p_r of scale * <q[l][h, r, :], k[l][g, j, :]>
 *   per_query_head = 1:  A[l, h, j] = (1/w) sum_r P[h, r, j]          [L, Hq, n]
 *   per_query_head = 0:  A[l, g, j] = mean over the group's heads      [L, Hkv, n]
 *   per_query_head = 2:  A_out[0, l, g, j] = the group mean (as 0) and
 *                        A_out[1, l, g, j] = max over the group's heads of
 *                        A[l, h, j] (as 1)                          [2, L, Hkv, n]
 *                        (what SelKV's VATP union and merge need, without
 *                        the per-head rows; bf16 needs w <= 32, Hq/Hkv <= 4)
 *   q_win      host array of L device pointers, each [Hq, w, d] of dtype.
 *   k          host array of L device pointers, each [Hkv, n, d] of dtype.
 *   A_out      device float32, shape above.  Every row of A sums to 1.
 *   scale: finite and > 0 (1/sqrt(d) in the pages' attention).
 *   1 <= w <= n; Hq % Hkv == 0; bf16 needs d in {64, 128} and
 *   (Hq/Hkv) * ceil(w/32) <= 8; float32 needs d <= 256.
 *   ws         device workspace, kvc_score_window_attn_workspace_size() bytes;
 *              calls that share one workspace must not overlap.
 * Two bf16 kernels: when one (layer, KV head)'s keys fit the registers of one
 * XCD (w <= 32, (Hq/Hkv) <= 4, n <= 32768 at d = 128 or 65536 at d = 64) they
 * are read once, by a cooperative launch that holds every CU while it runs;
 * otherwise, under stream capture, or when the device cannot hold that grid
 * (or the workspace is smaller than the size above), two passes read them
 * twice.  If the cooperative grid were ever not resident at once, its team
 * barriers give up after about a second and write NaN for the affected units.
 */
size_t kvc_score_window_attn_workspace_size(int L, int Hq, int Hkv, int64_t n,
                                            int w, int d, int dtype);
int kvc_score_window_attn(const void* const* q_win, const void* const* k, int dtype,
                          int L, int Hq, int Hkv, int64_t n, int w, int d,
                          float scale, int per_query_head, float* A_out,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * kvc_score_window_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation and kernels, with the workspace taken from
 * a fixed device scratch array of kvc_score_window_attn_noalloc_max_workspace()
 * bytes (32 MiB) that each GPU the library runs on holds until the process
 * ends.  Nothing is allocated or freed.  A shape whose
 * kvc_score_window_attn_workspace_size() exceeds the scratch returns
 * KVC_ERR_WORKSPACE before anything is enqueued (the Llama-shaped workloads
 * need 1.4 MB at 16K tokens and 13.1 MB at 102400).  Every call on one GPU
 * shares that GPU's scratch: calls that overlap on one GPU (other streams or
 * threads) race and must be ordered by the caller.  Arguments otherwise as
 * kvc_score_window_attn.
 */
size_t kvc_score_window_attn_noalloc_max_workspace(void);
int kvc_score_window_attn_noalloc(const void* const* q_win, const void* const* k, int dtype,
                                  int L, int Hq, int Hkv, int64_t n, int w, int d,
                                  float scale, int per_query_head, float* A_out, void* stream);

/*
 * Importance fusion ([InfoKV] Contributions, Method, Technical detail):
 *   E[l, i] = D[l, i] * H[i];  sigma[l, :] = softmax over the n tokens of E[l, :]
 *   S[l, g, i] = alpha_fuse * A[l, g, i] + (1 - alpha_fuse) * sigma[l, i]
 *   Ebar[l] = (1/n) sum_i E[l, i]      (the adaptive budget's layer share)
 *   A          device float32 [L, Hkv, n];  D device float32 [L, n];
 *   H          device float32 [n].
 *   S_out      device float32 [L, Hkv, n].
 *   Ebar_out   device float32 [L], or NULL.
 *   n >= 1; 0 <= alpha_fuse <= 1.
 */
size_t kvc_fuse_scores_workspace_size(int L, int64_t n);
int kvc_fuse_scores(const float* A, const float* D, const float* H, int L, int Hkv,
                    int64_t n, float alpha_fuse, float* S_out, float* Ebar_out,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * Importance fusion over cache slots, for compression repeated during decoding
 * ([InfoKV] Technical detail: compression is applied at prefill and again during
 * decoding, e.g. every 1024 generated tokens; Method: the fusion formula).
 * After a compaction each KV head holds its own token set, so the entropy score
 * is a row per (layer, KV head): slot j of head g carries E = D * H of the token
 * it holds (kept slots keep the value they had; new tokens get it from
 * kvc_append_entropy_scores).  Per (l, g):
 *   S_out[l, g, j] = alpha_fuse * A[l, g, j] + (1 - alpha_fuse) * softmax_j(E[l, g, :])
 *   Ebar_out[l]    = mean of E[l, :, :] over heads and slots
 * With equal rows across heads this is kvc_fuse_scores' result.
 *   A, E       device float32 [L, Hkv, n];  S_out device float32 [L, Hkv, n].
 *   Ebar_out   device float32 [L], or NULL.
 *   n >= 1; L * Hkv <= 65535; 0 <= alpha_fuse <= 1.
 */
size_t kvc_fuse_scores_slots_workspace_size(int L, int Hkv, int64_t n);
int kvc_fuse_scores_slots(const float* A, const float* E, int L, int Hkv, int64_t n,
                          float alpha_fuse, float* S_out, float* Ebar_out, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * Entropy scores of newly generated tokens appended to the slot rows
 * ([InfoKV] Method: E = D * H; Technical detail: compression during decoding):
 *   E[l, g, offset + i] = D[l, i] * H[i]   for every KV head g and i < t
 * so the old slots' scores are reused and only the new tokens' H and D are
 * computed (kvc_topk_entropy and kvc_repr_distance over their rows).
 *   D          device float32 [L, t];  H device float32 [t].
 *   E          device float32 [L, Hkv, cap]; slots [offset, offset + t) written.
 *   t >= 1; 0 <= offset; offset + t <= cap; L * Hkv <= 65535.
 */
int kvc_append_entropy_scores(const float* D, const float* H, int L, int Hkv, int64_t t,
                              float* E, int64_t cap, int64_t offset, void* stream);

/*
 * Uniform layer budget ([InfoKV] Contributions, Technical detail; host only):
 * k = floor(keep_fraction * n), clamped to [w, n].  Writes *k_out.
 */
int kvc_uniform_budget(double keep_fraction, int64_t n, int w, int64_t* k_out);

/*
 * Adaptive layer budget ([InfoKV] Method; Glossary, adaptive budget allocation;
 * host only, synchronous):  x_l = Ebar[l] / sum_m Ebar[m] * B (in double),
 * k_l = floor(x_l); the B - sum k_l leftover tokens go one each to the lowest
 * layer indices; each k_l is then clamped to [w, n].
 *   Ebar       host float32 [L], all > 0 (copy kvc_fuse_scores' Ebar_out back).
 *   k_out      host int64 [L].
 */
int kvc_adaptive_budget(const float* Ebar, int L, int64_t B, int w, int64_t n,
                        int64_t* k_out);

/*
 * Per-(layer, KV head) retention ([InfoKV] Method, Technical detail; [SelKV]
 * section 2, pipeline step 2 when S is the VATP union):
 * keep the last w tokens plus the k_l - w tokens of [0, n - w) with the largest
 * S (float32 compare, ties to the lower index); if k_l <= w keep the last k_l.
 * Indices are written in ascending order.  Exact and deterministic.  Scores
 * are compared as float32 values (-0 equals +0, +-inf allowed); NaN scores are
 * not supported (their rank is that of their bit pattern and not specified).
 *   S          device float32 [L, Hkv, n].
 *   k_keep     host int64 [L], each in [1, n].
 *   idx_out    host array of L device pointers, each int32 [Hkv, k_keep[l]].
 *   0 <= w <= n.
 */
int kvc_select_topk(const float* S, int L, int Hkv, int64_t n, const int64_t* k_keep,
                    int w, int32_t* const* idx_out, void* stream);

/*
 * Order-preserving gather of the kept rows ([InfoKV] Method: the top tokens are
 * retained): K_out[l][g, j, :] = K[l][g, idx[l][g, j], :], same for V.
 * Bit-exact copy.
 *   K, V       host arrays of L device pointers, each [Hkv, n, d] of dtype.
 *   idx        host array of L device pointers, each int32 [Hkv, k_keep[l]],
 *              every entry in [0, n).  An entry outside it is clamped to n - 1
 *              on the device: a wrong row is copied, nothing is read out of
 *              bounds, and no error is reported.
 *   k_keep     host int64 [L].
 *   K_out, V_out  host arrays of L device pointers, each [Hkv, k_keep[l], d].
 *   V and V_out may both be NULL (keys only).
 */
int kvc_compact(const void* const* K, const void* const* V, int dtype, int L, int Hkv,
                int64_t n, int d, const int32_t* const* idx, const int64_t* k_keep,
                void* const* K_out, void* const* V_out, void* stream);

/*
 * kvc_compact with a fixed output head stride, for a cache that keeps growing
 * after the compaction ([InfoKV] Technical detail: compression during decoding):
 *   K_out[l][g * out_rows + j, :] = K[l][g, idx[l][g, j], :], same for V,
 * so each head's kept rows fill the front of an [Hkv, out_rows, d] buffer and
 * rows [k_keep[l], out_rows) stay free for the tokens decoded next.  With d = 1
 * and float32 it gathers per-slot scores (kvc_fuse_scores_slots' E rows).
 *   Arguments as kvc_compact; out_rows >= every k_keep[l].  The outputs must not
 *   overlap the inputs.
 */
int kvc_compact_into(const void* const* K, const void* const* V, int dtype, int L, int Hkv,
                     int64_t n, int d, const int32_t* const* idx, const int64_t* k_keep,
                     int64_t out_rows, void* const* K_out, void* const* V_out, void* stream);

/*
 * VATP importance and its GQA union ([SelKV] section 2, pipeline steps 1-2):
 *   VATP[l, h, j] = A_hq[l, h, j] * ||v[l][g(h), j, :]||_2
 *   U_out[l, g, j]  = max over the group's heads of VATP
 *   Ag_out[l, g, j] = mean over the group's heads of A_hq (the group's prefill
 *                     attention used for routing and merge weights)
 *   A_hq       device float32 [L, Hq, n] (kvc_score_window_attn, per_query_head=1).
 *   V          host array of L device pointers, each [Hkv, n, d] of dtype,
 *              16-byte aligned; d * element size in {64, 128, 256, 512} bytes.
 *   U_out, Ag_out  device float32 [L, Hkv, n].
 */
int kvc_vatp_union(const float* A_hq, const void* const* V, int dtype, int L, int Hq,
                   int Hkv, int64_t n, int d, float* U_out, float* Ag_out, void* stream);

/*
 * The VATP union from the group max of the attention ([SelKV] section 2,
 * pipeline steps 1-2): U_out[l, g, j] = A_gmax[l, g, j] * ||v[l][g, j, :]||_2,
 * equal to kvc_vatp_union's U (max_h (A_h * ||v||) = (max_h A_h) * ||v|| for
 * ||v|| >= 0, and a rounded product is monotone in each factor).
 *   A_gmax     device float32 [L, Hkv, n]: plane 1 of kvc_score_window_attn
 *              with per_query_head = 2 (its plane 0 is A_g).
 *   V          as kvc_vatp_union.   U_out  device float32 [L, Hkv, n].
 */
int kvc_vatp_union_gmax(const float* A_gmax, const void* const* V, int dtype, int L,
                        int Hkv, int64_t n, int d, float* U_out, void* stream);

/*
 * Selective gated merge with attention compensation ([SelKV] section 2: soft
 * cosine gate, attention compensation, pipeline steps 3-5), fused with the
 * order-preserving gather.  For each layer l and KV head g, with kept indices
 * idx (ascending, from kvc_select_topk on U) and A = Ag[l, g, :]:
 *   - an evicted token e goes to t(e) = the kept token of its bucket
 *     [floor(e/bucket)*bucket, +bucket) with the largest A (ties: lower index);
 *     it is dropped if the bucket holds no kept token;
 *   - gate g_e = max(cos(v_e, v_t), 0)  (cos := 0 for a zero vector);
 *   - v'_t = (A_t v_t + sum_e g_e A_e v_e) / (A_t + sum_e g_e A_e);
 *     R_t = (A_t + sum_e g_e A_e) / A_t;  logR_out = ln R_t (0 if nothing merged);
 *   - K_out = K at the kept rows (keys are not merged), V_out = v' rounded to
 *     dtype (round to nearest even for bf16).
 *   K, V       host arrays of L device pointers, each [Hkv, n, d] of dtype.
 *   Ag         device float32 [L, Hkv, n].
 *   idx        host array of L device pointers, each int32 [Hkv, m_keep[l]],
 *              ascending, every entry in [0, n).
 *   m_keep     host int64 [L], each in [1, n];  bucket >= 1;
 *              d * element size in {64, 128, 256, 512} bytes; K, V, K_out,
 *              V_out 16-byte aligned.
 *   K_out, V_out  host arrays of L device pointers, each [Hkv, m_keep[l], d].
 *   logR_out   host array of L device pointers, each float32 [Hkv, m_keep[l]].
 */
int kvc_merge_gated(const void* const* K, const void* const* V, int dtype,
                    const float* Ag, int L, int Hkv, int64_t n, int d,
                    const int32_t* const* idx, const int64_t* m_keep, int bucket,
                    void* const* K_out, void* const* V_out, float* const* logR_out,
                    void* stream);

/*
 * RoPE re-positioning of the kept keys ([SelKV] section 2, pipeline overview,
 * step 6; the page turns it off for long contexts): key row j of each head,
 * carrying the rotary embedding of position pos_old[l][g, j], is re-embedded at
 * position new_pos0 + j, in place.  Element i pairs with element i + d/2 and
 * turns by (new_pos0 + j - pos_old[l][g, j]) * base^(-2i/d) radians (the page
 * gives neither the pairing nor the base).  The angle is reduced in float64;
 * bf16 results are rounded to nearest even.
 *   K          host array of L device pointers, each [Hkv, m, d] of dtype.
 *   pos_old    host array of L device pointers, each int32 [Hkv, m] (for a
 *              compacted cache: the kept indices).
 *   d even; base > 1; 0 <= new_pos0 < 2^31.
 */
int kvc_rope_reposition(void* const* K, int dtype, const int32_t* const* pos_old,
                        int64_t new_pos0, double base, int L, int Hkv, int64_t m, int d,
                        void* stream);

/*
 * Decode attention of one query per head over a (compacted) cache, with the
 * optional compensation bias ([SelKV] section 2, attention compensation; used
 * with [RECAS] section 2.B's bound as a check):
 *   logit[h, t] = scale * <q[l][h, :], K[l][g(h), t, :]> + alpha_bias * logR[l][g(h), t]
 *   o_out[l, h, :] = sum_t softmax(logit[h, :])_t * V[l][g(h), t, :]
 *   lse_out[l, h]  = ln sum_t exp(logit[h, t])   (may be NULL)
 *   q          host array of L device pointers, each [Hq, d] of dtype.
 *   K, V       host arrays of L device pointers, each [Hkv, len, d] of dtype.
 *   logR       host array of L device pointers, each float32 [Hkv, len], or NULL.
 *   o_out      device float32 [L, Hq, d];  lse_out device float32 [L, Hq].
 *   len >= 1; d <= 256; scale and alpha_bias finite.
 */
size_t kvc_decode_attn_workspace_size(int L, int Hq, int64_t len, int d);
int kvc_decode_attn(const void* const* q, const void* const* K, const void* const* V,
                    int dtype, const float* const* logR, float alpha_bias, int L,
                    int Hq, int Hkv, int64_t len, int d, float scale, float* o_out,
                    float* lse_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Dropped-attention-mass monitor of a compacted cache ([RECAS] section 2.B,
 * error-bounded compression: the formal bound ||o - o'||_2 <= 2 V_max delta,
 * checked exactly at a full-attention probe step).  With lse_full and lse_kept
 * the log normalisers of one decode query per head over the full cache and over
 * the kept rows only (two kvc_decode_attn calls without a bias):
 *   delta_out[l, h] = max(0, 1 - exp(lse_kept[l, h] - lse_full[l, h]))
 *                     (the evicted tokens' share of the full softmax)
 *   vmax_out[l, g]  = max over j of ||V[l][g, j, :]||_2 over the full cache
 *   bound_out[l, h] = 2 * vmax_out[l, g(h)] * delta_out[l, h]
 * With a merged, bias-compensated cache (SelKV) lse_kept is not the kept share
 * and delta is not the dropped mass.
 *   lse_kept, lse_full  device float32 [L, Hq].
 *   V          host array of L device pointers, each [Hkv, n, d] of dtype (the
 *              full cache).
 *   delta_out, bound_out  device float32 [L, Hq];  vmax_out device float32 [L, Hkv].
 *   n >= 1; 1 <= d <= 4096; Hq % Hkv == 0.
 */
int kvc_dropped_mass(const float* lse_kept, const float* lse_full, const void* const* V,
                     int dtype, int L, int Hq, int Hkv, int64_t n, int d, float* delta_out,
                     float* vmax_out, float* bound_out, void* stream);

/*
 * Active-set scores of one decode step ([RECAS] section 2.C, dynamic sparse
 * decoding attention: a query-aware sparse score over the retained cache, whose
 * top K_t entries form the active set attended this step):
 *   score_out[l, g, j] = max over the query heads h of group g of
 *                        scale * <q[l][h, :], K[l][g, j, :]>  +  beta * utility[l][g, j]
 * The page adds a utility score to the query-key compatibility without fixing
 * its inputs, so the utility row is the caller's (NULL: compatibility only).
 * The active set is kvc_select_topk(score_out, K_t, w = 0).
 *   q          host array of L device pointers, each [Hq, d] of dtype.
 *   K          host array of L device pointers, each [Hkv, len, d] of dtype.
 *   utility    host array of L device pointers, each float32 [Hkv, len], or NULL.
 *   score_out  device float32 [L, Hkv, len].
 *   Hq / Hkv <= 8; L * Hkv <= 65535; d <= 256; scale finite and > 0; beta finite.
 */
int kvc_active_scores(const void* const* q, const void* const* K, int dtype,
                      const float* const* utility, float beta, int L, int Hq, int Hkv,
                      int64_t len, int d, float scale, float* score_out, void* stream);

/*
 * Decode attention over an active set ([RECAS] section 2.C: only the active
 * entries take part in this step's attention; the others stay in the cache):
 * kvc_decode_attn with the softmax and the output taken over the rows
 * active[l][g, 0 .. k_active) of each KV head's cache (any order; a row listed
 * twice counts twice).  With every row listed it is kvc_decode_attn.
 *   active     host array of L device pointers, each int32 [Hkv, k_active],
 *              every entry in [0, len).  An entry outside it is clamped to
 *              len - 1 on the device: a wrong row takes part, nothing is read
 *              out of bounds, and no error is reported.
 *   1 <= k_active <= len; other arguments, the workspace size
 *   (kvc_decode_attn_workspace_size(L, Hq, len, d)) and errors as kvc_decode_attn.
 */
int kvc_decode_attn_active(const void* const* q, const void* const* K, const void* const* V,
                           int dtype, const float* const* logR, float alpha_bias,
                           const int32_t* const* active, int64_t k_active, int L, int Hq,
                           int Hkv, int64_t len, int d, float scale, float* o_out,
                           float* lse_out, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif  /* KVC_H_ */
