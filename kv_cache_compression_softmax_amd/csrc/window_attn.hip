// Observation-window attention A (group mean, or per query head).
//
// [InfoKV] Method and Technical detail: the attention each cached token receives
// from the queries of the last w positions of layer l, averaged over the window
// (and, for GQA, over the query heads sharing the KV head).  [SelKV] section 2,
// pipeline step 1 uses the per-head form for its VATP score.
//
// Layout: q_win[l] is [Hq, w, d], k[l] is [Hkv, n, d].  For KV head g the window
// queries of its G heads form the rows of an M x d matrix; each head's w rows are
// padded to a multiple of 32 so that every 32-row "tile" belongs to one head.
//
// A needs each row's softmax normaliser before any column can be summed, so the
// bf16 path makes two passes over K:
//   pass 1  per 32-key block, S^T = K * Q^T on MFMA (keys on M, queries on N);
//           each lane keeps a (reference, sum of exp2) pair for one query row:
//           the wave's first block sets the reference to the row's maximum there,
//           later blocks only add exp2(s - reference) (no running maximum; a sum
//           that overflows sends the wave back over its keys with one).  The
//           four waves of a workgroup merge in LDS and write one partial;
//           Each pass-2 workgroup merges its (layer, KV head)'s partials in index
//           order into c_r = max + log2(sum), +inf for padding rows;
//   pass 2  S = Q * K^T on MFMA (queries on M, keys on N): each lane owns one key
//           column, so exp2(s - c_r) summed over the lane's 16 rows plus its
//           partner lane is the column sum, with no atomics.
// Launch i runs pass 2 of layer chunk i-1 next to pass 1 of chunk i, so a chunk's
// keys are read again one chunk later, while they are still in the 256 MB MALL.
// Key rows go straight from HBM into MFMA operand registers in the instruction's
// own k layout: step s, lane (row i, half hf) holds elements 16s + 8hf .. +8, so
// the two halves of a wave read adjacent 16-byte pieces of each row and a load
// instruction touches 32 cache lines, not 64 (measured 5.9 vs 4.6 TB/s for a
// plain K stream).  Q is staged once per workgroup in LDS in fragment order, one
// ds_read_b128 per fragment.
#include <cmath>
#include <mutex>
#include <type_traits>

#include "common.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int NTW = 256;        // threads per workgroup (4 waves)
constexpr int MAX_TILES = 8;    // G * ceil(w/32)
constexpr int MAX_TG = 4;       // tiles per launch
constexpr int KPW = 512;        // keys per wave (twice that from kLongRow keys on)
// 1024 keys per wave halve the per-task costs (Q staging, pass-2 partial merge):
// 2.85 -> 2.74 ms at 102400 tokens, but 1.71 -> 1.83 ms at 65536 (8B shape)
constexpr int64_t kLongRow = 98304;
constexpr int64_t kMallBytes = 256ll << 20;  // MI355X last-level cache (MALL)
constexpr int kLargeChunk = 16;  // layers per chunk when a layer's keys exceed half the MALL
constexpr float LOG2E = 1.4426950408889634f;

struct Geo {
  int Hq, Hkv, G, w, d, tph, ntiles;   // tiles per head, tiles per KV group
  int64_t n;
  int nwg;                             // workgroups per (layer, KV head)
  int kpw;                             // keys per wave
};

struct Span { int l0, nl, pass; };     // layers [l0, l0 + nl) of the table, pass 1 or 2

struct WinArgs {
  ConstPtrs q, k;                      // per-layer pointers of the current layer group
  Geo g;
  int tile0;                           // first query tile of this launch
  float sl2;                           // scale * log2(e)
  int per_head;
  float2* part;                        // [32, Hkv, nwg, rows] pass-1 partials
  float* A;                            // output of the layer group
  int nspan;
  Span span[2];
  int64_t blocks0;                     // tasks of span 0
  int64_t ntask;                       // tasks of all spans
};

// x of this lane plus x of lane ^ 32, the same value in both lanes (one
// v_permlane32_swap: lane i < 32 receives (own, partner), lane i + 32 (partner,
// own), so the sum of the pair is the same in both halves)
__device__ __forceinline__ float add_halves(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  bf16x8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

// Streams the 32-key blocks jb, jb + 32, ... (nb of them) of one KV head through
// two register sets used in turn: block b + 1 is in flight while `block` runs on
// block b.  Rows past the end of K are clamped to the last key (the callers mask
// every key >= n), so every prefetch is unconditional; loads issued on only some
// paths, or re-issued by the compiler at their use (the data are read-only: the
// memory clobber pins them), would make every block wait for its own keys.
// `prologue` (the task's Q staging and workgroup barriers, run by every wave) is
// called after the first two blocks are requested, so their latency overlaps it.
template <int D, typename P, typename F>
__device__ __forceinline__ void stream_blocks(const uint16_t* kh, int64_t n, int64_t jb, int nb,
                                              int lane, P&& prologue, F&& block) {
  constexpr int S = D / 16;
  if (nb <= 0) { prologue(); return; }
  const int i = lane & 31, hf = lane >> 5;
  auto load = [&](int b, bf16x8 (&kf)[S]) __attribute__((always_inline)) {
    const int64_t key = min(jb + 32 * b + i, n - 1);
    const uint16_t* p = kh + key * D + 8 * hf;
#pragma unroll
    for (int st = 0; st < S; ++st) kf[st] = *reinterpret_cast<const bf16x8*>(p + 16 * st);
    asm volatile("" ::: "memory");
  };
  bf16x8 k0[S], k1[S];
  load(0, k0);
  load(min(1, nb - 1), k1);
  prologue();
  int b = 0;
#pragma unroll 1
  for (; b + 1 < nb; b += 2) {
    block(k0, jb + 32 * b);
    __builtin_amdgcn_sched_barrier(0);
    load(min(b + 2, nb - 1), k0);
    block(k1, jb + 32 * (b + 1));
    __builtin_amdgcn_sched_barrier(0);
    load(min(b + 3, nb - 1), k1);
  }
  if (b < nb) block(k0, jb + 32 * b);
}

// Q rows of TG tiles into LDS in fragment order: entry (t, s, lane) holds the 16
// bytes lane `lane` feeds to step s of tile t.  Global reads are row-contiguous.
template <int D, int TG>
__device__ __forceinline__ void stage_q(const uint16_t* q, const Geo& g, int kvh, int tile0, uint4* qlds) {
  constexpr int S = D / 16, C = D / 8;          // steps, 16-byte chunks per row
  for (int f = threadIdx.x; f < TG * 32 * C; f += NTW) {
    const int c16 = f % C, i = (f / C) % 32, t = f / (32 * C);
    const int hf = c16 & 1, st = c16 >> 1;
    const int tile = tile0 + t;
    const int head = kvh * g.G + tile / g.tph;
    const int rr = (tile % g.tph) * 32 + i;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (rr < g.w) v = *reinterpret_cast<const uint4*>(q + ((int64_t)head * g.w + rr) * D + c16 * 8);
    qlds[(t * S + st) * 64 + hf * 32 + i] = v;
  }
}

// The TG tiles of one 32-key block.  Tile t+1's Q fragment reads and MFMA chain
// are issued inside tile t's exp2 epilogue (one scheduling region per tile), so a
// single wave keeps the matrix cores and the vector ALU busy together instead of
// alternating between them.  KEYS_ON_M puts the keys on the M side (pass 1: S^T),
// else the queries (pass 2: S).  epi(t, acc) is straight-line code.
template <int S, int TG, bool KEYS_ON_M, typename Epi>
__device__ __forceinline__ void pipelined_tiles(const bf16x8 (&kc)[S], const uint4* qlds, int qo,
                                                Epi&& epi) {
  constexpr int NV = (72 + S - 1) / S;           // epilogue VALU per MFMA slot
  constexpr int PRE = S < 4 ? S : 4;             // Q reads issued before the first MFMA
  auto chain = [&](int t, f32x16& acc) __attribute__((always_inline)) {
    bf16x8 q[S];
#pragma unroll
    for (int st = 0; st < S; ++st) q[st] = as_bf16x8(qlds[(t * S + st) * 64 + qo]);
    acc = f32x16{};
#pragma unroll
    for (int st = 0; st < S; ++st)
      acc = KEYS_ON_M ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc[st], q[st], acc, 0, 0, 0)
                      : __builtin_amdgcn_mfma_f32_32x32x16_bf16(q[st], kc[st], acc, 0, 0, 0);
  };
  f32x16 acc[2];
  chain(0, acc[0]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    if (t + 1 < TG) chain(t + 1, acc[(t + 1) & 1]);
    epi(t, acc[t & 1]);
    if (t + 1 < TG) {
      __builtin_amdgcn_sched_group_barrier(0x100, PRE, 0);      // Q reads
      __builtin_amdgcn_sched_group_barrier(0x402, NV, 0);       // VALU / transcendental
#pragma unroll
      for (int i = 0; i < S; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // one MFMA
        if (i + PRE < S) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, NV, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D, int TG>
struct WinSmem {
  uint4 q[TG * (D / 16) * 64];
  union {
    float2 wst[NTW / 64][TG * 32];                 // pass 1: per-wave row stats
    struct {
      __attribute__((aligned(16))) float c[TG * 32]; // pass 2: row normalisers
      float2 red[NTW];                             // pass 2: partial merges
    };
  };
};

// ---------------------------------------------------------------- pass 1
template <int D, int TG>
__device__ __forceinline__ void pass1(const WinArgs& a, WinSmem<D, TG>& sm, int l, int kvh, int wgi) {
  constexpr int S = D / 16;
  const Geo& g = a.g;
  const int lane = threadIdx.x & 63, hf = lane >> 5, qi = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int64_t lg = (int64_t)l * g.Hkv + kvh;
  const uint16_t* kh = (const uint16_t*)a.k.p[l] + (int64_t)kvh * g.n * D;   // this KV head's keys
  auto prologue = [&]() __attribute__((always_inline)) {
    stage_q<D, TG>((const uint16_t*)a.q.p[l], g, kvh, a.tile0, sm.q);
    __syncthreads();
  };

  int pos[TG];                                   // window position of this lane's row
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    const int rr = ((a.tile0 + t) % g.tph) * 32 + qi;
    pos[t] = rr < g.w ? (int)(g.n - g.w) + rr : -1;
  }
  float m[TG], sm_[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) { m[t] = -INFINITY; sm_[t] = 0.f; }

  const int64_t jb = ((int64_t)wgi * (NTW / 64) + wv) * g.kpw;
  const int64_t je = min(g.n, jb + g.kpw);
  const int nb = (int)((je - jb + 31) / 32);     // <= 0 past the end of K
  const int64_t safe_end = g.n - g.w;            // keys <= this are seen by every row
  // one 32-key block; kc holds its key fragments
  // FULL: every key of the block is visible to every row (no mask code at all)
  // FIXED: the lane's rows keep the reference m set by the wave's first block and
  // add exp2(s - m) with no running maximum.  The partial (m, sum) is then a valid
  // normaliser pair for any m; a term above 2^128 would make the sum infinite,
  // which the check after the stream catches (the wave then redoes its keys with
  // the running maximum).
  auto block_t = [&](const bf16x8 (&kc)[S], int64_t j0, auto full_t, auto fixed_t) __attribute__((always_inline)) {
    constexpr bool full = decltype(full_t)::value;
    constexpr bool fixed = decltype(fixed_t)::value;
    int qo = lane;
    asm volatile("" : "+v"(qo));                 // keep the Q reads in the loop (LDS, not VGPRs)
    // scores in log2 units are acc * sl2 (sl2 > 0): take the block max on the raw
    // accumulator, then one FMA and one v_exp_f32 per element (results below
    // 2^-126 flush to zero, which changes no sum at float32 precision)
    auto epi = [&](int t, f32x16 acc) __attribute__((always_inline)) {
      if constexpr (fixed) {
        float sum = __builtin_amdgcn_exp2f(fmaf(acc[0], a.sl2, -m[t]));
#pragma unroll
        for (int v = 1; v < 16; ++v) sum += __builtin_amdgcn_exp2f(fmaf(acc[v], a.sl2, -m[t]));
        sm_[t] += sum;
        return;
      }
      float bm = -INFINITY;
      if constexpr (full) {
#pragma unroll
        for (int v = 0; v < 16; ++v) bm = fmaxf(bm, acc[v]);
      } else {
        // key offset limit within the block; blocks start below n and pos < n
        const int lim = (int)(min((int64_t)pos[t], g.n - 1) - j0) - 4 * hf;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int off = 8 * (v >> 2) + (v & 3);
          acc[v] = (off <= lim) ? acc[v] : -INFINITY;
          bm = fmaxf(bm, acc[v]);
        }
      }
      // no branch: a row that has seen no key yet keeps m = -inf and uses 0 as
      // the exponent offset (every term is then exp2(-inf) = 0)
      const float mn = fmaxf(m[t], bm * a.sl2);
      const float ms = full ? mn : (mn > -INFINITY ? mn : 0.f);
      float sum = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) sum += __builtin_amdgcn_exp2f(fmaf(acc[v], a.sl2, -ms));
      sm_[t] = sm_[t] * __builtin_amdgcn_exp2f(m[t] - ms) + sum;
      m[t] = mn;
    };
    pipelined_tiles<S, TG, true>(kc, sm.q, qo, epi);
  };
  // full blocks after the wave's first take the fixed reference; the first block
  // (where m is set) and the masked blocks at the end of K keep the running maximum
  auto block = [&](const bf16x8 (&kc)[S], int64_t j0) {
    if (j0 + 31 <= safe_end) {                   // wave-uniform branches
      if (j0 != jb) block_t(kc, j0, std::true_type{}, std::true_type{});
      else block_t(kc, j0, std::true_type{}, std::false_type{});
    } else {
      block_t(kc, j0, std::false_type{}, std::false_type{});
    }
  };
  auto careful = [&](const bf16x8 (&kc)[S], int64_t j0) {
    if (j0 + 31 <= safe_end) block_t(kc, j0, std::true_type{}, std::false_type{});
    else block_t(kc, j0, std::false_type{}, std::false_type{});
  };
  stream_blocks<D>(kh, g.n, jb, nb, lane, prologue, block);
  bool bad = false;
#pragma unroll
  for (int t = 0; t < TG; ++t) bad = bad || !(sm_[t] <= 3.0e38f);   // inf or NaN
  if (__builtin_amdgcn_ballot_w64(bad) != 0) {   // wave-uniform; not seen on finite logits
#pragma unroll
    for (int t = 0; t < TG; ++t) { m[t] = -INFINITY; sm_[t] = 0.f; }
    stream_blocks<D>(kh, g.n, jb, nb, lane, []() {}, careful);
  }
  // halves (lanes i, i+32 share a query row), then the 4 waves, in fixed order
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    const float mo = __shfl_xor(m[t], 32, 64), so = __shfl_xor(sm_[t], 32, 64);
    const float M = fmaxf(m[t], mo);
    float Sx = 0.f;
    if (M > -INFINITY) Sx = sm_[t] * exp2f(m[t] - M) + so * exp2f(mo - M);
    if (hf == 0) sm.wst[wv][t * 32 + qi] = make_float2(M, Sx);
  }
  __syncthreads();
  const int rows = g.ntiles * 32;
  float2* pl = a.part + lg * (int64_t)g.nwg * rows;
  for (int r = threadIdx.x; r < TG * 32; r += NTW) {
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < NTW / 64; ++w2) M = fmaxf(M, sm.wst[w2][r].x);
    float Sx = 0.f;
    if (M > -INFINITY) {
#pragma unroll
      for (int w2 = 0; w2 < NTW / 64; ++w2)
        if (sm.wst[w2][r].x > -INFINITY) Sx += sm.wst[w2][r].y * exp2f(sm.wst[w2][r].x - M);
    }
    pl[(int64_t)wgi * rows + a.tile0 * 32 + r] = make_float2(M, Sx);
  }
}

// ---------------------------------------------------------------- pass 2
template <int D, int TG, bool PH>
__device__ __forceinline__ void pass2(const WinArgs& a, WinSmem<D, TG>& sm, int l, int kvh, int wgi) {
  constexpr int S = D / 16;
  const Geo& g = a.g;
  const int lane = threadIdx.x & 63, hf = lane >> 5, qi = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int64_t lg = (int64_t)l * g.Hkv + kvh;
  const uint16_t* kh = (const uint16_t*)a.k.p[l] + (int64_t)kvh * g.n * D;   // this KV head's keys
  const int rows = g.ntiles * 32;
  // Q to LDS and the row normalisers from pass 1's workgroup partials: P threads
  // per row each merge every P-th partial (loads issued 8 at a time), then the P
  // results are merged in a fixed order; +inf for padding rows and rows that see
  // no key
  float cr[TG][16];                              // row normalisers (set by the prologue)
  auto prologue = [&]() __attribute__((always_inline)) {
    stage_q<D, TG>((const uint16_t*)a.q.p[l], g, kvh, a.tile0, sm.q);
    constexpr int R = TG * 32, P = NTW / R;
    const float2* pl = a.part + lg * (int64_t)g.nwg * rows + a.tile0 * 32;
    const int r = threadIdx.x % R, j = threadIdx.x / R;
    float M = -INFINITY, Sx = 0.f;
    if (j < P) {
      for (int bb = j; bb < g.nwg; bb += 8 * P) {
        float2 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = (bb + u * P < g.nwg) ? pl[(int64_t)(bb + u * P) * rows + r] : make_float2(-INFINITY, 0.f);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (v[u].x > -INFINITY) {
            const float mn = fmaxf(M, v[u].x);
            Sx = Sx * exp2f(M - mn) + v[u].y * exp2f(v[u].x - mn);
            M = mn;
          }
        }
      }
      sm.red[j * R + r] = make_float2(M, Sx);
    }
    __syncthreads();
    if (threadIdx.x < R) {
      float Mt = -INFINITY, St = 0.f;
      for (int jj = 0; jj < P; ++jj) {
        const float2 v = sm.red[jj * R + r];
        if (v.x > -INFINITY) {
          const float mn = fmaxf(Mt, v.x);
          St = St * exp2f(Mt - mn) + v.y * exp2f(v.x - mn);
          Mt = mn;
        }
      }
      const int row = a.tile0 * 32 + r;
      const bool pad = ((row >> 5) % g.tph) * 32 + (row & 31) >= g.w;
      sm.c[r] = (!pad && Mt > -INFINITY) ? Mt + log2f(St) : INFINITY;
    }
    __syncthreads();
    // this lane's 16 normalisers of each tile, held for the whole task (pass 2
    // would otherwise read them from LDS in every block, beside the Q fragments)
#pragma unroll
    for (int t = 0; t < TG; ++t)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const float4 c4 = reinterpret_cast<const float4*>(sm.c)[t * 8 + 2 * qd + hf];
        cr[t][4 * qd + 0] = c4.x; cr[t][4 * qd + 1] = c4.y;
        cr[t][4 * qd + 2] = c4.z; cr[t][4 * qd + 3] = c4.w;
      }
  };

  const int64_t jb = ((int64_t)wgi * (NTW / 64) + wv) * g.kpw;
  const int64_t je = min(g.n, jb + g.kpw);
  const int nb = (int)((je - jb + 31) / 32);
  const int64_t safe_end = g.n - g.w;
  const float inv_group = 1.0f / (float)(g.G * g.w), inv_w = 1.0f / (float)g.w;
  float* A = a.A;
  auto block_t = [&](const bf16x8 (&kc)[S], int64_t j0, auto full_t) __attribute__((always_inline)) {
    constexpr bool full = decltype(full_t)::value;
    const int64_t key = j0 + qi;                 // this lane's key column
    int qo = lane;
    asm volatile("" : "+v"(qo));                 // keep the Q reads in the loop (LDS, not VGPRs)
    // this lane's 16 rows of tile t: exp2(s - c_r) summed (the partner lane adds
    // the other 16 at the end of the block); the key is seen by rows rr with
    // key - (n - w) <= rr < w, and only if key < n
    float hs[TG];
    auto epi = [&](int t, const f32x16& acc) __attribute__((always_inline)) {
      const int base = ((a.tile0 + t) % g.tph) * 32 + 4 * hf;
      const int lo = (int)(key - safe_end) - base;
      const int hi = (key < g.n) ? g.w - base : -1;
      float colsum = 0.f;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int v = 4 * qd + u, off = 8 * qd + u;
          float e = __builtin_amdgcn_exp2f(fmaf(acc[v], a.sl2, -cr[t][v]));
          if constexpr (!full) e = (off >= lo && off < hi) ? e : 0.f;
          colsum += e;
        }
      }
      hs[t] = colsum;
    };
    pipelined_tiles<S, TG, false>(kc, sm.q, qo, epi);
    // pin the column sums here: otherwise the compiler sinks each tile's
    // epilogue into the per-head store branch below, after every MFMA
#pragma unroll
    for (int t = 0; t < TG; ++t) asm volatile("" : "+v"(hs[t]));
    float total = 0.f, hsum = 0.f;
    if constexpr (!PH) {                         // one cross-half add for the group
      float own = hs[0];
#pragma unroll
      for (int t = 1; t < TG; ++t) own += hs[t];
      total = add_halves(own);
    }
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      if constexpr (PH) {
        const float cs = add_halves(hs[t]);
        hsum += cs;
        const int tile = a.tile0 + t;
        const bool last_of_head = (t == TG - 1) || ((tile + 1) % g.tph == 0);
        if (last_of_head) {
          if (hf == 0 && key < g.n) {
            const int head = kvh * g.G + tile / g.tph;
            float* dst = A + ((int64_t)l * g.Hq + head) * g.n + key;
            const bool first_in_launch = (tile % g.tph) <= t;   // head started in this launch
            *dst = first_in_launch ? hsum * inv_w : *dst + hsum * inv_w;
          }
          hsum = 0.f;
        }
      }
    }
    if (!PH && hf == 0 && key < g.n) {
      float* dst = A + ((int64_t)l * g.Hkv + kvh) * g.n + key;
      *dst = a.tile0 == 0 ? total * inv_group : *dst + total * inv_group;
    }
  };
  auto block = [&](const bf16x8 (&kc)[S], int64_t j0) {
    if (j0 + 31 <= safe_end) block_t(kc, j0, std::true_type{});   // wave-uniform branch
    else block_t(kc, j0, std::false_type{});
  };
  stream_blocks<D>(kh, g.n, jb, nb, lane, prologue, block);
}

// PH: A per query head (else the group mean), fixed at compile time so that the
// pass-2 block stays one scheduling region
template <int D, int TG, bool PH>
__global__ void __launch_bounds__(NTW)
win_kernel(WinArgs a) {
  __shared__ WinSmem<D, TG> sm;
  // persistent grid: as many workgroups as fit at once, each looping over tasks, so
  // no launch ends with a sparsely occupied last round
  for (int64_t b = blockIdx.x; b < a.ntask; b += gridDim.x) {
    const int si = (a.nspan > 1 && b >= a.blocks0) ? 1 : 0;
    const Span sp = a.span[si];
    const int64_t local = si ? b - a.blocks0 : b;
    const int64_t lgl = local / a.g.nwg;         // (layer in span, KV head)
    const int wgi = (int)(local % a.g.nwg);
    const int l = sp.l0 + (int)(lgl / a.g.Hkv), kvh = (int)(lgl % a.g.Hkv);
    if (sp.pass == 1) pass1<D, TG>(a, sm, l, kvh, wgi);
    else pass2<D, TG, PH>(a, sm, l, kvh, wgi);
    __syncthreads();                             // LDS is reused by the next task
  }
}


// ---------------------------------------------------------------- float32 path
// Plain vector-ALU version for float32 inputs (small shapes).  Rows are indexed
// (head in group, window row) without padding.
constexpr int NTF = 256;

__global__ void __launch_bounds__(NTF)
win_f32_stats(ConstPtrs qs, ConstPtrs ks, Geo g, float scale_log2, float* __restrict__ c) {
  __shared__ float qsh[256];
  __shared__ float red[NTF / 64];
  const int R = g.G * g.w;
  const int64_t id = blockIdx.x;               // (l, kvh, row)
  const int r = (int)(id % R);
  const int kvh = (int)((id / R) % g.Hkv);
  const int l = (int)(id / ((int64_t)R * g.Hkv));
  const float* q = (const float*)qs.p[l] + ((int64_t)(kvh * g.G + r / g.w) * g.w + r % g.w) * g.d;
  const float* k = (const float*)ks.p[l] + (int64_t)kvh * g.n * g.d;
  for (int e = threadIdx.x; e < g.d; e += NTF) qsh[e] = q[e];
  __syncthreads();
  const int64_t p = g.n - g.w + r % g.w;
  float m = -INFINITY, s = 0.f;
  for (int64_t j = threadIdx.x; j <= p; j += NTF) {
    float dot = 0.f;
    for (int e = 0; e < g.d; ++e) dot += qsh[e] * k[j * g.d + e];
    const float x = dot * scale_log2;
    const float mn = fmaxf(m, x);
    s = s * exp2f(m - mn) + exp2f(x - mn);
    m = mn;
  }
  const float M = block_max<NTF>(m, red);
  const float S = block_sum<NTF>(m > -INFINITY ? s * exp2f(m - M) : 0.f, red);
  if (threadIdx.x == 0) c[id] = M + log2f(S);
}

// One thread per key: the key row is read once (into registers when d is one of
// the compiled sizes), then dotted with every window row of the group held in LDS.
// Blocks of NTA threads, so that short caches still spread over many CUs.
constexpr int NTA = 64;

template <int D>
__global__ void __launch_bounds__(NTA)
win_f32_accum(ConstPtrs qs, ConstPtrs ks, Geo g, float scale_log2, const float* __restrict__ c,
              int per_head, float* __restrict__ A) {
  extern __shared__ float qall[];              // [R, d]
  const int R = g.G * g.w;
  const int d = D > 0 ? D : g.d;
  const int64_t nblk = (g.n + NTA - 1) / NTA;
  const int64_t id = blockIdx.x;
  const int kvh = (int)((id / nblk) % g.Hkv);
  const int l = (int)(id / (nblk * g.Hkv));
  const int64_t j = (id % nblk) * NTA + threadIdx.x;
  const float* q = (const float*)qs.p[l] + (int64_t)kvh * g.G * g.w * d;
  for (int e = threadIdx.x; e < R * d; e += NTA) qall[e] = q[e];
  __syncthreads();
  if (j >= g.n) return;
  const float* kr = (const float*)ks.p[l] + ((int64_t)kvh * g.n + j) * d;
  const float* cr = c + ((int64_t)l * g.Hkv + kvh) * R;
  float kreg[D > 0 ? D : 1];
  if constexpr (D > 0) {
#pragma unroll
    for (int e = 0; e < D; ++e) kreg[e] = kr[e];
  }
  float total = 0.f;
  for (int h = 0; h < g.G; ++h) {
    float hs = 0.f;
    for (int rr = 0; rr < g.w; ++rr) {
      if (j > g.n - g.w + rr) continue;
      const float* qr = qall + (h * g.w + rr) * d;
      float dot = 0.f;
      if constexpr (D > 0) {
#pragma unroll
        for (int e = 0; e < D; ++e) dot += qr[e] * kreg[e];
      } else {
        for (int e = 0; e < d; ++e) dot += qr[e] * kr[e];
      }
      hs += exp2f(dot * scale_log2 - cr[h * g.w + rr]);
    }
    if (per_head) A[((int64_t)l * g.Hq + kvh * g.G + h) * g.n + j] = hs / (float)g.w;
    total += hs;
  }
  if (!per_head) A[((int64_t)l * g.Hkv + kvh) * g.n + j] = total / (float)(g.G * g.w);
}

// ---------------------------------------------------------------- host
struct Plan {
  Geo g;
  bool mfma;
  int lch;                      // layers per chunk
  size_t part_bytes, c_bytes;
};

void make_plan(int L, int Hq, int Hkv, int64_t n, int w, int d, int dtype, Plan* P) {
  Geo g{};
  g.Hq = Hq; g.Hkv = Hkv; g.G = Hq / Hkv; g.w = w; g.d = d; g.n = n;
  g.tph = (w + 31) / 32;
  g.ntiles = g.G * g.tph;
  g.kpw = n >= kLongRow ? 2 * KPW : KPW;
  g.nwg = (int)((n + 4LL * g.kpw - 1) / (4LL * g.kpw));
  P->g = g;
  P->mfma = (dtype == KVC_BF16);
  const int lg_max = L < kLayersPerLaunch ? L : kLayersPerLaunch;
  // Layers per chunk (a launch runs pass 2 of one chunk beside pass 1 of the
  // next).  While two layers' keys fit the MALL, a chunk holds about one MALL of
  // keys, so that pass 2 re-reads them from there (8B shape at 32K tokens: 4
  // layers, 1.00 ms against 1.06-1.09 with 3, 5, 6 or 8).  Larger layers cannot
  // be re-read from it at all, and fewer launches win (102400 tokens: 3.04 ms
  // with 8-32 layers per chunk against 3.20 with 2).
  const int64_t layer_k = (int64_t)Hkv * n * d * (dtype == KVC_BF16 ? 2 : 4);
  int64_t lch = 2 * layer_k <= kMallBytes ? (kMallBytes + layer_k / 2) / layer_k : kLargeChunk;
  lch = lch < 1 ? 1 : (lch > lg_max ? lg_max : lch);
  P->lch = (int)lch;
  if (P->mfma) {
    P->part_bytes = (size_t)lg_max * Hkv * g.nwg * g.ntiles * 32 * sizeof(float2);
    P->c_bytes = 0;
  } else {
    P->part_bytes = 0;
    P->c_bytes = (size_t)lg_max * Hkv * g.G * w * sizeof(float);
  }
}

// Workgroups of `kern` resident at once on the current device.
int resident_blocks(const void* kern) {
  int dev = 0, ncu = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, NTW, 0) != hipSuccess)
    return 1024;
  return (ncu > 0 ? ncu : 1) * (per_cu > 0 ? per_cu : 1);
}

template <int D, int TG, bool PH>
void launch_win_ph(WinArgs a, hipStream_t s) {
  const void* kern = reinterpret_cast<const void*>(&win_kernel<D, TG, PH>);
  const int64_t res = resident_blocks(kern);
  const dim3 grid((unsigned)(a.ntask < res ? a.ntask : res)), block(NTW);
  hipLaunchKernelGGL((win_kernel<D, TG, PH>), grid, block, 0, s, a);
}

template <int D, int TG>
void launch_win_tg(WinArgs a, hipStream_t s) {
  if (a.per_head) launch_win_ph<D, TG, true>(a, s);
  else launch_win_ph<D, TG, false>(a, s);
}

template <int D>
void launch_win(int tg, WinArgs a, hipStream_t s) {
  a.ntask = 0;
  for (int i = 0; i < a.nspan; ++i) a.ntask += (int64_t)a.span[i].nl * a.g.Hkv * a.g.nwg;
  switch (tg) {
    case 1: launch_win_tg<D, 1>(a, s); break;
    case 2: launch_win_tg<D, 2>(a, s); break;
    case 3: launch_win_tg<D, 3>(a, s); break;
    default: launch_win_tg<D, 4>(a, s); break;
  }
}

// One launch: up to two spans (pass 2 of one chunk, pass 1 of the next).
void launch_spans(const WinArgs& base, int tile0, int tg, int nspan, const Span* sp, hipStream_t s) {
  WinArgs a = base;
  a.tile0 = tile0;
  a.nspan = nspan;
  a.span[0] = sp[0];
  a.span[1] = nspan > 1 ? sp[1] : sp[0];
  a.blocks0 = (int64_t)sp[0].nl * a.g.Hkv * a.g.nwg;
  if (a.g.d == 64) launch_win<64>(tg, a, s);
  else launch_win<128>(tg, a, s);
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" size_t kvc_score_window_attn_workspace_size(int L, int Hq, int Hkv, int64_t n, int w,
                                                       int d, int dtype) {
  if (L < 1 || Hkv < 1 || Hq < Hkv || n < 1 || w < 1 || d < 1) return 0;
  Plan P;
  make_plan(L, Hq, Hkv, n, w, d, dtype, &P);
  return P.part_bytes + P.c_bytes + 256;
}

extern "C" int kvc_score_window_attn(const void* const* q_win, const void* const* k, int dtype,
                                     int L, int Hq, int Hkv, int64_t n, int w, int d, float scale,
                                     int per_query_head, float* A_out, void* ws, size_t ws_bytes,
                                     void* stream) {
  clear_error();
  if (!dtype_ok(dtype)) return KVC_FAIL(KVC_ERR_DTYPE, "kvc_score_window_attn: dtype %d", dtype);
  KVC_REQUIRE(L >= 1 && L <= KVC_MAX_LAYERS, "kvc_score_window_attn: need 1 <= L <= %d", KVC_MAX_LAYERS);
  KVC_REQUIRE(Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0, "kvc_score_window_attn: need Hq %% Hkv == 0");
  KVC_REQUIRE(n >= 1 && w >= 1 && w <= n, "kvc_score_window_attn: need 1 <= w <= n");
  KVC_REQUIRE(n <= 0x7fffffffLL, "kvc_score_window_attn: n > 2^31-1");
  KVC_REQUIRE(per_query_head == 0 || per_query_head == 1, "kvc_score_window_attn: per_query_head");
  // The passes keep running maxima of the raw dot products and scale them
  // afterwards, which is the maximum of the scaled logits only for scale > 0.
  KVC_REQUIRE(scale > 0.f && std::isfinite(scale), "kvc_score_window_attn: need a finite scale > 0");
  KVC_REQUIRE(q_win && k && A_out, "kvc_score_window_attn: null pointer");
  for (int l = 0; l < L; ++l)
    KVC_REQUIRE(q_win[l] && k[l], "kvc_score_window_attn: null pointer in layer %d", l);
  Plan P;
  make_plan(L, Hq, Hkv, n, w, d, dtype, &P);
  const Geo& g = P.g;
  if (P.mfma) {
    KVC_REQUIRE(d == 64 || d == 128, "kvc_score_window_attn: bf16 needs d in {64, 128}");
    KVC_REQUIRE(g.ntiles <= MAX_TILES, "kvc_score_window_attn: (Hq/Hkv)*ceil(w/32) > %d", MAX_TILES);
    for (int l = 0; l < L; ++l)
      KVC_REQUIRE((uintptr_t)q_win[l] % 16 == 0 && (uintptr_t)k[l] % 16 == 0,
                  "kvc_score_window_attn: bf16 tensors must be 16-byte aligned");
    KVC_REQUIRE((int64_t)2 * kLayersPerLaunch * Hkv * g.nwg <= 0x7fffffffLL,
                "kvc_score_window_attn: grid too large");
  } else {
    KVC_REQUIRE(d >= 1 && d <= 256, "kvc_score_window_attn: float32 needs d <= 256");
    KVC_REQUIRE((int64_t)g.G * w * d * 4 <= 64 * 1024,
                "kvc_score_window_attn: float32 path needs (Hq/Hkv)*w*d*4 <= 64 KB");
  }
  const size_t need = P.part_bytes + P.c_bytes;
  char* base = ws ? (char*)(((uintptr_t)ws + 255) & ~(uintptr_t)255) : nullptr;
  if (!ws || (size_t)(base - (char*)ws) + need > ws_bytes)
    return KVC_FAIL(KVC_ERR_WORKSPACE, "kvc_score_window_attn: workspace needs %zu bytes", need + 256);
  float2* part = (float2*)base;
  float* cfin = (float*)(base + P.part_bytes);
  hipStream_t s = as_stream(stream);
  const float sl2 = scale * LOG2E;
  const int Aheads = per_query_head ? Hq : Hkv;

  for (int l0 = 0; l0 < L; l0 += kLayersPerLaunch) {        // layer groups of at most 32
    const int lc = min(kLayersPerLaunch, L - l0);
    ConstPtrs qt{}, kt{};
    for (int i = 0; i < lc; ++i) { qt.p[i] = q_win[l0 + i]; kt.p[i] = k[l0 + i]; }
    float* A = A_out + (int64_t)l0 * Aheads * n;
    if (P.mfma) {
      WinArgs a{};
      a.q = qt; a.k = kt; a.g = g; a.sl2 = sl2; a.per_head = per_query_head;
      a.part = part; a.A = A;
      const int nch = (lc + P.lch - 1) / P.lch;
      if (g.ntiles <= MAX_TG) {
        // launch i: pass 2 of chunk i-1 beside pass 1 of chunk i
        for (int i = 0; i <= nch; ++i) {
          Span sp[2];
          int ns = 0;
          if (i >= 1) sp[ns++] = Span{(i - 1) * P.lch, min(P.lch, lc - (i - 1) * P.lch), 2};
          if (i < nch) sp[ns++] = Span{i * P.lch, min(P.lch, lc - i * P.lch), 1};
          launch_spans(a, 0, g.ntiles, ns, sp, s);
        }
      } else {
        for (int c = 0; c < nch; ++c) {
          const Span s1{c * P.lch, min(P.lch, lc - c * P.lch), 1};
          const Span s2{s1.l0, s1.nl, 2};
          for (int t0 = 0; t0 < g.ntiles; t0 += MAX_TG) launch_spans(a, t0, min(MAX_TG, g.ntiles - t0), 1, &s1, s);
          for (int t0 = 0; t0 < g.ntiles; t0 += MAX_TG) launch_spans(a, t0, min(MAX_TG, g.ntiles - t0), 1, &s2, s);
        }
      }
    } else {
      const int R = g.G * w;
      hipLaunchKernelGGL(win_f32_stats, dim3((unsigned)((int64_t)lc * Hkv * R)), dim3(NTF), 0, s,
                         qt, kt, g, sl2, cfin);
      const int64_t nblk = (n + NTA - 1) / NTA;
      const dim3 ga((unsigned)(lc * Hkv * nblk));
      const size_t lds = (size_t)R * d * sizeof(float);
#define KVC_A(DD) hipLaunchKernelGGL((win_f32_accum<DD>), ga, dim3(NTA), lds, s, qt, kt, g, sl2, \
                                     (const float*)cfin, per_query_head, A)
      switch (d) {
        case 16: KVC_A(16); break;
        case 32: KVC_A(32); break;
        case 64: KVC_A(64); break;
        case 128: KVC_A(128); break;
        default: KVC_A(0); break;
      }
#undef KVC_A
    }
  }
  return launch_status("kvc_score_window_attn");
}

// ------------------------------------------------------------------ no-alloc variant
// For callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid it): the workspace lives in a
// file-scope device array that every GPU the library runs on holds until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in): its device address is taken once per device
// with hipGetSymbolAddress, with that device current, and that address is what
// the kernels receive.  Every call on one GPU shares that GPU's copy, so calls
// that overlap on one GPU (different streams, or threads) race.  The workspace
// needs no initial contents, so nothing is cleared.
namespace {

constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;     // 32 MiB per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (looked up on first use).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return KVC_FAIL(KVC_ERR_HIP, "kvc_score_window_attn_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return KVC_FAIL(KVC_ERR_HIP, "kvc_score_window_attn_noalloc: device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return KVC_FAIL(KVC_ERR_HIP, "kvc_score_window_attn_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KVC_OK;
}

}  // namespace

extern "C" size_t kvc_score_window_attn_noalloc_max_workspace(void) { return kNoAllocScratchBytes; }

extern "C" int kvc_score_window_attn_noalloc(const void* const* q_win, const void* const* k, int dtype,
                                             int L, int Hq, int Hkv, int64_t n, int w, int d,
                                             float scale, int per_query_head, float* A_out,
                                             void* stream) {
  clear_error();
  // size check first, before the device is touched
  const size_t need = kvc_score_window_attn_workspace_size(L, Hq, Hkv, n, w, d, dtype);
  if (need > kNoAllocScratchBytes)
    return KVC_FAIL(KVC_ERR_WORKSPACE,
                    "kvc_score_window_attn_noalloc: this shape needs %zu bytes of workspace, more than "
                    "the %zu-byte device scratch (use kvc_score_window_attn with a workspace)",
                    need, kNoAllocScratchBytes);
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != KVC_OK) return st;
  return kvc_score_window_attn(q_win, k, dtype, L, Hq, Hkv, n, w, d, scale, per_query_head, A_out,
                               ws, kNoAllocScratchBytes, stream);
}
