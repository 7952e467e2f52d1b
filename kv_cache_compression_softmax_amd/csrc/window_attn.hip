// Observation-window attention A (group mean, per query head, or the group mean and the
// group max over query heads).
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
  int per_head;                        // output form: 0 group mean, 1 per head, 2 group mean and max
  float2* part;                        // [32, Hkv, nwg, rows] pass-1 partials
  float* A;                            // output of the layer group
  float* A2;                           // form 2: the group max plane of the layer group
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
template <int D, int TG, int OM>
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
    constexpr bool PH = OM == 1;
    if constexpr (OM == 2) {                     // every head of the group in this launch, one tile each
      // group mean (lower half-wave) and group max (upper half-wave) of the heads'
      // column sums, one store instruction for both planes
      float tot = 0.f, mx = 0.f;
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        const float cs = add_halves(hs[t]);
        tot += cs;
        mx = t == 0 ? cs : fmaxf(mx, cs);
      }
      if (key < g.n) {
        const int64_t o = ((int64_t)l * g.Hkv + kvh) * g.n + key;
        if (hf == 0) A[o] = tot * inv_group;
        else a.A2[o] = mx * inv_w;
      }
      return;
    }
    if constexpr (!PH) {                         // one cross-half add for the group
      float own = hs[0];
#pragma unroll
      for (int t = 1; t < TG; ++t) own += hs[t];
      total = add_halves(own);
    }
    if (PH && g.tph == 1) {                      // one tile per head (w <= 32): no sums over tiles
      // both halves hold every head's column sum; the upper half stores the
      // next head, so one store instruction writes two heads' 32 keys
      float cs[TG];
#pragma unroll
      for (int t = 0; t < TG; ++t) cs[t] = add_halves(hs[t]);
#pragma unroll
      for (int t = 0; t < TG; t += 2) {
        const bool two = t + 1 < TG;
        const float v = (two && hf) ? cs[t + 1] : cs[t];
        if ((two || hf == 0) && key < g.n) {
          const int head = kvh * g.G + a.tile0 + t + (two ? hf : 0);
          A[((int64_t)l * g.Hq + head) * g.n + key] = v * inv_w;
        }
      }
      return;
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

// OM: output form (0 group mean, 1 per query head, 2 group mean and group max),
// fixed at compile time so that the pass-2 block stays one scheduling region
template <int D, int TG, int OM>
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
    else pass2<D, TG, OM>(a, sm, l, kvh, wgi);
    __syncthreads();                             // LDS is reused by the next task
  }
}


// ---------------------------------------------------------------- XCD-resident path
// Pass 2 of the kernel above reads every key a second time.  When a (layer, KV
// head) unit's keys fit in the registers of one XCD's workgroups, this kernel
// reads them once: a team of workgroups on one XCD loads the unit's keys into
// registers (128 VGPRs of keys per wave), runs pass 1 on them, meets at a team
// barrier, merges the members' row normalisers and runs pass 2 on the same
// registers.  While pass 2 works through a key block, that block's registers are
// refilled with the team's next unit, and pass 1 of that unit follows right
// behind the loads.
//
// Workgroups are 512 threads (two waves per SIMD) and need more than half of a
// CU's registers, so a CU holds one; the launch is cooperative (every workgroup
// resident at once), so each XCD holds exactly as many workgroups as it has CUs.
// A workgroup learns its XCD from the hardware register and takes a slot on that
// XCD from an atomic counter; teams are formed from slots, so a team's members
// share one L2 whatever order the dispatcher used.  Pass-1 records are plain
// stores read back with plain loads through that L2 (each record line is read
// only after the team barrier, and only once); the team counters are atomics.
// A barrier that runs out of spins sets bit 1 of the status word and turns the
// team's outputs into NaN rather than leaving plausible wrong values.  (Teams of
// one workgroup per CU keep the members in step: with two 256-thread workgroups
// per CU the younger one lost the issue arbitration and every barrier waited
// for it.)
// stage_q for the threads t0 .. of a group of nthr (tile0 = 0).
template <int D, int TG>
__device__ __forceinline__ void stage_q_part(const uint16_t* q, const Geo& g, int kvh, uint4* qlds, int t0,
                                             int nthr) {
  constexpr int S = D / 16, C = D / 8;
  for (int f = t0; f < TG * 32 * C; f += nthr) {
    const int c16 = f % C, i = (f / C) % 32, t = f / (32 * C);
    const int hf = c16 & 1, st = c16 >> 1;
    const int head = kvh * g.G + t / g.tph;
    const int rr = (t % g.tph) * 32 + i;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (rr < g.w) v = *reinterpret_cast<const uint4*>(q + ((int64_t)head * g.w + rr) * D + c16 * 8);
    qlds[(t * S + st) * 64 + hf * 32 + i] = v;
  }
}

constexpr int kXcds = 8;
constexpr int NTX = 512;             // threads per workgroup
constexpr int kXRows = 128;          // partial record stride (rows, 512 bytes)
constexpr int kXCntStride = 32;      // team counters 128 bytes apart
constexpr int kXSpinLimit = 1 << 20; // polls before a team barrier gives up (seconds)
constexpr int kXMaxTeam = 32;        // workgroups per team at most (one XCD, one per CU)
constexpr int kXMaxRec = kXMaxTeam / 2;   // records each merging thread reads (>= 2 threads per row)

struct XArgs {
  ConstPtrs q, k;                    // per-layer pointers of the current layer group
  Geo g;
  float sl2;                         // scale * log2(e)
  int per_head;                      // output form (as WinArgs)
  int nunits;                        // (layer, KV head) units of the group
  int tw;                            // workgroups per team
  int tpx;                           // teams per XCD (workgroups past tpx * tw idle)
  int nteams;                        // teams on the chip (kXcds * tpx)
  int stagger;                       // start delay of odd XCDs, in 10 ns ticks
  float* part;                       // [nunits][kXRows][kXMaxTeam] row log-normalisers of each member
  unsigned* cnt;                     // [nunits][kXCntStride] team counters (first word used)
  unsigned* status;                  // bit 1: a barrier gave up; bit 2: an XCD beyond kXcds
  unsigned* reg;                     // [kXcds] slots taken on each XCD
  float* A;                          // output of the layer group
  float* A2;                         // form 2: the group max plane of the layer group
};

template <int D, int NT>
struct XSmem {
  uint4 q[2][NT * (D / 16) * 64];                // Q of this unit and of the next, fragment order
  float2 wst[NTX / 64][NT * 32];                 // pass 1: per-wave row stats
  __attribute__((aligned(16))) float c[NT * 32]; // pass 2: row normalisers
  float2 red[NTX];                               // partial merges
  int ok;                                        // team barrier completed
  int xcc, slot;                                 // this workgroup's XCD and its slot there
};

// Keys of one unit for this wave: blocks b0 .. b0 + KBM - 1 of 32 keys, in the
// MFMA k layout (step st, half hf: elements 16 st + 8 hf .. + 8 of key i).  Rows
// past the end of K are clamped to the last key, so the loads are unconditional.
template <int D, int KBM>
__device__ __forceinline__ void x_load_block(bf16x8 (&kr)[D / 16], const XArgs& a, int u, int64_t key0,
                                             int lane) {
  constexpr int S = D / 16;
  const int l = u / a.g.Hkv, kvh = u % a.g.Hkv;
  const int i = lane & 31, hf = lane >> 5;
  const uint16_t* kh = (const uint16_t*)a.k.p[l] + (int64_t)kvh * a.g.n * D;
  const int64_t key = min(key0 + i, a.g.n - 1);
  const uint16_t* p = kh + key * D + 8 * hf;
#pragma unroll
  for (int st = 0; st < S; ++st) kr[st] = *reinterpret_cast<const bf16x8*>(p + 16 * st);
}

template <int D, int NT, int OM>
__global__ void __launch_bounds__(NTX) __attribute__((amdgpu_waves_per_eu(2, 2)))
win_xcd(XArgs a) {
  constexpr int S = D / 16, KBM = 512 / D, R = NT * 32;
  __shared__ XSmem<D, NT> sm;
  const Geo& g = a.g;
  const int lane = threadIdx.x & 63, hf = lane >> 5, qi = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  // this workgroup's XCD (hardware register XCC_ID) and its slot there
  if (threadIdx.x == 0) {
    const int xcc = (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 15);
    int slot = 1 << 20;                          // no team
    if (xcc < kXcds) slot = (int)__hip_atomic_fetch_add(&a.reg[xcc], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else __hip_atomic_fetch_or(a.status, 4u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.xcc = xcc;
    sm.slot = slot;
  }
  __syncthreads();
  const int x = __builtin_amdgcn_readfirstlane(sm.xcc), rank = __builtin_amdgcn_readfirstlane(sm.slot);
  const int team = rank / a.tw, mem = rank % a.tw;
  const int first = team * kXcds + x;
  if (team >= a.tpx || first >= a.nunits) return;   // whole workgroup: no team, or no unit
  const int64_t nblk = (g.n + 31) / 32;
  const int64_t b0 = (int64_t)(mem * (NTX / 64) + wv) * KBM;     // this wave's first key block
  const int nb = (int)max((int64_t)0, min((int64_t)KBM, nblk - b0));
  const int64_t safe_end = g.n - g.w;            // keys <= this are seen by every row
  const float inv_group = 1.0f / (float)(g.G * g.w), inv_w = 1.0f / (float)g.w;

  int pos[NT];                                   // window position of this lane's row (pass 1)
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    pos[t] = qi < g.w ? (int)(g.n - g.w) + qi : -1;
  }

  bf16x8 kr[KBM][S];
  {
    const int u = first;
    stage_q_part<D, NT>((const uint16_t*)a.q.p[u / g.Hkv], g, u % g.Hkv, sm.q[0], threadIdx.x, NTX);
#pragma unroll
    for (int b = 0; b < KBM; ++b) x_load_block<D, KBM>(kr[b], a, u, (b0 + b) * 32, lane);
    __syncthreads();
  }
  // Odd XCDs start about half a unit later.  The XCDs then take turns: while
  // one half streams the next unit's keys (pass 2), the other half computes
  // pass 1 and meets at its barrier, instead of all eight loading at once.
  if (x & 1) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();    // 100 MHz
    while (__builtin_amdgcn_s_memrealtime() - t0 < (uint64_t)a.stagger) __builtin_amdgcn_s_sleep(8);
  }
  // pass 1 of unit u (keys in kr, Q in ql), its record, and the arrival at the
  // unit's team barrier
  auto do_p1 = [&](int u, const uint4* ql, int64_t bk) __attribute__((always_inline)) {
    // ---- pass 1: per-lane online (max, sum of exp2) of each row over this wave's keys
    float m[NT], sx[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) { m[t] = -INFINITY; sx[t] = 0.f; }
    auto p1 = [&](const bf16x8 (&kc)[S], int64_t j0, auto full_t, auto fixed_t) __attribute__((always_inline)) {
      constexpr bool full = decltype(full_t)::value;
      constexpr bool fixed = decltype(fixed_t)::value;
      int qo = lane;
      asm volatile("" : "+v"(qo));               // keep the Q reads in the loop (LDS, not VGPRs)
      auto epi = [&](int t, f32x16 acc) __attribute__((always_inline)) {
        if constexpr (fixed) {
          float sum = __builtin_amdgcn_exp2f(fmaf(acc[0], a.sl2, -m[t]));
#pragma unroll
          for (int v = 1; v < 16; ++v) sum += __builtin_amdgcn_exp2f(fmaf(acc[v], a.sl2, -m[t]));
          sx[t] += sum;
          return;
        }
        float bm = -INFINITY;
        if constexpr (full) {
#pragma unroll
          for (int v = 0; v < 16; ++v) bm = fmaxf(bm, acc[v]);
        } else {
          // key offset limit within the block.  The mask is a min with +inf or
          // -inf whose sign comes from lim - off (sign-bit arithmetic, no
          // compares), so it needs no per-element compare masks in SGPRs.
          const int lim = (int)(min((int64_t)pos[t], g.n - 1) - j0) - 4 * hf;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int off = 8 * (v >> 2) + (v & 3);
            const float cap = __uint_as_float(((unsigned)(lim - off) & 0x80000000u) | 0x7f800000u);
            acc[v] = fminf(acc[v], cap);
            bm = fmaxf(bm, acc[v]);
          }
        }
        const float mn = fmaxf(m[t], bm * a.sl2);
        const float ms = full ? mn : (mn > -INFINITY ? mn : 0.f);
        float sum = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) sum += __builtin_amdgcn_exp2f(fmaf(acc[v], a.sl2, -ms));
        sx[t] = sx[t] * __builtin_amdgcn_exp2f(m[t] - ms) + sum;
        m[t] = mn;
      };
      pipelined_tiles<S, NT, true>(kc, ql, qo, epi);
    };
#pragma unroll
    for (int b = 0; b < KBM; ++b) {
      if (b < nb) {                              // wave-uniform
        const int64_t j0 = (bk + b) * 32;
        if (j0 + 31 <= safe_end) {
          if (b > 0) p1(kr[b], j0, std::true_type{}, std::true_type{});
          else p1(kr[b], j0, std::true_type{}, std::false_type{});
        } else {
          p1(kr[b], j0, std::false_type{}, std::false_type{});
        }
      }
    }
    bool bad = false;
#pragma unroll
    for (int t = 0; t < NT; ++t) bad = bad || !(sx[t] <= 3.0e38f);     // inf or NaN
    if (__builtin_amdgcn_ballot_w64(bad) != 0) {  // again with the running maximum
#pragma unroll
      for (int t = 0; t < NT; ++t) { m[t] = -INFINITY; sx[t] = 0.f; }
#pragma unroll
      for (int b = 0; b < KBM; ++b) {
        if (b < nb) {
          const int64_t j0 = (bk + b) * 32;
          if (j0 + 31 <= safe_end) p1(kr[b], j0, std::true_type{}, std::false_type{});
          else p1(kr[b], j0, std::false_type{}, std::false_type{});
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {               // halves (lanes i, i+32 share a row), then waves
      const float mo = __shfl_xor(m[t], 32, 64), so = __shfl_xor(sx[t], 32, 64);
      const float M = fmaxf(m[t], mo);
      float Sx = 0.f;
      if (M > -INFINITY) Sx = sx[t] * exp2f(m[t] - M) + so * exp2f(mo - M);
      if (hf == 0) sm.wst[wv][t * 32 + qi] = make_float2(M, Sx);
    }
    __syncthreads();
    if (threadIdx.x < R) {
      float M = -INFINITY;
#pragma unroll
      for (int w2 = 0; w2 < NTX / 64; ++w2) M = fmaxf(M, sm.wst[w2][threadIdx.x].x);
      float Sx = 0.f;
      if (M > -INFINITY) {
#pragma unroll
        for (int w2 = 0; w2 < NTX / 64; ++w2)
          if (sm.wst[w2][threadIdx.x].x > -INFINITY)
            Sx += sm.wst[w2][threadIdx.x].y * exp2f(sm.wst[w2][threadIdx.x].x - M);
      }
      a.part[((int64_t)u * kXRows + threadIdx.x) * kXMaxTeam + mem] = Sx > 0.f ? M + log2f(Sx) : -INFINITY;
      __builtin_amdgcn_s_waitcnt(0xF70);         // vmcnt(0): the record is in L2 before we count
    }
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(&a.cnt[(int64_t)u * kXCntStride], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto wait_team = [&](int u) __attribute__((always_inline)) {
    if (threadIdx.x == 0) {
      int it = 0;
      for (; it < kXSpinLimit; ++it) {
        unsigned z = 0;
        asm volatile("" : "+v"(z));              // a real read-modify-write: it reads the atomic's value
        if (__hip_atomic_fetch_add(&a.cnt[(int64_t)u * kXCntStride], z, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT) >= (unsigned)a.tw)
          break;
        __builtin_amdgcn_s_sleep(2);
      }
      sm.ok = it < kXSpinLimit;
      if (it == kXSpinLimit) __hip_atomic_fetch_or(a.status, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
  };
  auto merge_c = [&](int u) __attribute__((always_inline)) {
    // ---- row normalisers: thread j of a row merges the j-th run of kXMaxRec
    // members, then the runs are merged in order (a fixed order: the result
    // does not depend on arrival); +inf for padding rows, NaN if the barrier
    // gave up
    {
      constexpr int P = NTX / R;
      const int r = threadIdx.x % R, j = threadIdx.x / R;
      if (j < P) {
        // members j*kXMaxRec .. +kXMaxRec of row r, contiguous: eight 16-byte
        // loads requested at once (one L2 round trip); members past the team
        // are read from the row's padding and ignored
        float M = -INFINITY, Sx = 0.f;
        if (j * kXMaxRec < a.tw) {
          const float4* pr = reinterpret_cast<const float4*>(a.part + ((int64_t)u * kXRows + r) * kXMaxTeam + j * kXMaxRec);
          float v[kXMaxRec];
#pragma unroll
          for (int e = 0; e < kXMaxRec / 4; ++e) {
            const float4 f = pr[e];
            v[4 * e] = f.x; v[4 * e + 1] = f.y; v[4 * e + 2] = f.z; v[4 * e + 3] = f.w;
          }
#pragma unroll
          for (int e = 0; e < kXMaxRec; ++e)
            if (j * kXMaxRec + e >= a.tw) v[e] = -INFINITY;
#pragma unroll
          for (int e = 0; e < kXMaxRec; ++e) M = fmaxf(M, v[e]);
          if (M > -INFINITY) {                   // independent terms, summed as a tree
            float t[kXMaxRec];
#pragma unroll
            for (int e = 0; e < kXMaxRec; ++e) t[e] = exp2f(v[e] - M);
#pragma unroll
            for (int h = kXMaxRec / 2; h > 0; h /= 2)
#pragma unroll
              for (int e = 0; e < h; ++e) t[e] += t[e + h];
            Sx = t[0];
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
        const bool pad = (r & 31) >= g.w;
        float cr = (!pad && Mt > -INFINITY) ? Mt + log2f(St) : INFINITY;
        if (!sm.ok) cr = __builtin_nanf("");
        sm.c[r] = cr;
      }
      __syncthreads();
    }

  };
  // pass 2 of unit u; each key block's registers then take the same block of
  // unit uload (the team's next unit, or u again after its last)
  auto do_p2 = [&](int u, int uload, const uint4* ql, int64_t bk) __attribute__((always_inline)) {
    const int l = u / g.Hkv, kvh = u % g.Hkv;
    // ---- pass 2: column sums of exp2(s - c_r); each block's registers then take
    // the same block of the team's next unit.  No load is in flight here (pass 1
    // consumed every key); saying so lets the compiler see that pass 2's reads of
    // the key registers wait for nothing, not for the next unit's loads.
    __builtin_amdgcn_s_waitcnt(0xF70);           // vmcnt(0)
    auto p2 = [&](const bf16x8 (&kc)[S], int64_t j0, auto full_t) __attribute__((always_inline)) {
      constexpr bool full = decltype(full_t)::value;
      const int64_t key = j0 + qi;               // this lane's key column
      int qo = lane, co = hf;
      asm volatile("" : "+v"(qo), "+v"(co));
      float hs[NT];
      auto epi = [&](int t, const f32x16& acc) __attribute__((always_inline)) {
        const int base = 4 * hf;
        const int lo = (int)(key - safe_end) - base;
        const int hi = (key < g.n) ? g.w - base : -1;
        float colsum = 0.f;
        int cot = co;                            // c reads of tile t not before its epilogue
        asm volatile("" : "+v"(cot));
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const float4 c4 = reinterpret_cast<const float4*>(sm.c)[t * 8 + 2 * qd + cot];
          const float cc[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
          for (int uu = 0; uu < 4; ++uu) {
            const int v = 4 * qd + uu, off = 8 * qd + uu;
            float z = fmaf(acc[v], a.sl2, -cc[uu]);
            if constexpr (!full) {                 // rows lo <= off < hi only: -inf otherwise
              const unsigned sg = (unsigned)((off - lo) | (hi - 1 - off)) & 0x80000000u;
              z = fminf(z, __uint_as_float(sg | 0x7f800000u));
            }
            colsum += __builtin_amdgcn_exp2f(z);
          }
        }
        hs[t] = colsum;
      };
      pipelined_tiles<S, NT, false>(kc, ql, qo, epi);
#pragma unroll
      for (int t = 0; t < NT; ++t) asm volatile("" : "+v"(hs[t]));
      if constexpr (OM == 1) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {           // one tile per query head
          const float cs = add_halves(hs[t]);
          if (hf == 0 && key < g.n) a.A[((int64_t)l * g.Hq + kvh * g.G + t) * g.n + key] = cs * inv_w;
        }
      } else if constexpr (OM == 2) {            // group mean (lower half), group max (upper half)
        float tot = 0.f, mx = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const float cs = add_halves(hs[t]);
          tot += cs;
          mx = t == 0 ? cs : fmaxf(mx, cs);
        }
        if (key < g.n) {
          const int64_t o = ((int64_t)l * g.Hkv + kvh) * g.n + key;
          if (hf == 0) a.A[o] = tot * inv_group;
          else a.A2[o] = mx * inv_w;
        }
      } else {
        float own = hs[0];
#pragma unroll
        for (int t = 1; t < NT; ++t) own += hs[t];
        const float total = add_halves(own);
        if (hf == 0 && key < g.n) a.A[((int64_t)l * g.Hkv + kvh) * g.n + key] = total * inv_group;
      }
    };
#pragma unroll
    for (int b = 0; b < KBM; ++b) {
      if (b < nb) {
        const int64_t j0 = (bk + b) * 32;
        if (j0 + 31 <= safe_end) p2(kr[b], j0, std::true_type{});
        else p2(kr[b], j0, std::false_type{});
      }
      x_load_block<D, KBM>(kr[b], a, uload, (bk + b) * 32, lane);
    }
  };
  int64_t bk0 = b0;
  asm volatile("" : "+s"(bk0));
  do_p1(first, sm.q[0], bk0);
  if (wv > 0 && first + a.nteams < a.nunits)     // waves 1..3 stage the next Q while wave 0 waits
    stage_q_part<D, NT>((const uint16_t*)a.q.p[(first + a.nteams) / g.Hkv], g, (first + a.nteams) % g.Hkv,
                        sm.q[1], threadIdx.x - 64, NTX - 64);
  int qb = 0;
#pragma unroll 1
  for (int u = first; u < a.nunits; u += a.nteams, qb ^= 1) {
    const int un = u + a.nteams;                 // this team's next unit
    const bool more = un < a.nunits;
    // the key offsets are the same for every unit; made opaque here so that the
    // masks derived from them are computed per unit, not hoisted out of the loop
    // and held in registers across it
    int64_t bk = b0;
    asm volatile("" : "+s"(bk));
    wait_team(u);
    merge_c(u);
    // No load is in flight here (pass 1 consumed every key); saying so lets the
    // compiler see that pass 2's reads of the key registers wait for nothing.
    __builtin_amdgcn_s_waitcnt(0xF70);           // vmcnt(0)
    do_p2(u, more ? un : u, sm.q[qb], bk);
    __syncthreads();                             // c and this unit's Q are rewritten next
    if (more) {
      // pass 1 of the next unit right behind the loads pass 2 issued, in the same
      // straight-line code, so that each block waits only for its own keys
      do_p1(un, sm.q[qb ^ 1], bk);
      const int un2 = un + a.nteams;
      if (wv > 0 && un2 < a.nunits)
        stage_q_part<D, NT>((const uint16_t*)a.q.p[un2 / g.Hkv], g, un2 % g.Hkv, sm.q[qb], threadIdx.x - 64, NTX - 64);
    }
  }
}

__global__ void win_xcd_zero(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
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
              int per_head, float* __restrict__ A, float* __restrict__ A2) {
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
  float total = 0.f, mx = 0.f;
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
    if (per_head == 1) A[((int64_t)l * g.Hq + kvh * g.G + h) * g.n + j] = hs / (float)g.w;
    total += hs;
    mx = h == 0 ? hs : fmaxf(mx, hs);
  }
  if (per_head != 1) A[((int64_t)l * g.Hkv + kvh) * g.n + j] = total / (float)(g.G * g.w);
  if (per_head == 2) A2[((int64_t)l * g.Hkv + kvh) * g.n + j] = mx / (float)g.w;
}

// ---------------------------------------------------------------- host
struct Plan {
  Geo g;
  bool mfma;
  int lch;                      // layers per chunk
  size_t part_bytes, c_bytes;
  // XCD-resident kernel: the shape fits it, workgroups per team, workspace
  bool xshape;
  int xtw;
  size_t x_head_bytes, x_part_bytes;
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
  // XCD-resident kernel: one tile per head (w <= 32), each wave holds 512/d key
  // blocks, a team is at most one XCD's workgroups (checked against the device at
  // launch).  Workspace: status word, XCD slot counters, team counters, records.
  P->xshape = false;
  P->xtw = 0;
  P->x_head_bytes = P->x_part_bytes = 0;
  if (P->mfma && (d == 64 || d == 128) && g.tph == 1 && g.ntiles <= MAX_TG) {
    const int64_t kbm = 512 / d, nblk = (n + 31) / 32, per_wg = (NTX / 64) * kbm;
    const int64_t tw = (nblk + per_wg - 1) / per_wg;
    if (tw <= kXMaxTeam) {
      P->xshape = true;
      P->xtw = (int)tw;
      P->x_head_bytes = 256 + (size_t)lg_max * Hkv * kXCntStride * sizeof(unsigned);
      P->x_part_bytes = (size_t)lg_max * Hkv * kXRows * kXMaxTeam * sizeof(float);
    }
  }
}

// Dynamic LDS that takes a workgroup of the XCD-resident kernel past half of a
// CU's 160 KB, so that a CU holds one (the slot counting relies on it).
constexpr size_t kXMinLds = 80 * 1024 + 256;

template <int D, int NT, int OM>
bool launch_xcd_t(XArgs a, hipStream_t s) {
  const void* kern = reinterpret_cast<const void*>(&win_xcd<D, NT, OM>);
  const size_t stat = sizeof(XSmem<D, NT>);
  const size_t dyn = stat < kXMinLds ? kXMinLds - stat : 0;
  int dev = 0, ncu = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, NTX, dyn) != hipSuccess)
    return false;
  if (per_cu != 1 || ncu <= 0 || ncu % kXcds) return false;
  const int wpx = ncu / kXcds;                   // workgroups on each XCD
  if (wpx < a.tw) return false;
  a.tpx = wpx / a.tw;
  a.nteams = kXcds * a.tpx;
  if (a.nunits <= a.nteams) a.stagger = 0;      // one unit per team: nothing to interleave
  void* args[] = {&a};
  // cooperative: every workgroup resident at once (the team barriers need it)
  return hipLaunchCooperativeKernel(kern, dim3((unsigned)ncu), dim3(NTX), args, (unsigned)dyn, s) == hipSuccess;
}

template <int D, int OM>
bool launch_xcd_d(const XArgs& a, hipStream_t s) {
  switch (a.g.ntiles) {
    case 1: return launch_xcd_t<D, 1, OM>(a, s);
    case 2: return launch_xcd_t<D, 2, OM>(a, s);
    case 3: return launch_xcd_t<D, 3, OM>(a, s);
    default: return launch_xcd_t<D, 4, OM>(a, s);
  }
}

bool launch_xcd(const XArgs& a, hipStream_t s) {
  if (a.g.d == 64)
    return a.per_head == 1 ? launch_xcd_d<64, 1>(a, s)
         : a.per_head == 2 ? launch_xcd_d<64, 2>(a, s) : launch_xcd_d<64, 0>(a, s);
  return a.per_head == 1 ? launch_xcd_d<128, 1>(a, s)
       : a.per_head == 2 ? launch_xcd_d<128, 2>(a, s) : launch_xcd_d<128, 0>(a, s);
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

template <int D, int TG, int OM>
void launch_win_ph(WinArgs a, hipStream_t s) {
  const void* kern = reinterpret_cast<const void*>(&win_kernel<D, TG, OM>);
  const int64_t res = resident_blocks(kern);
  const dim3 grid((unsigned)(a.ntask < res ? a.ntask : res)), block(NTW);
  hipLaunchKernelGGL((win_kernel<D, TG, OM>), grid, block, 0, s, a);
}

template <int D, int TG>
void launch_win_tg(WinArgs a, hipStream_t s) {
  if (a.per_head == 1) launch_win_ph<D, TG, 1>(a, s);
  else if (a.per_head == 2) launch_win_ph<D, TG, 2>(a, s);
  else launch_win_ph<D, TG, 0>(a, s);
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
  const size_t two = P.part_bytes + P.c_bytes, xcd = P.x_head_bytes + P.x_part_bytes;
  return (two > xcd ? two : xcd) + 256;
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
  KVC_REQUIRE(per_query_head >= 0 && per_query_head <= 2, "kvc_score_window_attn: per_query_head not 0, 1 or 2");
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
    // form 2 takes the group max over heads inside one launch: one tile per head
    // and every head of the group in the launch
    KVC_REQUIRE(per_query_head != 2 || (g.tph == 1 && g.ntiles <= MAX_TG),
                "kvc_score_window_attn: per_query_head 2 needs w <= 32 and Hq/Hkv <= %d", MAX_TG);
  } else {
    KVC_REQUIRE(d >= 1 && d <= 256, "kvc_score_window_attn: float32 needs d <= 256");
    KVC_REQUIRE((int64_t)g.G * w * d * 4 <= 64 * 1024,
                "kvc_score_window_attn: float32 path needs (Hq/Hkv)*w*d*4 <= 64 KB");
  }
  const size_t need = P.part_bytes + P.c_bytes;
  const size_t xneed = P.x_head_bytes + P.x_part_bytes;
  char* base = ws ? (char*)(((uintptr_t)ws + 255) & ~(uintptr_t)255) : nullptr;
  if (!ws || (size_t)(base - (char*)ws) + need > ws_bytes)
    return KVC_FAIL(KVC_ERR_WORKSPACE, "kvc_score_window_attn: workspace needs %zu bytes", need + 256);
  float2* part = (float2*)base;
  float* cfin = (float*)(base + P.part_bytes);
  hipStream_t s = as_stream(stream);
  const float sl2 = scale * LOG2E;
  const int Aheads = per_query_head == 1 ? Hq : Hkv;

  for (int l0 = 0; l0 < L; l0 += kLayersPerLaunch) {        // layer groups of at most 32
    const int lc = min(kLayersPerLaunch, L - l0);
    ConstPtrs qt{}, kt{};
    for (int i = 0; i < lc; ++i) { qt.p[i] = q_win[l0 + i]; kt.p[i] = k[l0 + i]; }
    float* A = A_out + (int64_t)l0 * Aheads * n;
    float* A2 = per_query_head == 2 ? A_out + ((int64_t)L + l0) * Hkv * n : nullptr;   // second plane
    bool done = false;
    if (P.xshape && (size_t)(base - (char*)ws) + xneed <= ws_bytes) {
      // keys read once; not under stream capture (cooperative launch), and the
      // two-pass kernel below when the device cannot hold the grid
      hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
      if (hipStreamIsCapturing(s, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone) {
        XArgs xa{};
        xa.q = qt; xa.k = kt; xa.g = g; xa.sl2 = sl2; xa.per_head = per_query_head;
        xa.nunits = lc * Hkv;
        xa.tw = P.xtw;
        // odd XCDs start about half a unit's time later (10 us at 1024 key
        // blocks), when the teams have more than one unit each
        const int64_t nblk = (n + 31) / 32;
        xa.stagger = (int)(nblk * 1000 / 1024);
        xa.status = (unsigned*)base;
        xa.reg = (unsigned*)(base + 64);
        xa.cnt = (unsigned*)(base + 256);
        xa.part = (float*)(base + P.x_head_bytes);
        xa.A = A;
        xa.A2 = A2;
        // status and counters start at zero (a fill kernel, not a memset)
        const int nz = (int)(P.x_head_bytes / sizeof(unsigned));
        hipLaunchKernelGGL(win_xcd_zero, dim3((nz + 255) / 256), dim3(256), 0, s, (unsigned*)base, nz);
        done = launch_xcd(xa, s);
        if (!done) (void)hipGetLastError();      // the two-pass kernel takes over
      }
    }
    if (done) {
    } else if (P.mfma) {
      WinArgs a{};
      a.q = qt; a.k = kt; a.g = g; a.sl2 = sl2; a.per_head = per_query_head;
      a.part = part; a.A = A; a.A2 = A2;
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
                                     (const float*)cfin, per_query_head, A, A2)
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
