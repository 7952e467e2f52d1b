// Decode attention of one query per head over a KV cache, with the optional
// compensation bias alpha * ln R on the logits.
//
// [SelKV] section 2, attention compensation: at decode time a merged entry's
// logit is raised by alpha * ln R so that it receives the attention mass of the
// tokens it stands for.  The same kernel over the full and the compacted cache
// gives the outputs compared by [RECAS] section 2.B's dropped-mass bound.
//
// Both kernels split the cache length into chunks and keep, per chunk and query
// head, the triple (max logit, sum of exp, unnormalised output); a second kernel
// merges a head's chunks in index order.  Each K/V row is read once per KV head,
// for all G query heads of its group.
//
// decode_mfma (bf16, d = 64 or 128, G <= 4): one wave per chunk of keys, in
// tiles of 16 keys.  The cache is split into equal chunks (a multiple of 32
// keys) so that the grid holds about one wave per SIMD (kWaveTarget): one long
// stream per SIMD ran at 6.7 TB/s where 512-key chunks (13 waves per SIMD)
// ran at 5.3 TB/s and unequal chunks left SIMDs idle at the end.
//   * Logits on the matrix core: v_mfma_f32_16x16x32_bf16 with the query heads
//     on M (row c holds head c mod 4, so every lane sees all four heads of its
//     key column) and 16 keys on N.  Each lane loads its key row's 16-byte
//     pieces in the instruction's own k layout: one load instruction reads 64
//     contiguous bytes of each of 16 rows.
//   * Online softmax in base 2 once per tile and head: a 16-lane max and one
//     exp2 per (key, head).  The reference max moves only when a logit passes it
//     by more than 2^8, so the accumulators are rarely rescaled.  The tile's
//     probabilities go through LDS (16 bytes per key).
//   * P V on the vector ALU: lane l owns 8 values of one V row (16-byte loads,
//     rows d/8 lanes wide), so the output accumulators are 8 per head.
//   * The next tile's K, V and ln R loads are in flight during this tile's work.
// decode_partial (the general kernel: float32, other d, G up to 8): a workgroup
// handles one (layer, KV head, chunk of CK keys); LG lanes hold one row (16
// bytes each); per key the G dot products are reduced inside the lane group,
// then an online softmax keeps (max, sum, output) per head.  Lane groups, then
// waves, are merged in a fixed order.
#include <cmath>

#include "common.h"

namespace kvc {
namespace {

constexpr int NT = 256;
constexpr int CK = 1024;          // keys per workgroup (decode_partial)
constexpr int kWaveTarget = 1024;  // decode_mfma waves per launch: MI355X's 256 CUs x 4 SIMDs
constexpr int kSets = 2;           // decode_mfma register sets (tiles) per wave
constexpr int kScoreWaves = 2048;  // waves of active_scores_mfma
constexpr int kScoreSets = 4;      // active_scores_mfma register sets (tiles) per wave
constexpr int MAXG = 8;           // query heads per KV head
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;     // decode_mfma: rescale threshold, base-2 logits

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct DE;
template <> struct DE<uint16_t> {
  static constexpr int N = 8;
  __device__ static void unpack(const uint4& u, float (&x)[8]) {
    x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
    x[4] = bf16_lo(u.z); x[5] = bf16_hi(u.z); x[6] = bf16_lo(u.w); x[7] = bf16_hi(u.w);
  }
};
template <> struct DE<float> {
  static constexpr int N = 4;
  __device__ static void unpack(const uint4& u, float (&x)[4]) {
    x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
    x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
  }
};

// ix: per layer an int32 [Hkv, npos] list of cache rows to attend over (the
// active set), or null for rows 0..len-1 (then npos = len)
__device__ __forceinline__ float elem_f32(uint16_t b) { return bf16_to_f32(b); }
__device__ __forceinline__ float elem_f32(float f) { return f; }

struct DecTables { ConstPtrs q, K, V, logR, ix; int64_t npos; };

// partial layout: [lc, Hq, nchunk] x (m, l, -, -, o[d]), 16-byte aligned rows
template <typename T, int LG, int G>
__global__ void __launch_bounds__(NT)
decode_partial(DecTables t, int Hq, int Hkv, int64_t len, int d, float scale, float alpha_bias,
               int nchunk, float* __restrict__ part) {
  constexpr int W = DE<T>::N;
  constexpr int NG = NT / LG;                    // lane groups per block
  __shared__ float sm_m[NT / 64][G], sm_l[NT / 64][G];
  __shared__ float sm_o[NT / 64][G][256];
  const int lane = threadIdx.x & 63, wv = threadIdx.x / 64;
  const int grp = threadIdx.x / LG, c = threadIdx.x % LG;
  const int64_t bid = blockIdx.x;
  const int ch = (int)(bid % nchunk);
  const int g = (int)((bid / nchunk) % Hkv);
  const int l = (int)(bid / ((int64_t)nchunk * Hkv));
  const T* q = (const T*)t.q.p[l];
  const T* K = (const T*)t.K.p[l] + (int64_t)g * len * d;
  const T* V = (const T*)t.V.p[l] + (int64_t)g * len * d;
  const float* lr = t.logR.p[l] ? (const float*)t.logR.p[l] + (int64_t)g * len : nullptr;
  const int32_t* ix = t.ix.p[l] ? (const int32_t*)t.ix.p[l] + (int64_t)g * t.npos : nullptr;

  float qv[G][W];
#pragma unroll
  for (int h = 0; h < G; ++h)
    DE<T>::unpack(*reinterpret_cast<const uint4*>(q + (int64_t)(g * G + h) * d + c * W), qv[h]);
  float m[G], s[G], o[G][W];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY; s[h] = 0.f;
#pragma unroll
    for (int e = 0; e < W; ++e) o[h][e] = 0.f;
  }
  const int64_t j0 = (int64_t)ch * CK, j1 = min(t.npos, j0 + CK);
  for (int64_t jp = j0 + grp; jp < j1; jp += NG) {
    const int64_t j = ix ? min((int64_t)(uint32_t)ix[jp], len - 1) : jp;   // listed rows clamped into [0, len)
    float kx[W], vx[W];
    DE<T>::unpack(*reinterpret_cast<const uint4*>(K + j * d + c * W), kx);
    DE<T>::unpack(*reinterpret_cast<const uint4*>(V + j * d + c * W), vx);
    const float bias = lr ? alpha_bias * lr[j] : 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < W; ++e) dot += qv[h][e] * kx[e];
      dot = group_sum<LG>(dot);
      const float x = dot * scale + bias;
      const float mn = fmaxf(m[h], x);
      const float a = expf(m[h] - mn), p = expf(x - mn);
      s[h] = s[h] * a + p;
#pragma unroll
      for (int e = 0; e < W; ++e) o[h][e] = o[h][e] * a + p * vx[e];
      m[h] = mn;
    }
  }
  // merge the lane groups of a wave (xor over the group bits), fixed order
#pragma unroll
  for (int off = LG; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off, 64), so = __shfl_xor(s[h], off, 64);
      const float mn = fmaxf(m[h], mo);
      const float a = mn > -INFINITY ? expf(m[h] - mn) : 0.f;
      const float b = mn > -INFINITY ? expf(mo - mn) : 0.f;
      s[h] = s[h] * a + so * b;
#pragma unroll
      for (int e = 0; e < W; ++e) {
        const float oo = __shfl_xor(o[h][e], off, 64);
        o[h][e] = o[h][e] * a + oo * b;
      }
      m[h] = mn;
    }
  }
  if (lane < LG) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (lane == 0) { sm_m[wv][h] = m[h]; sm_l[wv][h] = s[h]; }
#pragma unroll
      for (int e = 0; e < W; ++e) sm_o[wv][h][c * W + e] = o[h][e];
    }
  }
  __syncthreads();
  // merge the waves; thread (h, e) writes one output element
  for (int x = threadIdx.x; x < G * d; x += NT) {
    const int h = x / d, e = x % d;
    float M = -INFINITY;
    for (int w2 = 0; w2 < NT / 64; ++w2) M = fmaxf(M, sm_m[w2][h]);
    float S = 0.f, O = 0.f;
    for (int w2 = 0; w2 < NT / 64; ++w2) {
      const float a = M > -INFINITY ? expf(sm_m[w2][h] - M) : 0.f;
      S += sm_l[w2][h] * a;
      O += sm_o[w2][h][e] * a;
    }
    float* p = part + (((int64_t)l * Hq + g * G + h) * nchunk + ch) * (d + 4);
    if (e == 0) { p[0] = M; p[1] = S; }
    p[4 + e] = O;
  }
}

// One tile's loads: K in MFMA B-operand order (key l%16, d = 32s + 8(l/16) .. +8),
// V as 4 values per lane (key 16 t/... see decode_mfma), ln R of key l%16.
template <int D>
struct DecTile {
  static constexpr int KB = D / 32;          // 16x16x32 k-blocks per key row
  static constexpr int VL = D / 8;           // lanes per V row (8 values each)
  static constexpr int VI = 16 * VL / 64;    // V load instructions per tile
  bf16x8 k[KB];
  u32x4 v[VI];
  float lr;
};

// The cache rows one tile reads: lane l's K row (key l % 16) and its V rows.
// jb, jlast are positions; with IDX the row of position p is ix[p] (loaded),
// otherwise p itself.
template <int D>
struct DecRows {
  int32_t k;
  int32_t v[DecTile<D>::VI];
};

template <int D, bool IDX>
__device__ __forceinline__ void dec_rows(DecRows<D>& r, const int32_t* ix, int64_t jb, int64_t jlast,
                                         int lane) {
  constexpr int VL = DecTile<D>::VL, KPI = 64 / VL;
  const int64_t kp = min(jb + (lane & 15), jlast);
  r.k = IDX ? ix[kp] : (int32_t)kp;
#pragma unroll
  for (int i = 0; i < DecTile<D>::VI; ++i) {
    const int64_t vp = min(jb + i * KPI + lane / VL, jlast);
    r.v[i] = IDX ? ix[vp] : (int32_t)vp;
  }
}

// Rows are clamped to rmax = len - 1 where they are used (a no-op for positions;
// for a listed row, a bad entry reads a wrong row, never one outside the head).
template <int D, bool BIAS>
__device__ __forceinline__ void dec_load(DecTile<D>& t, const uint16_t* K, const uint16_t* V,
                                         const float* lr, const DecRows<D>& r, uint32_t rmax, int lane) {
  constexpr int VL = DecTile<D>::VL;
  const uint32_t rk = min((uint32_t)r.k, rmax);
  const uint16_t* kr = K + (int64_t)rk * D + 8 * (lane >> 4);
#pragma unroll
  for (int s = 0; s < DecTile<D>::KB; ++s) {
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kr + 32 * s));
    t.k[s] = __builtin_bit_cast(bf16x8, x);
  }
#pragma unroll
  for (int i = 0; i < DecTile<D>::VI; ++i)
    t.v[i] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(V + (int64_t)min((uint32_t)r.v[i], rmax) * D + 8 * (lane % VL)));
  t.lr = BIAS ? lr[rk] : 0.f;
}

// partial layout as decode_partial: [lc, Hq, nchunk] x (m, l, -, -, o[d]), m in natural
// log units.  `nw` = lc * Hkv * nchunk waves in all.
// Max over the 16 lanes of a DPP row (quad swaps, then half-row and row mirrors).
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}

template <int D, bool BIAS, bool IDX>
__global__ void __launch_bounds__(NT)
decode_mfma(DecTables t, int Hq, int Hkv, int G, int64_t len, float sl2, float bl2, int nchunk,
            int64_t ckm, int64_t nw, float* __restrict__ part) {
  constexpr int KB = DecTile<D>::KB, VL = DecTile<D>::VL, VI = DecTile<D>::VI, KPI = 64 / VL;
  __shared__ f32x4 sp[NT / 64][16];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t wid = (int64_t)blockIdx.x * (NT / 64) + wv;
  if (wid >= nw) return;
  const int ch = (int)(wid % nchunk);
  const int g = (int)((wid / nchunk) % Hkv);
  const int l = (int)(wid / ((int64_t)nchunk * Hkv));
  const uint16_t* q = (const uint16_t*)t.q.p[l];
  const uint16_t* K = (const uint16_t*)t.K.p[l] + (int64_t)g * len * D;
  const uint16_t* V = (const uint16_t*)t.V.p[l] + (int64_t)g * len * D;
  const float* lr = BIAS ? (const float*)t.logR.p[l] + (int64_t)g * len : nullptr;
  const int32_t* ix = IDX ? (const int32_t*)t.ix.p[l] + (int64_t)g * t.npos : nullptr;

  // A operand: row c = lane % 16 holds query head c % 4 (zero if that head is >= G)
  bf16x8 qa[KB];
  {
    const int h = (lane & 15) & 3;
    const unsigned keep = h < G ? ~0u : 0u;
    const uint16_t* qr = q + (int64_t)(g * G + (h < G ? h : 0)) * D + 8 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < KB; ++s) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qr + 32 * s);
      x &= keep;
      qa[s] = __builtin_bit_cast(bf16x8, x);
    }
  }
  const int64_t j0 = (int64_t)ch * ckm, j1 = min(t.npos, j0 + ckm), jlast = j1 - 1;
  const uint32_t rmax = (uint32_t)(len - 1);
  const int ntile = (int)((j1 - j0 + 15) / 16);
  float m[4], ls[4], o[4][8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    m[e] = -INFINITY; ls[e] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[e][i] = 0.f;
  }
  // one tile: logits on the matrix core, online softmax, P V on the vector ALU
  auto tile = [&](const DecTile<D>& c, int64_t jb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KB; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], c.k[s], acc, 0, 0, 0);
    // this lane: key jb + lane % 16, head e in acc[e]
    const bool valid = jb + (lane & 15) <= jlast;
    const float b = BIAS ? bl2 * c.lr : 0.f;
    // The reference max m moves only when a logit exceeds it by more than
    // kLazy (base 2), so probabilities stay below 2^kLazy and the accumulators
    // are rescaled on few tiles (always on the first, where m = -inf).  The tile
    // max is the same in all four rows of 16 lanes, so the branch is uniform.
    float x[4], tm[4];
    bool grow = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = valid ? acc[e] * sl2 + b : -INFINITY;
      tm[e] = row16_max(x[e]);                          // finite: a tile holds a valid key
      grow |= tm[e] > m[e] + kLazy;
    }
    if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float mn = fmaxf(m[e], tm[e]);
        const float al = __builtin_amdgcn_exp2f(m[e] - mn);   // 0 when m = -inf
        m[e] = mn;
        ls[e] *= al;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[e][i] *= al;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // v_exp_f32 without the denormal path: a probability below 2^-126 of the
      // largest is flushed to 0
      x[e] = __builtin_amdgcn_exp2f(x[e] - m[e]);
      ls[e] += x[e];
    }
    if (lane < 16) sp[wv][lane] = f32x4{x[0], x[1], x[2], x[3]};
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const f32x4 p = sp[wv][i * KPI + lane / VL];
      float v[8];
#pragma unroll
      for (int u = 0; u < 4; ++u) { v[2 * u] = bf16_lo(c.v[i][u]); v[2 * u + 1] = bf16_hi(c.v[i][u]); }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int u = 0; u < 8; ++u) o[e][u] += p[e] * v[u];
    }
    // the products are complete here: nothing of this tile is sunk below the
    // refill of its register set (which would rename the set)
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int u = 0; u < 8; ++u) asm volatile("" : "+v"(o[e][u]));
    asm volatile("" ::: "memory");
  };
  // tiles from a ring of kSets register sets, kSets - 1 tiles' loads always in
  // flight.  Loads past the chunk's last tile are clamped to it (a re-read of rows
  // just fetched); a tile past the end is fully masked and changes nothing.
  // The rows of tile T + kSets are found (with IDX: their indices loaded) while
  // tile T is computed, one step before that tile's K/V loads are issued: the
  // wait for the indices then does not include the K/V loads in flight, which
  // complete in order behind them.
  const int64_t jl = j0 + (int64_t)(ntile - 1) * 16;      // the last tile
  DecTile<D> ts[kSets];
  DecRows<D> rs[kSets];
#pragma unroll
  for (int u = 0; u < kSets; ++u) dec_rows<D, IDX>(rs[u], ix, min(j0 + 16 * u, jl), jlast, lane);
#pragma unroll
  for (int u = 0; u + 1 < kSets; ++u) dec_load<D, BIAS>(ts[u], K, V, lr, rs[u], rmax, lane);
  for (int ti = 0; ti < ntile; ti += kSets) {
    const int64_t jb = j0 + (int64_t)ti * 16;
#pragma unroll
    for (int u = 0; u < kSets; ++u) {
      // the scheduling barrier keeps each refill below the last use of the set it
      // overwrites (otherwise the sets are renamed and copied, with a wait per copy)
      __builtin_amdgcn_sched_barrier(0);
      dec_rows<D, IDX>(rs[u], ix, min(jb + 16 * (u + kSets), jl), jlast, lane);
      dec_load<D, BIAS>(ts[(u + kSets - 1) % kSets], K, V, lr, rs[(u + kSets - 1) % kSets], rmax, lane);
      asm volatile("" ::: "memory");
      tile(ts[u], jb + 16 * u);
    }
  }
  // sum of exp per head over the 16 key lanes; output over the lanes sharing a d-slice
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ls[e] += __shfl_xor(ls[e], 1, 64);
    ls[e] += __shfl_xor(ls[e], 2, 64);
    ls[e] += __shfl_xor(ls[e], 4, 64);
    ls[e] += __shfl_xor(ls[e], 8, 64);
#pragma unroll
    for (int off = VL; off < 64; off <<= 1)
#pragma unroll
      for (int i = 0; i < 8; ++i) o[e][i] += __shfl_xor(o[e][i], off, 64);
  }
  if (lane < VL) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (e >= G) break;
      float* p = part + (((int64_t)l * Hq + g * G + e) * nchunk + ch) * (D + 4);
      if (lane == 0) { p[0] = m[e] * LN2; p[1] = ls[e]; }
      *reinterpret_cast<float4*>(p + 4 + 8 * lane) = make_float4(o[e][0], o[e][1], o[e][2], o[e][3]);
      *reinterpret_cast<float4*>(p + 8 + 8 * lane) = make_float4(o[e][4], o[e][5], o[e][6], o[e][7]);
    }
  }
}

// ---- active set of a decode step ([RECAS] section 2.C) -------------------------
// score[l, g, j] = max over the group's query heads of scale * <q_h, k_j>
//                  (+ beta * u[l][g, j] when a utility row is given)
// One wave per chunk of keys, 16-key tiles of K in the MFMA B layout (as in
// decode_mfma, without V), logits on v_mfma_f32_16x16x32_bf16.  UT: a utility row
// is given; its value for a key is loaded with the key's tile (a load issued at
// the store would make the in-order wait include the next tile's K loads).
template <int D, bool UT>
__global__ void __launch_bounds__(NT)
active_scores_mfma(DecTables t, int Hkv, int G, int64_t len, float scale, float beta,
                   int nchunk, int64_t ckm, int64_t nw, float* __restrict__ score) {
  constexpr int KB = D / 32;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t wid = (int64_t)blockIdx.x * (NT / 64) + wv;
  if (wid >= nw) return;
  const int ch = (int)(wid % nchunk);
  const int g = (int)((wid / nchunk) % Hkv);
  const int l = (int)(wid / ((int64_t)nchunk * Hkv));
  const uint16_t* q = (const uint16_t*)t.q.p[l];
  const uint16_t* K = (const uint16_t*)t.K.p[l] + (int64_t)g * len * D;
  const float* u = (const float*)t.logR.p[l];          // utility rows, or null
  if (u) u += (int64_t)g * len;
  float* out = score + ((int64_t)l * Hkv + g) * len;
  bf16x8 qa[KB];
  {
    const int h = (lane & 15) & 3;
    const unsigned keep = h < G ? ~0u : 0u;
    const uint16_t* qr = q + (int64_t)(g * G + (h < G ? h : 0)) * D + 8 * (lane >> 4);
#pragma unroll
    for (int s2 = 0; s2 < KB; ++s2) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qr + 32 * s2);
      x &= keep;
      qa[s2] = __builtin_bit_cast(bf16x8, x);
    }
  }
  const int64_t j0 = (int64_t)ch * ckm, j1 = min(len, j0 + ckm), jlast = j1 - 1;
  const int ntile = (int)((j1 - j0 + 15) / 16);
  auto load = [&](bf16x8 (&kt)[KB], float& uv, int64_t jb) __attribute__((always_inline)) {
    const int64_t kk = min(jb + (lane & 15), jlast);
    const uint16_t* kr = K + kk * D + 8 * (lane >> 4);
#pragma unroll
    for (int s2 = 0; s2 < KB; ++s2)
      kt[s2] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kr + 32 * s2)));
    if constexpr (UT) uv = __builtin_nontemporal_load(u + kk);
  };
  auto tile = [&](const bf16x8 (&kt)[KB], float uv, int64_t jb) __attribute__((always_inline)) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < KB; ++s2) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s2], kt[s2], acc, 0, 0, 0);
    float m = acc[0];
#pragma unroll
    for (int e = 1; e < 4; ++e) m = e < G ? fmaxf(m, acc[e]) : m;
    const int64_t j = jb + (lane & 15);
    if (lane < 16 && j <= jlast) out[j] = m * scale + (UT ? beta * uv : 0.f);
  };
  // a ring of kScoreSets register sets, kScoreSets - 1 tiles' loads in flight; loads
  // past the chunk's last tile are clamped to it, and a tile past the end is not stored
  const int64_t jl = j0 + (int64_t)(ntile - 1) * 16;
  bf16x8 kt[kScoreSets][KB];
  float ut[kScoreSets] = {};
#pragma unroll
  for (int v = 0; v + 1 < kScoreSets; ++v) load(kt[v], ut[v], min(j0 + 16 * v, jl));
  for (int ti = 0; ti < ntile; ti += kScoreSets) {
    const int64_t jb = j0 + (int64_t)ti * 16;
#pragma unroll
    for (int v = 0; v < kScoreSets; ++v) {
      __builtin_amdgcn_sched_barrier(0);
      load(kt[(v + kScoreSets - 1) % kScoreSets], ut[(v + kScoreSets - 1) % kScoreSets],
           min(jb + 16 * (v + kScoreSets - 1), jl));
      asm volatile("" ::: "memory");
      if (jb + 16 * v <= jlast) tile(kt[v], ut[v], jb + 16 * v);
    }
  }
}

// General path (float32, other d, G up to 8): one thread per key.
template <typename T>
__global__ void __launch_bounds__(NT)
active_scores_any(DecTables t, int Hkv, int G, int64_t len, int d, float scale, float beta,
                  float* __restrict__ score) {
  const int64_t row = blockIdx.y;                      // (layer, KV head)
  const int l = (int)(row / Hkv), g = (int)(row % Hkv);
  const int64_t j = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (j >= len) return;
  const T* q = (const T*)t.q.p[l];
  const T* k = (const T*)t.K.p[l] + ((int64_t)g * len + j) * d;
  float m = -INFINITY;
  for (int h = 0; h < G; ++h) {
    const T* qh = q + (int64_t)(g * G + h) * d;
    float acc = 0.f;
    for (int e = 0; e < d; ++e) acc += elem_f32(qh[e]) * elem_f32(k[e]);
    m = fmaxf(m, acc);
  }
  const float* u = (const float*)t.logR.p[l];
  score[row * len + j] = m * scale + (u ? beta * u[(int64_t)g * len + j] : 0.f);
}

__global__ void decode_combine(const float* __restrict__ part, int nchunk, int d, int64_t nhead,
                               float* __restrict__ o, float* __restrict__ lse) {
  const int64_t hh = blockIdx.x;                 // (layer, query head)
  if (hh >= nhead) return;
  const float* p = part + hh * nchunk * (d + 4);
  float M = -INFINITY;
  for (int c = 0; c < nchunk; ++c) M = fmaxf(M, p[(int64_t)c * (d + 4)]);
  float S = 0.f;
  for (int c = 0; c < nchunk; ++c) {
    const float* pc = p + (int64_t)c * (d + 4);
    S += pc[1] * (M > -INFINITY ? expf(pc[0] - M) : 0.f);
  }
  for (int e = threadIdx.x; e < d; e += blockDim.x) {
    float O = 0.f;
    for (int c = 0; c < nchunk; ++c) {
      const float* pc = p + (int64_t)c * (d + 4);
      O += pc[4 + e] * (M > -INFINITY ? expf(pc[0] - M) : 0.f);
    }
    o[hh * d + e] = O / S;
  }
  if (lse && threadIdx.x == 0) lse[hh] = M + logf(S);
}

// decode_mfma's chunks per (layer, KV head): about kWaveTarget waves in all,
// at least 32 keys each.  The chunk length is then ceil(len / nchunk) rounded up
// to whole rings of kSets tiles.
int64_t mfma_chunks(int lc, int Hkv, int64_t len, int target = kWaveTarget) {
  const int64_t per = (target + (int64_t)lc * Hkv - 1) / ((int64_t)lc * Hkv);
  return max((int64_t)1, min(per, (len + 31) / 32));
}
int64_t mfma_chunk_len(int64_t len, int64_t nchunk) {
  constexpr int q = 16 * kSets;
  return ((len + nchunk - 1) / nchunk + q - 1) / q * q;
}

template <typename T, int LG>
void launch_g(int G, dim3 grid, hipStream_t s, const DecTables& t, int Hq, int Hkv, int64_t len,
              int d, float scale, float ab, int nchunk, float* part) {
#define KVC_D(GG) hipLaunchKernelGGL((decode_partial<T, LG, GG>), grid, dim3(NT), 0, s, t, Hq, Hkv, len, d, scale, ab, nchunk, part)
  switch (G) {
    case 1: KVC_D(1); break;
    case 2: KVC_D(2); break;
    case 3: KVC_D(3); break;
    case 4: KVC_D(4); break;
    case 5: KVC_D(5); break;
    case 6: KVC_D(6); break;
    case 7: KVC_D(7); break;
    default: KVC_D(8); break;
  }
#undef KVC_D
}

template <typename T>
void launch_dec(int LG, int G, dim3 grid, hipStream_t s, const DecTables& t, int Hq, int Hkv,
                int64_t len, int d, float scale, float ab, int nchunk, float* part) {
  switch (LG) {
    case 4: launch_g<T, 4>(G, grid, s, t, Hq, Hkv, len, d, scale, ab, nchunk, part); break;
    case 8: launch_g<T, 8>(G, grid, s, t, Hq, Hkv, len, d, scale, ab, nchunk, part); break;
    case 16: launch_g<T, 16>(G, grid, s, t, Hq, Hkv, len, d, scale, ab, nchunk, part); break;
    default: launch_g<T, 32>(G, grid, s, t, Hq, Hkv, len, d, scale, ab, nchunk, part); break;
  }
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" size_t kvc_decode_attn_workspace_size(int L, int Hq, int64_t len, int d) {
  if (L < 1 || Hq < 1 || len < 1 || d < 1) return 0;
  // partials of one launch (at most kLayersPerLaunch layers), for either kernel and
  // any Hkv >= 1; the last launch of L layers may cover fewer layers
  auto launch_bytes = [&](int lc) {
    const int64_t nchunk = max((len + CK - 1) / CK, mfma_chunks(lc, 1, len));
    return (size_t)lc * Hq * nchunk * (d + 4) * sizeof(float);
  };
  const int lc = L < kLayersPerLaunch ? L : kLayersPerLaunch;
  const int rest = L % kLayersPerLaunch;
  return max(launch_bytes(lc), rest ? launch_bytes(rest) : (size_t)0) + 256;
}

namespace {

int decode_impl(const char* fn, const void* const* q, const void* const* K, const void* const* V,
                int dtype, const float* const* logR, float alpha_bias, const int32_t* const* ix,
                int64_t npos, int L, int Hq, int Hkv, int64_t len, int d, float scale, float* o_out,
                float* lse_out, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  if (!dtype_ok(dtype)) return KVC_FAIL(KVC_ERR_DTYPE, "%s: dtype %d", fn, dtype);
  KVC_REQUIRE(L >= 1 && L <= KVC_MAX_LAYERS, "%s: need 1 <= L <= %d", fn, KVC_MAX_LAYERS);
  KVC_REQUIRE(Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0, "%s: need Hq %% Hkv == 0", fn);
  KVC_REQUIRE(Hq / Hkv <= MAXG, "%s: more than %d query heads per KV head", fn, MAXG);
  KVC_REQUIRE(len >= 1 && len <= 0x7fffffffLL, "%s: need 1 <= len < 2^31", fn);
  KVC_REQUIRE(q && K && V && o_out, "%s: null pointer", fn);
  KVC_REQUIRE(std::isfinite(scale) && std::isfinite(alpha_bias), "%s: scale and alpha_bias must be finite", fn);
  const int rb = d * dtype_size(dtype);
  KVC_REQUIRE(d <= 256 && rb % 16 == 0 && (rb / 16 == 4 || rb / 16 == 8 || rb / 16 == 16 || rb / 16 == 32),
              "%s: need d * elsize in {64, 128, 256, 512} bytes and d <= 256", fn);
  const int LG = rb / 16;
  for (int l = 0; l < L; ++l) {
    KVC_REQUIRE(q[l] && K[l] && V[l], "%s: null pointer in layer %d", fn, l);
    KVC_REQUIRE((uintptr_t)q[l] % 16 == 0 && (uintptr_t)K[l] % 16 == 0 && (uintptr_t)V[l] % 16 == 0,
                "%s: layer %d tensors not 16-byte aligned", fn, l);
    KVC_REQUIRE(!logR || logR[l], "%s: logR[%d] is null", fn, l);
    KVC_REQUIRE(!ix || ix[l], "%s: active index list of layer %d is null", fn, l);
  }
  KVC_REQUIRE(npos >= 1 && npos <= len, "%s: need 1 <= positions <= len", fn);
  const size_t need = kvc_decode_attn_workspace_size(L, Hq, len, d);
  if (!ws || ws_bytes < need)
    return KVC_FAIL(KVC_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  float* part = (float*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
  hipStream_t s = as_stream(stream);
  const int G = Hq / Hkv;
  const bool mfma = dtype == KVC_BF16 && G <= 4 && (d == 64 || d == 128);
  const int nchunk_g = (int)((npos + CK - 1) / CK);
  for (int l0 = 0; l0 < L; l0 += kLayersPerLaunch) {
    const int lc = min(kLayersPerLaunch, L - l0);
    DecTables t{};
    for (int i = 0; i < lc; ++i) {
      t.q.p[i] = q[l0 + i]; t.K.p[i] = K[l0 + i]; t.V.p[i] = V[l0 + i];
      t.logR.p[i] = logR ? logR[l0 + i] : nullptr;
      t.ix.p[i] = ix ? ix[l0 + i] : nullptr;
    }
    t.npos = npos;
    int nchunk = nchunk_g;
    if (mfma) {
      const int64_t ckm = mfma_chunk_len(npos, mfma_chunks(lc, Hkv, npos));
      nchunk = (int)((npos + ckm - 1) / ckm);
      const int64_t nw = (int64_t)lc * Hkv * nchunk;
      const dim3 grid((unsigned)((nw + NT / 64 - 1) / (NT / 64)));
      const float sl2 = scale * LOG2E, bl2 = alpha_bias * LOG2E;
#define KVC_M(DD, BB, II) hipLaunchKernelGGL((decode_mfma<DD, BB, II>), grid, dim3(NT), 0, s, t, Hq, Hkv, G, len, sl2, bl2, nchunk, ckm, nw, part)
      if (ix) {
        if (d == 128) { if (logR) KVC_M(128, true, true); else KVC_M(128, false, true); }
        else { if (logR) KVC_M(64, true, true); else KVC_M(64, false, true); }
      } else {
        if (d == 128) { if (logR) KVC_M(128, true, false); else KVC_M(128, false, false); }
        else { if (logR) KVC_M(64, true, false); else KVC_M(64, false, false); }
      }
#undef KVC_M
    } else {
      const dim3 grid((unsigned)((int64_t)lc * Hkv * nchunk));
      if (dtype == KVC_BF16) launch_dec<uint16_t>(LG, G, grid, s, t, Hq, Hkv, len, d, scale, alpha_bias, nchunk, part);
      else launch_dec<float>(LG, G, grid, s, t, Hq, Hkv, len, d, scale, alpha_bias, nchunk, part);
    }
    const int64_t nhead = (int64_t)lc * Hq;
    hipLaunchKernelGGL(decode_combine, dim3((unsigned)nhead), dim3(128), 0, s, (const float*)part, nchunk,
                       d, nhead, o_out + (int64_t)l0 * Hq * d, lse_out ? lse_out + (int64_t)l0 * Hq : nullptr);
  }
  return launch_status(fn);
}

}  // namespace

extern "C" int kvc_decode_attn(const void* const* q, const void* const* K, const void* const* V,
                               int dtype, const float* const* logR, float alpha_bias, int L, int Hq,
                               int Hkv, int64_t len, int d, float scale, float* o_out, float* lse_out,
                               void* ws, size_t ws_bytes, void* stream) {
  return decode_impl("kvc_decode_attn", q, K, V, dtype, logR, alpha_bias, nullptr, len, L, Hq, Hkv,
                     len, d, scale, o_out, lse_out, ws, ws_bytes, stream);
}

extern "C" int kvc_decode_attn_active(const void* const* q, const void* const* K,
                                      const void* const* V, int dtype, const float* const* logR,
                                      float alpha_bias, const int32_t* const* active,
                                      int64_t k_active, int L, int Hq, int Hkv, int64_t len, int d,
                                      float scale, float* o_out, float* lse_out, void* ws,
                                      size_t ws_bytes, void* stream) {
  if (!active) {
    clear_error();
    return KVC_FAIL(KVC_ERR_ARG, "kvc_decode_attn_active: null active index list");
  }
  return decode_impl("kvc_decode_attn_active", q, K, V, dtype, logR, alpha_bias, active, k_active,
                     L, Hq, Hkv, len, d, scale, o_out, lse_out, ws, ws_bytes, stream);
}


extern "C" int kvc_active_scores(const void* const* q, const void* const* K, int dtype,
                                 const float* const* utility, float beta, int L, int Hq, int Hkv,
                                 int64_t len, int d, float scale, float* score_out, void* stream) {
  clear_error();
  if (!dtype_ok(dtype)) return KVC_FAIL(KVC_ERR_DTYPE, "kvc_active_scores: dtype %d", dtype);
  KVC_REQUIRE(L >= 1 && L <= KVC_MAX_LAYERS, "kvc_active_scores: need 1 <= L <= %d", KVC_MAX_LAYERS);
  KVC_REQUIRE(Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0, "kvc_active_scores: need Hq %% Hkv == 0");
  KVC_REQUIRE(Hq / Hkv <= MAXG, "kvc_active_scores: more than %d query heads per KV head", MAXG);
  KVC_REQUIRE(len >= 1 && len <= 0x7fffffffLL && d >= 1 && d <= 256,
              "kvc_active_scores: need 1 <= len < 2^31 and 1 <= d <= 256");
  KVC_REQUIRE(q && K && score_out, "kvc_active_scores: null pointer");
  // The group maximum is taken over raw dot products and scaled afterwards,
  // which equals the maximum of the scaled ones only for scale > 0.
  KVC_REQUIRE(scale > 0.f && std::isfinite(scale) && std::isfinite(beta),
              "kvc_active_scores: need a finite scale > 0 and a finite beta");
  KVC_REQUIRE((int64_t)L * Hkv <= 65535, "kvc_active_scores: L * Hkv > 65535");
  const int G = Hq / Hkv;
  const bool mfma = dtype == KVC_BF16 && G <= 4 && (d == 64 || d == 128);
  for (int l = 0; l < L; ++l) {
    KVC_REQUIRE(q[l] && K[l], "kvc_active_scores: null pointer in layer %d", l);
    KVC_REQUIRE(!utility || utility[l], "kvc_active_scores: utility[%d] is null", l);
    KVC_REQUIRE(!mfma || ((uintptr_t)q[l] % 16 == 0 && (uintptr_t)K[l] % 16 == 0),
                "kvc_active_scores: layer %d tensors not 16-byte aligned", l);
  }
  hipStream_t s = as_stream(stream);
  for (int l0 = 0; l0 < L; l0 += kLayersPerLaunch) {
    const int lc = min(kLayersPerLaunch, L - l0);
    DecTables t{};
    for (int i = 0; i < lc; ++i) {
      t.q.p[i] = q[l0 + i]; t.K.p[i] = K[l0 + i];
      t.logR.p[i] = utility ? utility[l0 + i] : nullptr;
    }
    float* out = score_out + (int64_t)l0 * Hkv * len;
    if (mfma) {
      const int64_t ckm = mfma_chunk_len(len, mfma_chunks(lc, Hkv, len, kScoreWaves));
      const int nchunk = (int)((len + ckm - 1) / ckm);
      const int64_t nw = (int64_t)lc * Hkv * nchunk;
      const dim3 grid((unsigned)((nw + NT / 64 - 1) / (NT / 64)));
#define KVC_AS(DD, UU) hipLaunchKernelGGL((active_scores_mfma<DD, UU>), grid, dim3(NT), 0, s, t, Hkv, G, len, \
                                         scale, beta, nchunk, ckm, nw, out)
      if (d == 128) { if (utility) KVC_AS(128, true); else KVC_AS(128, false); }
      else { if (utility) KVC_AS(64, true); else KVC_AS(64, false); }
#undef KVC_AS
    } else {
      const dim3 grid((unsigned)((len + NT - 1) / NT), (unsigned)(lc * Hkv));
      if (dtype == KVC_BF16) hipLaunchKernelGGL(active_scores_any<uint16_t>, grid, dim3(NT), 0, s, t, Hkv, G, len, d, scale, beta, out);
      else hipLaunchKernelGGL(active_scores_any<float>, grid, dim3(NT), 0, s, t, Hkv, G, len, d, scale, beta, out);
    }
  }
  return launch_status("kvc_active_scores");
}
