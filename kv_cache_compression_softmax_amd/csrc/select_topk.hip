// Per-(layer, KV head) retention: the last w tokens plus the k - w highest scores
// of the rest, ties to the lower index, indices written in ascending order.
//
// [InfoKV] Method and Technical detail: each layer keeps its top-k_l tokens by the
// fused score.  [SelKV] section 2, pipeline step 2: the same selection on the
// VATP union keeps the top tokens plus the recent window.
//
// One workgroup per (layer, KV head):
//   1. radix select on order-preserving 32-bit keys of the float32 scores (four
//      8-bit digits, LDS histograms) finds T, the (k - w)-th largest key of
//      [0, n - w), and cgt = the number of keys above it;
//   2. one ordered pass over [0, n - w) keeps every key > T and the first
//      k - w - cgt keys == T in index order.  Output positions come from a block
//      scan of (count > T, count == T) per thread, so the indices come out
//      ascending and the result is exact and deterministic.
// Each thread keeps several loads in flight; with rows a multiple of 4 floats long
// they are 16-byte loads, since a lone workgroup per CU is bound by the bytes it
// has in flight, not by the histogram work.  When [0, n - w) fits in LDS beside
// the histograms, the first pass copies it there and the other four passes read
// it from LDS, so the row comes from memory once.  A longer row of up to
// REGV * 512 vectors of 4 scores (102400 scores) is held in registers instead,
// by a 512-thread workgroup: thread t keeps vectors t, t + 512, ..., which is
// also the vector it needs in
// each chunk of the ordered pass, so again the row is read once (all of a
// thread's loads in flight together).  Longer rows still are re-read by every
// pass.  The histograms are per wave, with wave-aggregated increments where
// lanes crowd into one bin.
#include "common.h"

namespace kvc {
namespace {

constexpr int NT = 1024;
constexpr int NW = NT / 64;     // waves
constexpr int EPT = 4;          // consecutive elements per thread in the output pass
constexpr int HU = 8;           // elements per thread loaded together in a histogram pass
constexpr int NTR = 512;        // threads of the register path (2 waves per SIMD)
constexpr int REGV = 50;        // 16-byte vectors per thread held in registers (register path)

// Adds 1 to hist[bin] for every active lane with valid set.  When many lanes share
// the first valid lane's bin (scores spread over few binades make the high digits
// crowd into a few bins) the wave counts each distinct bin with a ballot and one
// lane adds the count; otherwise every lane adds its own 1.
__device__ __forceinline__ void hist_add(int* hist, bool valid, int bin) {
  uint64_t act = __ballot(valid);
  if (act == 0) return;
  const int b0 = __builtin_amdgcn_readlane(bin, __builtin_ctzll(act));
  if (__builtin_popcountll(__ballot(valid && bin == b0)) < 16) {
    if (valid) atomicAdd(&hist[bin], 1);
    return;
  }
  const int lane = threadIdx.x & 63;
  while (act) {                                   // one round per distinct bin
    const int lead = __builtin_ctzll(act);
    const int b = __builtin_amdgcn_readlane(bin, lead);
    const uint64_t same = __ballot(valid && bin == b);
    if (lane == lead) atomicAdd(&hist[b], __builtin_popcountll(same));
    act &= ~same;
  }
}

// VEC: 16-byte loads (n % 4 == 0, S 16-byte aligned).  CACHE: [0, n - w) is held in
// dynamic LDS, as float4, from the first pass on.
template <bool VEC, bool CACHE>
__global__ void __launch_bounds__(NT)
select_kernel(const float* __restrict__ S, int Hkv, int64_t n, I64s kk, int w, MutPtrs idx) {
  constexpr int NTB = NT;
  constexpr int NWB = NTB / 64;
  extern __shared__ float4 rc[];
  __shared__ int hist[NWB][256];                   // one histogram per wave
  __shared__ int scan[NTB / 64];
  __shared__ int pick[2];
  const int tid = threadIdx.x;
  const int wv = tid / 64;
  const int l = blockIdx.x / Hkv, g = blockIdx.x % Hkv;
  const int64_t k = kk.v[l];
  const float* row = S + ((int64_t)l * Hkv + g) * n;
  int32_t* out = (int32_t*)idx.p[l] + (int64_t)g * k;
  if (k <= w) {                                   // the window alone overflows the budget
    for (int64_t j = tid; j < k; j += NTB) out[j] = (int32_t)(n - k + j);
    return;
  }
  const int64_t nb = n - w, need = k - w;
  for (int64_t j = tid; j < w; j += NTB) out[need + j] = (int32_t)(nb + j);
  if (need >= nb) {                               // everything is kept
    for (int64_t j = tid; j < nb; j += NTB) out[j] = (int32_t)j;
    return;
  }
  // ---- 1. radix select of the need-th largest key
  uint32_t prefix = 0;
  int64_t above = 0, rem = need;
#pragma unroll 1
  for (int p = 3; p >= 0; --p) {
    const int shift = 8 * p;
    const uint32_t hi_mask = (p == 3) ? 0u : (uint32_t)(~0ull << (shift + 8));
    for (int i = tid; i < NWB * 256; i += NTB) (&hist[0][0])[i] = 0;
    __syncthreads();
    auto count = [&](uint32_t key, bool in) __attribute__((always_inline)) {
      hist_add(hist[wv], in && (key & hi_mask) == (prefix & hi_mask), (int)((key >> shift) & 255));
    };
    if constexpr (VEC) {
      // vectors [0, nv) of 4 scores; the last may reach past nb but not past n
      const int64_t nv = (nb + 3) / 4;
      const float4* row4 = reinterpret_cast<const float4*>(row);
      const bool lds = CACHE && p != 3;
#pragma unroll 1
      for (int64_t i0 = 0; i0 < nv; i0 += (int64_t)NTB * HU) {
        float4 v[HU];                             // HU 16-byte loads in flight per thread
        if (lds) {
#pragma unroll
          for (int u = 0; u < HU; ++u) v[u] = rc[min(i0 + (int64_t)u * NTB + tid, nv - 1)];
        } else {
#pragma unroll
          for (int u = 0; u < HU; ++u) v[u] = row4[min(i0 + (int64_t)u * NTB + tid, nv - 1)];
          if (CACHE) {
#pragma unroll
            for (int u = 0; u < HU; ++u)
              if (i0 + (int64_t)u * NTB + tid < nv) rc[i0 + (int64_t)u * NTB + tid] = v[u];
          }
        }
#pragma unroll
        for (int u = 0; u < HU; ++u) {
          const int64_t e0 = 4 * (i0 + (int64_t)u * NTB + tid);
          count(f32_key(v[u].x), e0 < nb);
          count(f32_key(v[u].y), e0 + 1 < nb);
          count(f32_key(v[u].z), e0 + 2 < nb);
          count(f32_key(v[u].w), e0 + 3 < nb);
        }
      }
    } else {
#pragma unroll 1
      for (int64_t i0 = 0; i0 < nb; i0 += (int64_t)NTB * HU) {
        float v[HU];                              // HU loads in flight per thread
#pragma unroll
        for (int u = 0; u < HU; ++u) v[u] = row[min(i0 + (int64_t)u * NTB + tid, nb - 1)];
#pragma unroll
        for (int u = 0; u < HU; ++u) count(f32_key(v[u]), i0 + (int64_t)u * NTB + tid < nb);
      }
    }
    __syncthreads();
    int c = 0;
    if (tid < 256) {
#pragma unroll
      for (int x = 0; x < NWB; ++x) c += hist[x][255 - tid];
    }
    int tot;
    const int incl = block_exclusive_scan<NTB>(c, scan, &tot) + c;
    if (tid < 256 && incl >= rem && incl - c < rem) { pick[0] = 255 - tid; pick[1] = incl - c; }
    __syncthreads();
    prefix |= (uint32_t)pick[0] << shift;
    above += pick[1];
    rem -= pick[1];
    __syncthreads();
  }
  const uint32_t T = prefix;
  const int64_t take_eq = need - above;           // >= 1 copies of T are kept
  // ---- 2. ordered output of [0, nb); the next chunk's scores are requested
  // before this chunk's block scan
  int64_t run_gt = 0, run_eq = 0;
  float cur[EPT];
  static_assert(EPT == 4, "one float4 per thread and chunk");
  auto fetch = [&](int64_t c0, float (&v)[EPT]) __attribute__((always_inline)) {
    const int64_t i0 = c0 + (int64_t)tid * EPT;
    if constexpr (VEC) {
      const int64_t vi = min(i0 / 4, (nb - 1) / 4);
      const float4 f = CACHE ? rc[vi] : reinterpret_cast<const float4*>(row)[vi];
      v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    } else {
#pragma unroll
      for (int e = 0; e < EPT; ++e) v[e] = row[min(i0 + e, nb - 1)];
    }
  };
  fetch(0, cur);
#pragma unroll 1
  for (int64_t c0 = 0; c0 < nb; c0 += (int64_t)NTB * EPT) {
    const int64_t i0 = c0 + (int64_t)tid * EPT;
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const uint32_t key = f32_key(cur[e]);
      const bool in = i0 + e < nb;
      gt |= (uint32_t)(in && key > T) << e;
      eq |= (uint32_t)(in && key == T) << e;
    }
    fetch(min(c0 + (int64_t)NTB * EPT, nb - 1), cur);
    const int packed = __builtin_popcount(gt) | (__builtin_popcount(eq) << 16);
    int tot;
    const int ex = block_exclusive_scan<NTB>(packed, scan, &tot);
    int64_t gtb = run_gt + (ex & 0xffff), eqb = run_eq + (ex >> 16);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      if (gt & (1u << e)) {
        out[gtb + min(eqb, take_eq)] = (int32_t)(i0 + e);
        ++gtb;
      } else if (eq & (1u << e)) {
        if (eqb < take_eq) out[gtb + eqb] = (int32_t)(i0 + e);
        ++eqb;
      }
    }
    run_gt += tot & 0xffff;
    run_eq += tot >> 16;
  }
}

// ---------------------------------------------------------------- register path
// A row of up to REGV * NTR vectors of 4 scores (102400 scores) is held in
// registers, as order-preserving keys, by a workgroup of NTR threads: thread t
// keeps vectors t, t + NTR, ..., all loads in flight together, so the row is read
// once.
//   1. The row's smallest and largest keys bound the search.  Each pass cuts
//      the current key range [lo, lo + 2^sp) into at most 256 bins of width
//      2^(sp-8), so scores spread over a few binades fill many bins (digits of
//      the raw key would put a whole binade into one or two).  The bin holding
//      the need-th largest key becomes the next range; keys outside the range
//      were counted by earlier passes and are not counted again.
//   2. After the first pass the keys of the chosen bin (when at most CAND) are
//      copied to an LDS list, and the remaining passes read the list only.
//   3. Ordered output: chunk r of the row is vector r * NTR + t of thread t.
//      Per chunk and element, each wave's counts and lane prefixes come from
//      ballots (popcounts and mbcnts); the chunk and wave offsets come from one
//      table in LDS, so the whole output takes two barriers.
constexpr int NWR = NTR / 64;   // waves of the register path
constexpr int CAND = 8192;      // candidate keys copied to LDS after the first pass

__global__ void __launch_bounds__(NTR)
select_reg_kernel(const float* __restrict__ S, int Hkv, int64_t n, I64s kk, int w, MutPtrs idx) {
  __shared__ int hist[NWR][256];                   // one histogram per wave
  __shared__ uint32_t cand[CAND];
  __shared__ uint32_t red[2][NWR];
  __shared__ int wtot[REGV][NWR];                  // per chunk and wave: gt | eq << 16
  __shared__ int wpre[REGV][NWR];                  // exclusive prefix over waves, packed
  __shared__ int cbase[REGV][2];                   // exclusive prefix over chunks (gt, eq)
  __shared__ int scan[NWR];
  __shared__ int pick[3];
  __shared__ int wcnt[NWR];                        // candidates of each wave's list segment
  __shared__ int flag[2];                          // crowded bins seen; a list segment overflowed
  const int tid = threadIdx.x, lane = tid & 63, wv = tid / 64;
  const int l = blockIdx.x / Hkv, g = blockIdx.x % Hkv;
  const int64_t k = kk.v[l];
  const float* row = S + ((int64_t)l * Hkv + g) * n;
  int32_t* out = (int32_t*)idx.p[l] + (int64_t)g * k;
  if (k <= w) {                                   // the window alone overflows the budget
    for (int64_t j = tid; j < k; j += NTR) out[j] = (int32_t)(n - k + j);
    return;
  }
  const int nb = (int)(n - w), need = (int)(k - w);  // n < 2^31
  for (int j = tid; j < w; j += NTR) out[need + j] = nb + j;
  if (need >= nb) {                               // everything is kept
    for (int j = tid; j < nb; j += NTR) out[j] = j;
    return;
  }
  // the thread's vectors t + r NTR, loaded once (vectors past the row repeat its
  // last one and are never counted); element 4 (r NTR + t) + e is in the row iff
  // 4 r NTR + e < lim
  uint4 rk[REGV];
  const int lim = nb - 4 * tid;
  uint32_t kmin = ~0u, kmax = 0u;                 // the row's key range, formed as the keys arrive
  {
    const int nv = (nb + 3) / 4;
    const float4* row4 = reinterpret_cast<const float4*>(row);
    float4 t[REGV];
#pragma unroll
    for (int r = 0; r < REGV; ++r) t[r] = row4[min(r * NTR + tid, nv - 1)];
#pragma unroll
    for (int r = 0; r < REGV; ++r) {
      rk[r] = make_uint4(f32_key(t[r].x), f32_key(t[r].y), f32_key(t[r].z), f32_key(t[r].w));
      const uint32_t k4[4] = {rk[r].x, rk[r].y, rk[r].z, rk[r].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * r * NTR + e < lim) { kmin = min(kmin, k4[e]); kmax = max(kmax, k4[e]); }
    }
  }
  // f(key, in the row) for every held key.  The limit is made opaque per call
  // so that the 136 row-membership masks are formed where they are used, not
  // hoisted out of the pass loop and held in scalar registers across it.
  auto each = [&](auto&& f) __attribute__((always_inline)) {
    int lm = lim;
    asm volatile("" : "+v"(lm));
#pragma unroll
    for (int r = 0; r < REGV; ++r) {
      f(rk[r].x, 4 * r * NTR + 0 < lm);
      f(rk[r].y, 4 * r * NTR + 1 < lm);
      f(rk[r].z, 4 * r * NTR + 2 < lm);
      f(rk[r].w, 4 * r * NTR + 3 < lm);
    }
  };
  // ---- 1. the row's key range
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
  }
  if (lane == 0) { red[0][wv] = kmin; red[1][wv] = kmax; }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < NWR; ++x) { kmin = min(kmin, red[0][x]); kmax = max(kmax, red[1][x]); }
  // ---- 2. descent over the range: T = the need-th largest key, above = keys > T
  uint32_t lo = kmin;
  int above = 0, rem = need;
  if (kmax != kmin) {
    int sp = 32 - __builtin_clz(kmax - kmin);   // the range is [lo, lo + 2^sp)
    bool list = false;
#pragma unroll 1
    for (;;) {
      const int s = sp > 8 ? sp - 8 : 0;          // bin width 2^s: at most 256 bins
      const uint32_t dmax = sp >= 32 ? ~0u : (1u << sp) - 1u;
      for (int i = tid; i < NWR * 256; i += NTR) (&hist[0][0])[i] = 0;
      if (tid == 0) flag[0] = 0;
      __syncthreads();
      // keys in [lo, lo + 2^sp): key - lo <= dmax (a key below lo wraps past
      // dmax, except in the first pass, where every key is >= lo); bin
      // (key - lo) >> s, below 256 for every valid key
      auto bin_of = [&](uint32_t key, bool in, bool& valid) __attribute__((always_inline)) {
        const uint32_t d = key - lo;
        valid = in && d <= dmax;
        return (int)(d >> s);
      };
      auto count_agg = [&](uint32_t key, bool in) __attribute__((always_inline)) {
        bool v;
        const int b = bin_of(key, in, v);
        hist_add(hist[wv], v, b);
      };
      if (list) {
        for (int i = tid; i < CAND; i += NTR) count_agg(cand[i], (i & (CAND / NWR - 1)) < wcnt[i / (CAND / NWR)]);
      } else {
        // A sample (two chunks of the row) tells whether many lanes share bins;
        // if not, every lane adds its own 1 (no ballots), else the wave
        // aggregates per bin.
        bool crowd = false;
        int lm = lim;
        asm volatile("" : "+v"(lm));
#pragma unroll
        for (int r = 0; r < REGV; r += REGV / 2) {
          const uint32_t k4[4] = {rk[r].x, rk[r].y, rk[r].z, rk[r].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            bool v;
            const int b = bin_of(k4[e], 4 * r * NTR + e < lm, v);
            const uint64_t act = __ballot(v);
            if (act) {
              const int b0 = __builtin_amdgcn_readlane(b, __builtin_ctzll(act));
              crowd |= __builtin_popcountll(__ballot(v && b == b0)) >= 16;
            }
          }
        }
        if (crowd && lane == 0) flag[0] = 1;
        __syncthreads();
        if (flag[0]) {
          each(count_agg);
        } else {
          each([&](uint32_t key, bool in) {
            bool v;
            const int b = bin_of(key, in, v);
            if (v) atomicAdd(&hist[wv][b], 1);
          });
        }
      }
      __syncthreads();
      int c = 0;
      if (tid < 256) {
#pragma unroll
        for (int x = 0; x < NWR; ++x) c += hist[x][255 - tid];
      }
      int tot;
      const int incl = block_exclusive_scan<NTR>(c, scan, &tot) + c;
      if (tid < 256 && incl >= rem && incl - c < rem) { pick[0] = 255 - tid; pick[1] = incl - c; pick[2] = c; }
      __syncthreads();
      const int b = pick[0], bin_count = pick[2];
      above += pick[1];
      rem -= pick[1];
      lo += (uint32_t)b << s;
      sp = s;
      if (s == 0) break;
      if (!list && bin_count <= CAND) {         // the chosen bin's keys to LDS
        // each wave appends to its own segment of CAND / NWR slots (a running
        // count, no atomics); a segment that would overflow drops the list
        constexpr int SEG = CAND / NWR;
        const uint32_t width = 1u << s;
        int wn = 0;                               // wave-uniform
        if (tid == 0) flag[1] = 0;
        each([&](uint32_t key, bool in) {
          const bool hit = in && key >= lo && key - lo < width;
          const uint64_t m = __ballot(hit);
          if (m) {
            const int at = wn + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (hit && at < SEG) cand[wv * SEG + at] = key;
            wn += __builtin_popcountll(m);
          }
        });
        __syncthreads();                          // flag[1] cleared before any wave sets it
        if (lane == 0) {
          wcnt[wv] = wn;
          if (wn > SEG) flag[1] = 1;
        }
        __syncthreads();
        list = flag[1] == 0;
      }
    }
  }
  const uint32_t T = lo;
  const int teq = need - above;                   // >= 1 copies of T are kept
  // ---- 3. ordered output.  Per chunk and element e, the lanes keeping their
  // element as "> T" or "== T" are compare masks, so the wave totals are
  // popcounts and a lane's prefix is a sum of mbcnts.
  const int nchunk = (nb + 4 * NTR - 1) / (4 * NTR);
  auto masks = [&](int r, bool (&g)[4], bool (&q)[4]) __attribute__((always_inline)) {
    const uint32_t k4[4] = {rk[r].x, rk[r].y, rk[r].z, rk[r].w};
    int lm = lim;
    asm volatile("" : "+v"(lm));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = 4 * r * NTR + e < lm;
      g[e] = in && k4[e] > T;
      q[e] = in && k4[e] == T;
    }
  };
  auto below = [&](uint64_t m) __attribute__((always_inline)) {   // set lanes below this one
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  };
#pragma unroll
  for (int r = 0; r < REGV; ++r) {
    if (r < nchunk) {                             // uniform
      bool g[4], q[4];
      masks(r, g, q);
      int tg = 0, te = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) { tg += __builtin_popcountll(__ballot(g[e])); te += __builtin_popcountll(__ballot(q[e])); }
      if (lane == 0) wtot[r][wv] = tg | (te << 16);
    }
  }
  __syncthreads();
  if (tid < 64) {                                 // wave 0: offsets of chunks and waves
    int cg = 0, ce = 0;
    if (tid < nchunk) {
      int run = 0;
#pragma unroll
      for (int x = 0; x < NWR; ++x) { wpre[tid][x] = run; run += wtot[tid][x]; }
      cg = run & 0xffff;
      ce = run >> 16;
    }
    const int ig = wave_inclusive_scan(cg), ie = wave_inclusive_scan(ce);
    if (tid < nchunk) { cbase[tid][0] = ig - cg; cbase[tid][1] = ie - ce; }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < REGV; ++r) {
    if (r < nchunk) {                             // uniform
      bool g[4], q[4];
      masks(r, g, q);
      const int wp = wpre[r][wv];
      int gtb = cbase[r][0] + (wp & 0xffff), eqb = cbase[r][1] + (wp >> 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) gtb += below(__ballot(g[e]));
      const bool anyq = __ballot(q[0] || q[1] || q[2] || q[3]) != 0;   // rare: copies of T
      if (anyq) {
#pragma unroll
        for (int e = 0; e < 4; ++e) eqb += below(__ballot(q[e]));
      }
      const int i0 = 4 * (r * NTR + tid);
#pragma unroll
      for (int e = 0; e < 4; ++e) {              // positions without branches, one masked store
        const int pos = gtb + min(eqb, teq);      // for "== T" kept: eqb < teq, so pos = gtb + eqb
        const bool keep = g[e] || (q[e] && eqb < teq);
        if (keep) out[pos] = i0 + e;
        gtb += g[e] ? 1 : 0;
        eqb += q[e] ? 1 : 0;
      }
    }
  }
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" int kvc_select_topk(const float* S, int L, int Hkv, int64_t n, const int64_t* k_keep,
                               int w, int32_t* const* idx_out, void* stream) {
  clear_error();
  KVC_REQUIRE(L >= 1 && L <= KVC_MAX_LAYERS, "kvc_select_topk: need 1 <= L <= %d", KVC_MAX_LAYERS);
  KVC_REQUIRE(Hkv >= 1 && n >= 1 && n <= 0x7fffffffLL, "kvc_select_topk: need Hkv >= 1, 1 <= n < 2^31");
  KVC_REQUIRE(w >= 0 && w <= n, "kvc_select_topk: need 0 <= w <= n");
  KVC_REQUIRE(S && k_keep && idx_out, "kvc_select_topk: null pointer");
  for (int l = 0; l < L; ++l) {
    KVC_REQUIRE(k_keep[l] >= 1 && k_keep[l] <= n, "kvc_select_topk: k_keep[%d] outside [1, n]", l);
    KVC_REQUIRE(idx_out[l], "kvc_select_topk: idx_out[%d] is null", l);
  }
  hipStream_t s = as_stream(stream);
  // 16-byte loads need 16-byte rows; the LDS copy of [0, n - w) must fit beside
  // the kernel's own LDS
  const bool vec = n % 4 == 0 && (uintptr_t)S % 16 == 0;
  const size_t cache = (size_t)((n - w + 3) / 4) * sizeof(float4);
  bool use_cache = false;
  if (vec && n > w) {
    int dev = 0, max_lds = 0;
    const void* kern = reinterpret_cast<const void*>(&select_kernel<true, true>);
    hipFuncAttributes fa{};
    use_cache = hipGetDevice(&dev) == hipSuccess &&
                hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess &&
                hipFuncGetAttributes(&fa, kern) == hipSuccess &&
                fa.sharedSizeBytes + cache <= (size_t)max_lds &&
                hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)cache) == hipSuccess;
    if (!use_cache) (void)hipGetLastError();      // a refused query only selects the other path
  }
  // a row too long for LDS but within REGV vectors per thread stays in registers
  const bool use_reg = vec && !use_cache && n > w && (n - w + 3) / 4 <= (int64_t)REGV * NTR;
  for (int l0 = 0; l0 < L; l0 += kLayersPerLaunch) {
    const int lc = min(kLayersPerLaunch, L - l0);
    I64s kk{};
    MutPtrs ip{};
    for (int i = 0; i < lc; ++i) { kk.v[i] = k_keep[l0 + i]; ip.p[i] = idx_out[l0 + i]; }
    const dim3 grid((unsigned)(lc * Hkv));
    const float* Sl = S + (int64_t)l0 * Hkv * n;
    if (use_cache) hipLaunchKernelGGL((select_kernel<true, true>), grid, dim3(NT), cache, s, Sl, Hkv, n, kk, w, ip);
    else if (use_reg) hipLaunchKernelGGL(select_reg_kernel, grid, dim3(NTR), 0, s, Sl, Hkv, n, kk, w, ip);
    else if (vec) hipLaunchKernelGGL((select_kernel<true, false>), grid, dim3(NT), 0, s, Sl, Hkv, n, kk, w, ip);
    else hipLaunchKernelGGL((select_kernel<false, false>), grid, dim3(NT), 0, s, Sl, Hkv, n, kk, w, ip);
  }
  return launch_status("kvc_select_topk");
}
