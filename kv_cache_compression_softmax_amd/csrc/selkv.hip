// SelKV's selective merge path: VATP score with its GQA union, then per-bucket
// routing, soft cosine gate, gated merge and the log-ratio compensation.
//
// [SelKV] section 2.  Pipeline step 1 scores each token by its window attention
// times the norm of its value vector (VATP); step 2 keeps the top tokens (for
// GQA, over the union of the group's heads) plus the recent window; step 3 sends
// every evicted token to a kept token of its positional bucket chosen by prefill
// attention; step 4 weights each evicted value by the soft cosine gate
// g = max(cos, 0) before the attention-weighted merge; step 5 records the ratio R
// of the attention mass the merged entry stands for to the mass of the kept
// token, applied at decode time as a logit bias alpha * ln R.
//
// Both kernels are bound by the V stream.  Rows are read as 16-byte lanes, LG
// lanes per row (LG = row bytes / 16), so a wave covers 64/LG rows per load.
#include <type_traits>

#include "common.h"

namespace kvc {
namespace {

template <typename T> struct El;
template <> struct El<uint16_t> {
  static constexpr int N = 8;
  __device__ static void unpack(const uint4& u, float (&x)[8]) {
    x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
    x[4] = bf16_lo(u.z); x[5] = bf16_hi(u.z); x[6] = bf16_lo(u.w); x[7] = bf16_hi(u.w);
  }
  __device__ static uint4 pack(const float (&x)[8]) {
    uint4 u;
    u.x = f32_to_bf16_rne(x[0]) | ((uint32_t)f32_to_bf16_rne(x[1]) << 16);
    u.y = f32_to_bf16_rne(x[2]) | ((uint32_t)f32_to_bf16_rne(x[3]) << 16);
    u.z = f32_to_bf16_rne(x[4]) | ((uint32_t)f32_to_bf16_rne(x[5]) << 16);
    u.w = f32_to_bf16_rne(x[6]) | ((uint32_t)f32_to_bf16_rne(x[7]) << 16);
    return u;
  }
};
template <> struct El<float> {
  static constexpr int N = 4;
  __device__ static void unpack(const uint4& u, float (&x)[4]) {
    x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
    x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
  }
  __device__ static uint4 pack(const float (&x)[4]) {
    return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                      __float_as_uint(x[3]));
  }
};

// ------------------------------------------------------------- VATP + union
constexpr int NT = 256;         // 4 waves
constexpr int VNL = 8;          // most V loads per lane (all issued before any is used)
constexpr int MAXG = 8;         // query heads per KV head whose A loads are issued up front
// chunks of rows per wave, all requested up front (1.18 ms against 1.25 with one
// chunk per wave, 102400 tokens)
constexpr int CPW = 4;

// One wave per min(VNL, LG) * 64 / LG rows (at most 64) of one (layer, KV head):
// the rows' V are read
// with 16-byte loads (LG lanes per row, non-temporal: the values are not reread
// before the merge pass evicts them), squared norms are reduced per row, then
// lane q takes row q: it reads the group's G attention values of its row
// (coalesced across lanes) and writes U = max_h A_h * |v| and the group mean A_g.
// GM: the attention input is already the group's max over heads ([L, Hkv, n]):
// one value per row, U = A_max * |v| (the same value, since |v| >= 0 and a
// rounded product is monotone in each factor), and no A_g.
template <typename T, int LG, bool GM>
__global__ void __launch_bounds__(NT)
vatp_union_kernel(const float* A_hq, ConstPtrs V, int Hq, int Hkv, int64_t n, int d,
                  int64_t nchunk, int64_t nwave, float* __restrict__ U, float* __restrict__ Ag) {
  constexpr int W = El<T>::N;
  constexpr int RPI = 64 / LG;                  // rows per load instruction
  constexpr int NL = LG < VNL ? LG : VNL;       // loads per lane
  constexpr int RW = RPI * NL;                  // rows per wave (at most 64)
  static_assert(RW <= 64, "one lane per row in the attention phase");
  const int lane = threadIdx.x & 63;
  // wave-uniform (scalar pointer loads); the launch keeps wave counts below 2^31,
  // so the index arithmetic is 32-bit
  const uint32_t wid = blockIdx.x * (NT / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  if (wid >= (uint64_t)nwave) return;           // waves are independent (no barriers)
  const uint32_t ngrp = ((uint32_t)nchunk + CPW - 1) / CPW;   // chunk groups per (layer, head)
  const uint32_t grp = wid % ngrp;
  const int g = (int)((wid / ngrp) % (uint32_t)Hkv);
  const int l = (int)(wid / (ngrp * (uint32_t)Hkv));
  const int G = Hq / Hkv;
  const int rg = lane / LG, c = lane % LG;
  const T* Vg = (const T*)V.p[l] + (int64_t)g * n * d;
  const int q = lane;
  // all loads of the wave's CPW chunks are issued before any result is used:
  // V rows (rows past n are clamped to n - 1: read, never used) and, for lane q,
  // row q's attention values of the group's first MAXG heads (unconditional,
  // clamped loads: loads on a branch or in a runtime loop each wait for their
  // own round trip)
  uint4 raw[CPW][NL];
  float av[CPW][MAXG];
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) {
    const int64_t j0 = ((int64_t)grp * CPW + cc) * RW;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int64_t j = min(j0 + u * RPI + rg, n - 1);
      raw[cc][u] = ld_stream(Vg + j * d + c * W);
    }
    if constexpr (GM) {
      av[cc][0] = A_hq[((int64_t)l * Hkv + g) * n + min(j0 + q, n - 1)];
    } else {
      const float* Ah = A_hq + ((int64_t)l * Hq + (int64_t)g * G) * n + min(j0 + q, n - 1);
#pragma unroll
      for (int h = 0; h < MAXG; ++h) av[cc][h] = Ah[(int64_t)min(h, G - 1) * n];
    }
  }
  // without this the attention loads are sunk into the branch below and the
  // first V row is waited for before the others are requested (A_hq is not
  // __restrict__ for the same reason: a restrict read-only load may be moved past
  // the clobber)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) {
    const int64_t j0 = ((int64_t)grp * CPW + cc) * RW;
    float ss[NL];
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      float x[W];
      El<T>::unpack(raw[cc][u], x);
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < W; ++e) a += x[e] * x[e];
      ss[u] = group_sum<LG>(a);
    }
    // row q = u * RPI + r lives in register u of the lanes of row group r
    float s2 = 0.f;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const float v = __shfl(ss[u], (q % RPI) * LG, 64);
      s2 = (q / RPI == u) ? v : s2;
    }
    const int64_t j = j0 + q;
    if (GM && q < RW && j < n) {
      U[((int64_t)l * Hkv + g) * n + j] = av[cc][0] * sqrtf(s2);
    } else if (!GM && q < RW && j < n) {
      const float vn = sqrtf(s2);
      float mx = -INFINITY, sum = 0.f;
#pragma unroll
      for (int h = 0; h < MAXG; ++h) {
        if (h < G) {
          mx = fmaxf(mx, av[cc][h] * vn);
          sum += av[cc][h];
        }
      }
      const float* Ah = A_hq + ((int64_t)l * Hq + (int64_t)g * G) * n + j;
      for (int h = MAXG; h < G; ++h) {           // groups above MAXG heads
        const float a = Ah[(int64_t)h * n];
        mx = fmaxf(mx, a * vn);
        sum += a;
      }
      const int64_t o = ((int64_t)l * Hkv + g) * n + j;
      U[o] = mx;
      Ag[o] = sum / (float)G;
    }
  }
}

// ------------------------------------------------------------- merge
constexpr int NTM = 256;        // 4 waves, one bucket each

__device__ __forceinline__ int64_t lower_bound(const int32_t* a, int64_t m, int64_t x) {
  int64_t lo = 0, hi = m;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

struct MergeTables {
  ConstPtrs K, V, idx;
  MutPtrs Ko, Vo, logR;
  I64s m;
  I64s task0;     // first bucket task of each layer (tasks of a layer = Hkv * nbuckets)
};

// Any bucket size: one wave per bucket, binary searches and a walk of the kept
// list (used for buckets above 64 tokens).
template <typename T, int LG>
__global__ void __launch_bounds__(NTM)
merge_kernel_any(MergeTables t, int lc, const float* __restrict__ Ag, int Hkv, int64_t n, int d,
                 int bucket, int64_t nbuckets, int64_t ntask) {
  constexpr int W = El<T>::N;
  constexpr int RPP = 64 / LG;                   // rows per wave pass
  const int lane = threadIdx.x & 63;
  const int64_t task = (int64_t)blockIdx.x * (NTM / 64) + threadIdx.x / 64;
  if (task >= ntask) return;                     // waves are independent (no barriers)
  int l = 0;
  while (l + 1 < lc && t.task0.v[l + 1] <= task) ++l;
  const int64_t local = task - t.task0.v[l];
  const int g = (int)(local / nbuckets);
  const int64_t b0 = (local % nbuckets) * bucket;
  const int64_t b1 = min(n, b0 + bucket);
  const int64_t m = t.m.v[l];
  const int32_t* ip = (const int32_t*)t.idx.p[l] + (int64_t)g * m;
  const int64_t lo = lower_bound(ip, m, b0), hi = lower_bound(ip, m, b1);
  if (lo == hi) return;                          // no kept token: evicted tokens dropped
  const float* A = Ag + ((int64_t)l * Hkv + g) * n;
  const T* Vg = (const T*)t.V.p[l] + (int64_t)g * n * d;
  const T* Kg = (const T*)t.K.p[l] + (int64_t)g * n * d;
  T* Vo = (T*)t.Vo.p[l] + (int64_t)g * m * d;
  T* Ko = (T*)t.Ko.p[l] + (int64_t)g * m * d;
  float* lR = (float*)t.logR.p[l] + (int64_t)g * m;

  // merge target: the kept token with the largest A, ties to the lower index
  float bv = -INFINITY;
  int64_t bs = INT64_MAX;
  for (int64_t s = lo + lane; s < hi; s += 64) {
    const float a = A[ip[s]];
    if (bs == INT64_MAX || a > bv) { bv = a; bs = s; }   // s ascends per lane: first max kept
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int64_t os = __shfl_xor(bs, o, 64);
    if (ov > bv || (ov == bv && os < bs)) { bv = ov; bs = os; }
  }
  // every lane holds the same winner; the clamp only guards against NaN scores
  const int64_t ts = (bs >= lo && bs < hi) ? bs : lo, tt = ip[ts];
  const float At = A[tt];

  const int rg = lane / LG, c = lane % LG;
  float vt[W];
  El<T>::unpack(*reinterpret_cast<const uint4*>(Vg + tt * d + c * W), vt);
  float nt2 = 0.f;
#pragma unroll
  for (int e = 0; e < W; ++e) nt2 += vt[e] * vt[e];
  nt2 = group_sum<LG>(nt2);
  const float nt = sqrtf(nt2);

  float num[W];
#pragma unroll
  for (int e = 0; e < W; ++e) num[e] = 0.f;
  float den = 0.f;
  int64_t ptr = lo;                              // walk of the kept list, per row group
  for (int64_t e = b0 + rg; e < b1; e += RPP) {
    while (ptr < hi && ip[ptr] < e) ++ptr;
    const bool kept = ptr < hi && ip[ptr] == e;
    const uint4 raw = *reinterpret_cast<const uint4*>(Vg + e * d + c * W);
    if (kept) {
      *reinterpret_cast<uint4*>(Ko + ptr * d + c * W) = *reinterpret_cast<const uint4*>(Kg + e * d + c * W);
      if (e != tt) {
        *reinterpret_cast<uint4*>(Vo + ptr * d + c * W) = raw;
        if (c == 0) lR[ptr] = 0.f;
      }
      continue;
    }
    float ve[W];
    El<T>::unpack(raw, ve);
    float dot = 0.f, ne2 = 0.f;
#pragma unroll
    for (int i = 0; i < W; ++i) { dot += ve[i] * vt[i]; ne2 += ve[i] * ve[i]; }
    dot = group_sum<LG>(dot);
    ne2 = group_sum<LG>(ne2);
    const float nd = sqrtf(ne2) * nt;
    const float gate = nd > 0.f ? fmaxf(dot / nd, 0.f) : 0.f;
    const float wgt = gate * A[e];
#pragma unroll
    for (int i = 0; i < W; ++i) num[i] += wgt * ve[i];
    den += wgt;
  }
  // sum the row groups (lanes with the same chunk c)
#pragma unroll
  for (int o = LG; o < 64; o <<= 1) {
#pragma unroll
    for (int i = 0; i < W; ++i) num[i] += __shfl_xor(num[i], o, 64);
    den += __shfl_xor(den, o, 64);
  }
  if (rg == 0) {
    float out[W];
    float lr = 0.f;
    if (den > 0.f) {
      const float inv = 1.0f / (At + den);
#pragma unroll
      for (int i = 0; i < W; ++i) out[i] = (At * vt[i] + num[i]) * inv;
      lr = log1pf(den / At);
      *reinterpret_cast<uint4*>(Vo + ts * d + c * W) = El<T>::pack(out);
    } else {
      *reinterpret_cast<uint4*>(Vo + ts * d + c * W) =
          *reinterpret_cast<const uint4*>(Vg + tt * d + c * W);
    }
    if (c == 0) lR[ts] = lr;
  }
}

// Kept slots of one bucket, in two steps.  search_kept narrows [lo, hi], the range
// that holds the first index s in [0, m) with a[s] >= x (a ascending, m >= 1), to
// at most 64 entries: the first round probes 128 evenly spaced entries at once (2
// per lane), rounds of 64 follow while needed.  The caller then loads the
// 128-entry window a[lo .. lo + 127], and finish_kept takes from it both the exact
// first slot and the 64 entries after it.  For 25600 kept indices that is three
// dependent round trips, against fifteen for a binary search and one more for
// the entries.  (Scattered probes are costly: with 512 in the first round, one
// round trip fewer, the merge ran 12% slower.)
__device__ __forceinline__ void search_kept(const int32_t* a, int64_t m, int64_t x, int lane,
                                            int64_t& lo, int64_t& hi) {
  lo = 0; hi = m;
  // one probe round: probe k (0 <= k < 64 * U) at lo + k * step; the probes below
  // x form a prefix in k.  Loads are unconditional (clamped into [lo, hi)) so that
  // all U of a lane are in flight together.
  auto round = [&](auto U_t) __attribute__((always_inline)) {
    constexpr int U = decltype(U_t)::value;
    const int64_t step = (hi - lo + 64 * U - 1) / (64 * U);
    int v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = a[min(lo + (int64_t)(64 * u + lane) * step, hi - 1)];
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t p = lo + (int64_t)(64 * u + lane) * step;
      cnt += __builtin_popcountll(__ballot(p < hi && v[u] < x));
    }
    if (cnt == 0) { hi = lo; return; }           // a[lo] >= x
    const int64_t nlo = lo + (int64_t)(cnt - 1) * step + 1;
    hi = min(hi, lo + (int64_t)cnt * step);
    lo = nlo;
  };
  if (hi - lo > 64) round(std::integral_constant<int, 2>{});
  while (hi - lo > 64) round(std::integral_constant<int, 1>{});
}

// w0 = a[lo + lane], w1 = a[lo + 64 + lane] (clamped loads).  Returns the first
// slot; lane s receives a[first + s], INT64_MAX past m.
__device__ __forceinline__ int64_t finish_kept(int64_t m, int x, int lane, int64_t lo,
                                               int64_t hi, int w0, int w1, int64_t& out) {
  // 32-bit compare: a widening of w0 would be placed right after its load, and
  // wait for it there
  const int off = __builtin_popcountll(__ballot(lo + lane < hi && w0 < x));
  const int src = (off + lane) & 63;
  const int e0 = __shfl(w0, src, 64), e1 = __shfl(w1, src, 64);
  const int64_t first = lo + off;
  out = first + lane < m ? (int64_t)(off + lane < 64 ? e0 : e1) : INT64_MAX;
  return first;
}

// Buckets of at most 64 tokens: one wave per bucket.  The kept list of the
// bucket takes three dependent round trips (two rounds of search_kept, then a
// window load that finish_kept reads), and K of its first 4 * RPP kept rows a
// fourth; the bucket's V rows and A values (lane r holds A of row r; shuffles
// hand each row group its value) are requested right after the window, so they
// arrive meanwhile.
// The kept rows form a 64-bit mask, so a kept row's output slot is a popcount.
// Target (largest A_g, ties to the lower index), gates, sums and outputs are as in
// merge_kernel_any, in the same order.  (Ag is not __restrict__ here: a restrict
// read-only load may be moved past the memory clobber that pins it.)
template <typename T, int LG>
__global__ void __launch_bounds__(NTM)
merge_kernel(MergeTables t, int lc, const float* Ag, int Hkv, int64_t n, int d,
             int bucket, int64_t nbuckets, int64_t ntask) {
  constexpr int W = El<T>::N;
  constexpr int RPP = 64 / LG;                   // rows per wave pass
  constexpr int NP = 64 / RPP;                   // passes over a 64-row bucket
  const int lane = threadIdx.x & 63;
  // wave-uniform, so that the per-layer pointers are scalar loads
  const int64_t task = (int64_t)blockIdx.x * (NTM / 64) +
                       __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  if (task >= ntask) return;                     // waves are independent (no barriers)
  int l = 0;
  while (l + 1 < lc && t.task0.v[l + 1] <= task) ++l;
  const int64_t local = task - t.task0.v[l];
  const int g = (int)(local / nbuckets);
  const int64_t b0 = (local % nbuckets) * bucket;
  const int64_t b1 = min(n, b0 + bucket);
  const int nrow = (int)(b1 - b0);
  const int64_t m = t.m.v[l];
  const int32_t* ip = (const int32_t*)t.idx.p[l] + (int64_t)g * m;
  const float* A = Ag + ((int64_t)l * Hkv + g) * n;
  const T* Vg = (const T*)t.V.p[l] + (int64_t)g * n * d;
  const T* Kg = (const T*)t.K.p[l] + (int64_t)g * n * d;
  T* Vo = (T*)t.Vo.p[l] + (int64_t)g * m * d;
  T* Ko = (T*)t.Ko.p[l] + (int64_t)g * m * d;
  float* lR = (float*)t.logR.p[l] + (int64_t)g * m;
  const int rg = lane / LG, c = lane % LG;

  if (m == 0) return;                            // nothing kept in this layer
  // the kept list is narrowed to <= 64 candidates, then three groups of loads go
  // out in this order: the 128-entry window of the kept list, the bucket's V rows
  // (rows past b1 are clamped to b1 - 1: read, never used) and its A values.
  // Loads complete in order, so the window arrives without waiting for V.
  int64_t slo, shi;
  search_kept(ip, m, b0, lane, slo, shi);
  const int w0 = ip[min(slo + lane, m - 1)], w1 = ip[min(slo + 64 + lane, m - 1)];
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  uint4 raw[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int64_t e = min(b0 + p * RPP + rg, b1 - 1);
    raw[p] = ld_stream(Vg + e * d + c * W);      // read once
  }
  const float arow = A[b0 + min(lane, nrow - 1)];
  // keeps the loads above here: otherwise they are sunk into the branch below,
  // or scheduled after the first use of the window
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  int64_t kid;
  const int64_t lo = finish_kept(m, (int)b0, lane, slo, shi, w0, w1, kid);
  const bool kin = kid < b1;
  const int nk = __builtin_popcountll(__ballot(kin));
  if (nk == 0) return;                           // no kept token: evicted tokens dropped
  uint64_t rowmask = kin ? (1ull << (kid - b0)) : 0ull;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) rowmask |= __shfl_xor(rowmask, o, 64);

  // K of the first 4 * RPP kept rows (four named registers: an array here is
  // placed in LDS by the compiler, with a wait after every load)
  auto kload = [&](int q) __attribute__((always_inline)) {
    const int s = min(q * RPP + rg, nk - 1);
    const int64_t src = __shfl(kid, s, 64);
    return ld_stream(Kg + src * d + c * W);      // kept K rows are read once
  };
  auto kstore = [&](int q, const uint4& v) __attribute__((always_inline)) {
    const int s = min(q * RPP + rg, nk - 1);     // clamped lanes rewrite the last row
    st_stream(Ko + (lo + s) * d + c * W, v);
  };
  const uint4 k0 = kload(0), k1 = kload(1), k2 = kload(2), k3 = kload(3);

  // merge target: the kept row with the largest A, ties to the lower row (the
  // lower token index)
  const bool rkept = lane < nrow && ((rowmask >> lane) & 1ull);
  float bv = rkept ? arow : -INFINITY;
  int bs = rkept ? lane : 64;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int os = __shfl_xor(bs, o, 64);
    if (ov > bv || (ov == bv && os < bs)) { bv = ov; bs = os; }
  }
  // every lane holds the same winner; the fallback only guards against NaN scores
  const int rt = bs < 64 ? bs : __builtin_ctzll(rowmask);
  const int64_t tt = b0 + rt;
  const int64_t ts = lo + __builtin_popcountll(rowmask & ((1ull << rt) - 1ull));
  const float At = __shfl(arow, rt, 64);

  kstore(0, k0); kstore(1, k1); kstore(2, k2); kstore(3, k3);
  // more kept rows than a batch; the loop is wave-uniform so that every lane the
  // shuffle reads from is active
  for (int s0 = 4 * RPP; s0 < nk; s0 += RPP) {
    const int s = min(s0 + rg, nk - 1);
    const int64_t src = __shfl(kid, s, 64);
    st_stream(Ko + (lo + s) * d + c * W, ld_stream(Kg + src * d + c * W));
  }

  // the target's V row is one of the bucket rows already in registers: pass
  // rt / RPP (wave-uniform), lanes of row group rt % RPP
  const int pt = __builtin_amdgcn_readfirstlane(rt / RPP);
  uint4 tv = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    uint32_t mk = p == pt ? ~0u : 0u;
    asm volatile("" : "+v"(mk));                 // masks and ORs, not an indexed array
    tv.x |= raw[p].x & mk; tv.y |= raw[p].y & mk; tv.z |= raw[p].z & mk; tv.w |= raw[p].w & mk;
  }
  const int tsrc = (rt % RPP) * LG + c;
  tv.x = __shfl(tv.x, tsrc, 64); tv.y = __shfl(tv.y, tsrc, 64);
  tv.z = __shfl(tv.z, tsrc, 64); tv.w = __shfl(tv.w, tsrc, 64);
  float vt[W];
  El<T>::unpack(tv, vt);
  float nt2 = 0.f;
#pragma unroll
  for (int e = 0; e < W; ++e) nt2 += vt[e] * vt[e];
  nt2 = group_sum<LG>(nt2);
  const float nt = sqrtf(nt2);

  float num[W];
#pragma unroll
  for (int e = 0; e < W; ++e) num[e] = 0.f;
  float den = 0.f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int r = p * RPP + rg;                  // row within the bucket
    const float ae = __shfl(arow, r, 64);        // A of row r (uniform control flow here)
    const int64_t e = b0 + r;
    if (e >= b1) continue;
    if ((rowmask >> r) & 1ull) {                 // kept: copy its V (the target is merged below)
      if (e != tt) {
        const int64_t slot = lo + __builtin_popcountll(rowmask & ((1ull << r) - 1ull));
        st_stream(Vo + slot * d + c * W, raw[p]);
        if (c == 0) lR[slot] = 0.f;
      }
      continue;
    }
    float ve[W];
    El<T>::unpack(raw[p], ve);
    float dot = 0.f, ne2 = 0.f;
#pragma unroll
    for (int i = 0; i < W; ++i) { dot += ve[i] * vt[i]; ne2 += ve[i] * ve[i]; }
    dot = group_sum<LG>(dot);
    ne2 = group_sum<LG>(ne2);
    const float nd = sqrtf(ne2) * nt;
    const float gate = nd > 0.f ? fmaxf(dot / nd, 0.f) : 0.f;
    const float wgt = gate * ae;
#pragma unroll
    for (int i = 0; i < W; ++i) num[i] += wgt * ve[i];
    den += wgt;
  }
  // sum the row groups (lanes with the same chunk c)
#pragma unroll
  for (int o = LG; o < 64; o <<= 1) {
#pragma unroll
    for (int i = 0; i < W; ++i) num[i] += __shfl_xor(num[i], o, 64);
    den += __shfl_xor(den, o, 64);
  }
  if (rg == 0) {
    float out[W];
    float lr = 0.f;
    if (den > 0.f) {
      const float inv = 1.0f / (At + den);
#pragma unroll
      for (int i = 0; i < W; ++i) out[i] = (At * vt[i] + num[i]) * inv;
      lr = log1pf(den / At);
      st_stream(Vo + ts * d + c * W, El<T>::pack(out));
    } else {
      st_stream(Vo + ts * d + c * W, tv);
    }
    if (c == 0) lR[ts] = lr;
  }
}

template <typename T, bool GM>
bool launch_vatp(int LG, int lc, hipStream_t s, const float* A_hq, const ConstPtrs& V, int Hq,
                 int Hkv, int64_t n, int d, float* U, float* Ag) {
  const int64_t rw = (int64_t)(64 / LG) * (LG < VNL ? LG : VNL);
  const int64_t nchunk = (n + rw - 1) / rw;
  const int64_t nwave = (int64_t)lc * Hkv * ((nchunk + CPW - 1) / CPW);
  const dim3 grid((unsigned)((nwave + NT / 64 - 1) / (NT / 64)));
#define KVC_V(LGV) hipLaunchKernelGGL((vatp_union_kernel<T, LGV, GM>), grid, dim3(NT), 0, s, A_hq, V, Hq, Hkv, n, d, nchunk, nwave, U, Ag)
  switch (LG) {
    case 4: KVC_V(4); return true;
    case 8: KVC_V(8); return true;
    case 16: KVC_V(16); return true;
    case 32: KVC_V(32); return true;
    default: return false;
  }
#undef KVC_V
}

template <typename T>
bool launch_merge(int LG, dim3 grid, hipStream_t s, const MergeTables& t, int lc, const float* Ag,
                  int Hkv, int64_t n, int d, int bucket, int64_t nbuckets, int64_t ntask) {
#define KVC_M(LGV)                                                                                \
  do {                                                                                            \
    if (bucket <= 64)                                                                             \
      hipLaunchKernelGGL((merge_kernel<T, LGV>), grid, dim3(NTM), 0, s, t, lc, Ag, Hkv, n, d,     \
                         bucket, nbuckets, ntask);                                                \
    else                                                                                          \
      hipLaunchKernelGGL((merge_kernel_any<T, LGV>), grid, dim3(NTM), 0, s, t, lc, Ag, Hkv, n, d, \
                         bucket, nbuckets, ntask);                                                \
  } while (0)
  switch (LG) {
    case 4: KVC_M(4); return true;
    case 8: KVC_M(8); return true;
    case 16: KVC_M(16); return true;
    case 32: KVC_M(32); return true;
    default: return false;
  }
#undef KVC_M
}

bool lg_ok(int d, int dtype, int* LG) {
  const int rb = d * dtype_size(dtype);
  if (rb % 16) return false;
  *LG = rb / 16;
  return *LG == 4 || *LG == 8 || *LG == 16 || *LG == 32;
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" int kvc_vatp_union(const float* A_hq, const void* const* V, int dtype, int L, int Hq,
                              int Hkv, int64_t n, int d, float* U_out, float* Ag_out, void* stream) {
  clear_error();
  if (!dtype_ok(dtype)) return KVC_FAIL(KVC_ERR_DTYPE, "kvc_vatp_union: dtype %d", dtype);
  KVC_REQUIRE(L >= 1 && L <= KVC_MAX_LAYERS, "kvc_vatp_union: need 1 <= L <= %d", KVC_MAX_LAYERS);
  KVC_REQUIRE(Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0, "kvc_vatp_union: need Hq %% Hkv == 0");
  KVC_REQUIRE(n >= 1 && n <= 0x7fffffffLL, "kvc_vatp_union: need 1 <= n < 2^31");
  KVC_REQUIRE(A_hq && V && U_out && Ag_out, "kvc_vatp_union: null pointer");
  int LG = 0;
  KVC_REQUIRE(lg_ok(d, dtype, &LG), "kvc_vatp_union: need d * elsize in {64, 128, 256, 512} bytes");
  for (int l = 0; l < L; ++l)
    KVC_REQUIRE(V[l] && (uintptr_t)V[l] % 16 == 0, "kvc_vatp_union: V[%d] null or not 16-byte aligned", l);
  KVC_REQUIRE((int64_t)kLayersPerLaunch * Hkv * ((n + 31) / 32) / 4 <= 0x7fffffffLL,
              "kvc_vatp_union: grid too large");
  hipStream_t s = as_stream(stream);
  for (int l0 = 0; l0 < L; l0 += kLayersPerLaunch) {
    const int lc = min(kLayersPerLaunch, L - l0);
    ConstPtrs vt{};
    for (int i = 0; i < lc; ++i) vt.p[i] = V[l0 + i];
    const int64_t off = (int64_t)l0 * Hkv * n;
    if (dtype == KVC_BF16)
      launch_vatp<uint16_t, false>(LG, lc, s, A_hq + (int64_t)l0 * Hq * n, vt, Hq, Hkv, n, d, U_out + off, Ag_out + off);
    else
      launch_vatp<float, false>(LG, lc, s, A_hq + (int64_t)l0 * Hq * n, vt, Hq, Hkv, n, d, U_out + off, Ag_out + off);
  }
  return launch_status("kvc_vatp_union");
}

extern "C" int kvc_vatp_union_gmax(const float* A_gmax, const void* const* V, int dtype, int L,
                                   int Hkv, int64_t n, int d, float* U_out, void* stream) {
  clear_error();
  if (!dtype_ok(dtype)) return KVC_FAIL(KVC_ERR_DTYPE, "kvc_vatp_union_gmax: dtype %d", dtype);
  KVC_REQUIRE(L >= 1 && L <= KVC_MAX_LAYERS, "kvc_vatp_union_gmax: need 1 <= L <= %d", KVC_MAX_LAYERS);
  KVC_REQUIRE(Hkv >= 1, "kvc_vatp_union_gmax: need Hkv >= 1");
  KVC_REQUIRE(n >= 1 && n <= 0x7fffffffLL, "kvc_vatp_union_gmax: need 1 <= n < 2^31");
  KVC_REQUIRE(A_gmax && V && U_out, "kvc_vatp_union_gmax: null pointer");
  int LG = 0;
  KVC_REQUIRE(lg_ok(d, dtype, &LG), "kvc_vatp_union_gmax: need d * elsize in {64, 128, 256, 512} bytes");
  for (int l = 0; l < L; ++l)
    KVC_REQUIRE(V[l] && (uintptr_t)V[l] % 16 == 0, "kvc_vatp_union_gmax: V[%d] null or not 16-byte aligned", l);
  KVC_REQUIRE((int64_t)kLayersPerLaunch * Hkv * ((n + 31) / 32) / 4 <= 0x7fffffffLL,
              "kvc_vatp_union_gmax: grid too large");
  hipStream_t s = as_stream(stream);
  for (int l0 = 0; l0 < L; l0 += kLayersPerLaunch) {
    const int lc = min(kLayersPerLaunch, L - l0);
    ConstPtrs vt{};
    for (int i = 0; i < lc; ++i) vt.p[i] = V[l0 + i];
    const int64_t off = (int64_t)l0 * Hkv * n;
    if (dtype == KVC_BF16)
      launch_vatp<uint16_t, true>(LG, lc, s, A_gmax + off, vt, Hkv, Hkv, n, d, U_out + off, nullptr);
    else
      launch_vatp<float, true>(LG, lc, s, A_gmax + off, vt, Hkv, Hkv, n, d, U_out + off, nullptr);
  }
  return launch_status("kvc_vatp_union_gmax");
}

extern "C" int kvc_merge_gated(const void* const* K, const void* const* V, int dtype, const float* Ag,
                               int L, int Hkv, int64_t n, int d, const int32_t* const* idx,
                               const int64_t* m_keep, int bucket, void* const* K_out,
                               void* const* V_out, float* const* logR_out, void* stream) {
  clear_error();
  if (!dtype_ok(dtype)) return KVC_FAIL(KVC_ERR_DTYPE, "kvc_merge_gated: dtype %d", dtype);
  KVC_REQUIRE(L >= 1 && L <= KVC_MAX_LAYERS, "kvc_merge_gated: need 1 <= L <= %d", KVC_MAX_LAYERS);
  KVC_REQUIRE(Hkv >= 1 && n >= 1 && n <= 0x7fffffffLL, "kvc_merge_gated: need Hkv >= 1, 1 <= n < 2^31");
  KVC_REQUIRE(bucket >= 1, "kvc_merge_gated: bucket < 1");
  KVC_REQUIRE(K && V && Ag && idx && m_keep && K_out && V_out && logR_out, "kvc_merge_gated: null pointer");
  int LG = 0;
  KVC_REQUIRE(lg_ok(d, dtype, &LG), "kvc_merge_gated: need d * elsize in {64, 128, 256, 512} bytes");
  for (int l = 0; l < L; ++l) {
    KVC_REQUIRE(K[l] && V[l] && idx[l] && K_out[l] && V_out[l] && logR_out[l],
                "kvc_merge_gated: null pointer in layer %d", l);
    KVC_REQUIRE((uintptr_t)K[l] % 16 == 0 && (uintptr_t)V[l] % 16 == 0 && (uintptr_t)K_out[l] % 16 == 0 &&
                (uintptr_t)V_out[l] % 16 == 0, "kvc_merge_gated: tensors of layer %d not 16-byte aligned", l);
    KVC_REQUIRE(m_keep[l] >= 1 && m_keep[l] <= n, "kvc_merge_gated: m_keep[%d] outside [1, n]", l);
  }
  const int64_t nbuckets = (n + bucket - 1) / bucket;
  KVC_REQUIRE((int64_t)kLayersPerLaunch * Hkv * nbuckets / 4 <= 0x7fffffffLL, "kvc_merge_gated: too many buckets");
  hipStream_t s = as_stream(stream);
  for (int l0 = 0; l0 < L; l0 += kLayersPerLaunch) {
    const int lc = min(kLayersPerLaunch, L - l0);
    MergeTables t{};
    int64_t ntask = 0;
    for (int i = 0; i < lc; ++i) {
      t.K.p[i] = K[l0 + i]; t.V.p[i] = V[l0 + i]; t.idx.p[i] = idx[l0 + i];
      t.Ko.p[i] = K_out[l0 + i]; t.Vo.p[i] = V_out[l0 + i]; t.logR.p[i] = logR_out[l0 + i];
      t.m.v[i] = m_keep[l0 + i];
      t.task0.v[i] = ntask;
      ntask += (int64_t)Hkv * nbuckets;
    }
    const dim3 grid((unsigned)((ntask + 3) / 4));
    const float* Agl = Ag + (int64_t)l0 * Hkv * n;
    if (dtype == KVC_BF16)
      launch_merge<uint16_t>(LG, grid, s, t, lc, Agl, Hkv, n, d, bucket, nbuckets, ntask);
    else
      launch_merge<float>(LG, grid, s, t, lc, Agl, Hkv, n, d, bucket, nbuckets, ntask);
  }
  return launch_status("kvc_merge_gated");
}
