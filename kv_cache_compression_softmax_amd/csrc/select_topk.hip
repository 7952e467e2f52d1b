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
// thread's loads in flight together; its descent and output are described with
// the kernel below).  Longer rows still are re-read by every pass.  The
// histograms of the other paths are per wave, with wave-aggregated increments
// where lanes crowd into one bin.
#include "common.h"

namespace kvc {
namespace {

constexpr int NT = 1024;
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
// A row of up to RV * NTR vectors of 4 scores (RV = 16 or REGV: 32768 or 102400
// scores) is held in registers, as order-preserving keys, by a workgroup of NTR
// threads: thread t keeps vectors t, t + NTR, ..., all loads in flight together,
// so the row is read once.  Every step over the held keys is unrolled over all of them, so a step
// costs its body's instruction count per key: each body is kept to a few
// instructions, with no per-key membership tests and no exec-mask branches.
//   0. Keys outside [0, n - w) (the window, and the repeated last vector) are
//      replaced by key 0, the lowest key; the row's smallest and largest keys
//      are taken over the row alone.  Extra copies of the lowest key never move
//      the need-th largest key (need < n - w) and are never counted above it.
//   1. Each pass cuts the current key range [lo, lo + 2^sp) into nbin <= 256
//      bins of width 2^(sp-8), so scores spread over a few binades fill many
//      bins.  A key outside the range lands in bin nbin, which is not read; keys
//      below lo are tested as such, since key - lo wraps into the range when the
//      range spans 2^31 or more (scores of both signs) or lies near the top of
//      the key space.  The bin holding the need-th largest key becomes the next
//      range.
//   2. After the first pass every thread copies its keys of the chosen bin to
//      its own LDS slots (slot j of thread t at j * NTR + t; the key is written
//      at every step and the slot advances on a hit, so no branches).  The next
//      passes read each thread's own list into one histogram for the block;
//      once the chosen bin holds at most 64 keys they are gathered and one wave
//      ranks them.  If a thread has more than LSLOT hits, the passes run over
//      the registers instead.
//   3. Ordered output: chunk r of the row is vector r * NTR + t of thread t.
//      When every copy of T is kept (the usual case), a key is kept iff
//      key >= T, and each wave's counts and lane positions come from one ballot
//      per key (popcounts and mbcnts).  With a tie at the cut, the index c of
//      the last kept copy of T is found first, and a key is kept iff key > T or
//      (key == T and index <= c), again one ballot per key.  The chunk and
//      wave offsets come from one table in LDS.
// A global int32 pointer the whole wave shares, moved to scalar registers.
using GlobalI32 = __attribute__((address_space(1))) int32_t;
__device__ __forceinline__ GlobalI32* uniform_global(int32_t* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (GlobalI32*)(((uint64_t)hi << 32) | lo);
}
constexpr int NWR = NTR / 64;   // waves of the register path
constexpr int LSLOT = 24;       // candidate slots per thread after the first pass
constexpr int CAND = LSLOT * NTR;

constexpr int HCOPY = 4;        // histogram copies per wave (by lane % HCOPY): fewer lanes per address
struct RegDescent {             // LDS of the descent
  union {
    struct {
      int hist[NWR][HCOPY][257];                   // passes over the registers; bin 256: outside
    } h;
    struct {
      uint32_t cand[(LSLOT + 1) * NTR];            // slot LSLOT: the sink of a full list
    };
  };
};
struct RegOutput {              // LDS of the ordered output
  int wtot[REGV][NWR];                             // per chunk and wave: above T | copies of T << 16
  int wpre[REGV][NWR];                             // kept in the chunk's earlier waves
  int cbase[REGV];                                 // kept in earlier chunks
  uint8_t eqm[REGV][NTR];                          // with a tie: each thread's copies of T per chunk
};
union RegShared {
  RegDescent d;
  RegOutput o;
};

template <int RV>
__global__ void __launch_bounds__(NTR)
select_reg_kernel(const float* __restrict__ S, int Hkv, int64_t n, I64s kk, int w, MutPtrs idx) {
  __shared__ RegShared sh;
  __shared__ int wh[257];                          // histogram of the passes over the lists
  __shared__ uint32_t fin[64];                     // the last bin's keys
  __shared__ int fcnt[1];
  __shared__ int cut[4];                           // tie at the cut: chunk, wave, rank there; index
  __shared__ uint32_t red[2][NWR];
  __shared__ int scan[NWR];
  __shared__ int pick[3];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid / 64;
  const int l = blockIdx.x / Hkv, g = blockIdx.x % Hkv;
  const int64_t k = kk.v[l];
  const float* row = S + ((int64_t)l * Hkv + g) * n;
  // the output row's address is uniform: held in scalar registers, with 32-bit
  // unsigned offsets from it
  GlobalI32* const out = uniform_global((int32_t*)idx.p[l] + (int64_t)g * k);
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
  // last one); element 4 (r NTR + t) + e is in the row iff 4 r NTR + e < lim
  uint4 rk[RV];
  const int lim = nb - 4 * tid;
  uint32_t kmin = ~0u, kmax = 0u;                 // over the row's keys
  {
    const int nv = (nb + 3) / 4;
    const float4* row4 = reinterpret_cast<const float4*>(row);
    float4 t[RV];
#pragma unroll
    for (int r = 0; r < RV; ++r) t[r] = row4[min(r * NTR + tid, nv - 1)];
    int lm = lim;                                 // opaque: the membership masks die here
    asm volatile("" : "+v"(lm));
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      uint32_t k4[4] = {f32_key(t[r].x), f32_key(t[r].y), f32_key(t[r].z), f32_key(t[r].w)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool in = 4 * r * NTR + e < lm;
        kmin = min(kmin, in ? k4[e] : ~0u);
        k4[e] = in ? k4[e] : 0u;
        kmax = max(kmax, k4[e]);
      }
      rk[r] = make_uint4(k4[0], k4[1], k4[2], k4[3]);
    }
  }
  auto each = [&](auto&& f) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < RV; ++r) { f(rk[r].x); f(rk[r].y); f(rk[r].z); f(rk[r].w); }
  };
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
  }
  if (lane == 0) { red[0][wv] = kmin; red[1][wv] = kmax; }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < NWR; ++x) { kmin = min(kmin, red[0][x]); kmax = max(kmax, red[1][x]); }
  // ---- descent: T = the need-th largest key, above = keys > T, eqc = keys == T
  // (eqc may include pad keys when T is the lowest key; then it exceeds the
  // copies of T that are kept, and the output takes the tie path)
  uint32_t lo = kmin;
  int above = 0, rem = need, eqc = nb;
  if (kmax != kmin) {
    int sp = 32 - __builtin_clz(kmax - kmin);   // the range is [lo, lo + 2^sp)
    bool list = false;
    int cnt = 0;                                  // the thread's list length
#pragma unroll 1
    for (int pass = 0;; ++pass) {
      const int s = sp > 8 ? sp - 8 : 0;          // bin width 2^s
      const uint32_t dmax = sp >= 32 ? ~0u : (1u << sp) - 1u;
      const uint32_t nbin = (dmax >> s) + 1u;     // <= 256; key - lo > dmax <=> bin >= nbin
      for (int i = tid; i < NWR * HCOPY * 257; i += NTR) (&sh.d.h.hist[0][0][0])[i] = 0;
      __syncthreads();
      {
        int* hh = sh.d.h.hist[wv][lane % HCOPY];
        each([&](uint32_t key) { atomicAdd(&hh[key >= lo ? min((key - lo) >> s, nbin) : nbin], 1); });
      }
      __syncthreads();
      int c = 0;
      if (tid < 256 && 255 - tid < (int)nbin) {
#pragma unroll
        for (int x = 0; x < NWR * HCOPY; ++x) c += (&sh.d.h.hist[0][0][0])[x * 257 + 255 - tid];
      }
      int tot;
      const int incl = block_exclusive_scan<NTR>(c, scan, &tot) + c;
      if (tid < 256 && incl >= rem && incl - c < rem) { pick[0] = 255 - tid; pick[1] = incl - c; pick[2] = c; }
      __syncthreads();
      const int b = pick[0];
      eqc = pick[2];
      above += pick[1];
      rem -= pick[1];
      lo += (uint32_t)b << s;
      sp = s;
      if (s == 0) break;
      if (pass == 0 && eqc <= CAND) {             // the chosen bin's keys to per-thread lists
        const uint32_t width = 1u << s;
        each([&](uint32_t key) {
          sh.d.cand[min(cnt, LSLOT) * NTR + tid] = key;
          cnt += ((key >= lo) & (key - lo < width)) ? 1 : 0;
        });
        list = !__syncthreads_or(cnt > LSLOT);
        if (list) break;
      }
    }
    if (list) {
      // The remaining passes read each thread's own list (one 256-bin histogram
      // for the block).  Once the chosen bin holds at most 64 keys they are
      // gathered and wave 0 ranks them directly.
      auto list_keys = [&](auto&& f) __attribute__((always_inline)) {
#pragma unroll 1
        for (int j = 0; j < cnt; j += 4) {        // four reads in flight
          uint32_t x[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) x[q] = sh.d.cand[min(j + q, LSLOT) * NTR + tid];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (j + q < cnt) f(x[q]);
        }
      };
#pragma unroll 1
      for (;;) {
        const int s = sp > 8 ? sp - 8 : 0;
        const uint32_t nbin = (((1u << sp) - 1u) >> s) + 1u;   // sp < 32 here
        if (tid < 257) wh[tid] = 0;
        if (tid == 0) fcnt[0] = 0;
        __syncthreads();
        list_keys([&](uint32_t key) { atomicAdd(&wh[key >= lo ? min((key - lo) >> s, nbin) : nbin], 1); });
        __syncthreads();
        if (wv == 0) {                            // lane i walks bins 255 - 4i - q downwards
          int c4[4], sum = 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int bn = 255 - 4 * lane - q;
            c4[q] = bn < (int)nbin ? wh[bn] : 0;
            sum += c4[q];
          }
          int run = wave_inclusive_scan(sum) - sum;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (run < rem && run + c4[q] >= rem) { pick[0] = 255 - 4 * lane - q; pick[1] = run; pick[2] = c4[q]; }
            run += c4[q];
          }
        }
        __syncthreads();
        eqc = pick[2];
        above += pick[1];
        rem -= pick[1];
        lo += (uint32_t)pick[0] << s;
        sp = s;
        if (s == 0) break;
        if (eqc <= 64) {                          // gather the bin's keys, then rank them in wave 0
          const uint32_t width = 1u << s;
          list_keys([&](uint32_t key) {
            if (key >= lo && key - lo < width) {
              const int at = atomicAdd(&fcnt[0], 1);
              if (at < 64) fin[at] = key;
            }
          });
          __syncthreads();
          if (wv == 0) {
            const bool valid = lane < eqc;
            const uint32_t x = valid ? fin[lane] : 0u;
            int gt = 0, ge = 0;
#pragma unroll 1
            for (int j = 0; j < eqc; ++j) {
              const uint32_t y = __builtin_amdgcn_readlane(x, j);
              gt += y > x ? 1 : 0;
              ge += y >= x ? 1 : 0;
            }
            const uint64_t hm = __ballot(valid && gt < rem && ge >= rem);
            if (hm != 0 && lane == (int)__builtin_ctzll(hm)) { pick[0] = (int)x; pick[1] = gt; pick[2] = ge - gt; }
          }
          __syncthreads();
          lo = (uint32_t)pick[0];
          above += pick[1];
          eqc = pick[2];
          break;
        }
      }
    }
  }
  const uint32_t T = __builtin_amdgcn_readfirstlane(lo);
  const int teq = need - above;                   // >= 1 copies of T are kept
  const int nchunk = (nb + 4 * NTR - 1) / (4 * NTR);
  const bool untied = eqc == teq;                 // every copy of T kept (T > 0 then)
  __syncthreads();                                // the descent's LDS is reused below
  // ---- ordered output.  Chunk r is vector r * NTR + t of every thread t, so a
  // lane's place is the chunk's offset, its wave's offset in the chunk, and the
  // kept elements of the lanes below it (mbcnts of one ballot per element).
  // Without a tie at the cut, a key is kept iff key >= T.  With one, the kept
  // copies of T are the first teq in index order; with c the index of the last
  // of them, a key is kept iff key > T, or key == T and its index <= c.  Pad
  // keys need no test: they are never above T, and their places (past n - w)
  // come after every copy of T in the row, of which there are at least teq.
  //   1. per chunk and wave: keys above T and copies of T (popcounts);
  //   2. wave 0, one lane per chunk: offsets that count the copies of T only
  //      up to copy teq, and the chunk, wave and rank there of copy teq;
  //   3. with a tie, that wave finds the copy's lane and element, hence c;
  //   4. one masked store per kept element.
  // Chunk loops end at the row's last chunk; the bound is made opaque per loop
  // so that no per-chunk flags are kept across loops.
  auto below = [&](uint64_t m, int base) __attribute__((always_inline)) {   // base + set lanes below this one
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)base));
  };
  auto bound = [&]() __attribute__((always_inline)) {
    int c = nchunk;
    asm volatile("" : "+s"(c));
    return c;
  };
  const int last = need - 1;                      // places are < need; the clamp keeps any slip in the row
  if (untied) {
    const int nc = bound();
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      if (r < nc) {                              // uniform
        const uint32_t k4[4] = {rk[r].x, rk[r].y, rk[r].z, rk[r].w};
        int tg = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) tg += __builtin_popcountll(__ballot(k4[e] >= T));
        if (lane == 0) sh.o.wtot[r][wv] = tg;
      }
    }
  } else {
    const int nc = bound();
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      if (r < nc) {                              // uniform
        const uint32_t k4[4] = {rk[r].x, rk[r].y, rk[r].z, rk[r].w};
        int tg = 0, te = 0;
        uint32_t q = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          tg += __builtin_popcountll(__ballot(k4[e] > T));
          te += __builtin_popcountll(__ballot(k4[e] == T));
          q |= (k4[e] == T ? 1u : 0u) << e;
        }
        sh.o.eqm[r][tid] = (uint8_t)q;
        if (lane == 0) sh.o.wtot[r][wv] = tg | (te << 16);
      }
    }
  }
  if (tid == 0) { cut[0] = -1; cut[1] = -1; cut[2] = 0; cut[3] = -1; }
  __syncthreads();
  if (tid < 64) {
    int ce = 0;
    if (tid < nchunk) {
#pragma unroll
      for (int x = 0; x < NWR; ++x) ce += sh.o.wtot[tid][x] >> 16;
    }
    int eb = wave_inclusive_scan(ce) - ce;        // copies of T before chunk tid
    int run = 0;
    if (tid < nchunk) {
#pragma unroll
      for (int x = 0; x < NWR; ++x) {
        const int wt = sh.o.wtot[tid][x], tg = wt & 0xffff, te = wt >> 16;
        if (eb < teq && teq <= eb + te) { cut[0] = tid; cut[1] = x; cut[2] = teq - eb; }
        sh.o.wpre[tid][x] = run;
        run += tg + min(max(teq - eb, 0), te);    // kept: the copies of T up to copy teq
        eb += te;
      }
    }
    const int inc = wave_inclusive_scan(run);
    if (tid < nchunk) sh.o.cbase[tid] = inc - run;
  }
  __syncthreads();
  if (untied) {
    const int nc = bound();
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      if (r < nc) {                              // uniform
        const uint32_t k4[4] = {rk[r].x, rk[r].y, rk[r].z, rk[r].w};
        int pos = __builtin_amdgcn_readfirstlane(sh.o.cbase[r] + sh.o.wpre[r][wv]);
#pragma unroll
        for (int e = 0; e < 4; ++e) pos = below(__ballot(k4[e] >= T), pos);
        const int i0 = 4 * (r * NTR + tid);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool kp = k4[e] >= T;
          if (kp) out[(uint32_t)min(pos, last)] = i0 + e;
          pos += kp ? 1 : 0;
        }
      }
    }
    return;
  }
  const int cr = cut[0], cx = cut[1], ck = cut[2];
  if (cr >= 0 && wv == cx) {                      // the wave holding copy teq: its lane and element
    const uint32_t q = sh.o.eqm[cr][tid];
    const int own = __builtin_popcount(q);
    const int bl = wave_inclusive_scan(own) - own;   // copies in the lanes below
    if (bl < ck && ck <= bl + own) {
      int left = ck - bl, e = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const bool one = (q >> b) & 1u;
        if (one && left == 1) e = b;
        left -= one ? 1 : 0;
      }
      cut[3] = 4 * (cr * NTR + tid) + e;
    }
  }
  __syncthreads();
  const int cidx = cut[3];
  const int nc = bound();
#pragma unroll
  for (int r = 0; r < RV; ++r) {
    if (r < nc) {                              // uniform
      const uint32_t k4[4] = {rk[r].x, rk[r].y, rk[r].z, rk[r].w};
      const int i0 = 4 * (r * NTR + tid);
      bool kp[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) kp[e] = (k4[e] > T) | ((k4[e] == T) & (i0 + e <= cidx));   // no branches
      int pos = __builtin_amdgcn_readfirstlane(sh.o.cbase[r] + sh.o.wpre[r][wv]);
#pragma unroll
      for (int e = 0; e < 4; ++e) pos = below(__ballot(kp[e]), pos);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (kp[e]) out[(uint32_t)min(pos, last)] = i0 + e;
        pos += kp[e] ? 1 : 0;
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
  // A row of more than 8192 scores, up to REGV vectors per thread, is held in
  // registers (16 vectors per thread when that holds it): 50 -> 22 us for 256
  // rows of 32768 scores against the LDS copy.  Shorter rows, where the LDS
  // path was a little faster (a decode period's 7577-slot rows), keep it; a row
  // too long for either is re-read by every pass.
  const int64_t nvr = (n - w + 3) / 4;
  const bool use_reg = vec && n > w && nvr <= (int64_t)REGV * NTR && (nvr > 4 * NTR || !use_cache);
  const bool rv16 = nvr <= 16 * NTR;
  for (int l0 = 0; l0 < L; l0 += kLayersPerLaunch) {
    const int lc = min(kLayersPerLaunch, L - l0);
    I64s kk{};
    MutPtrs ip{};
    for (int i = 0; i < lc; ++i) { kk.v[i] = k_keep[l0 + i]; ip.p[i] = idx_out[l0 + i]; }
    const dim3 grid((unsigned)(lc * Hkv));
    const float* Sl = S + (int64_t)l0 * Hkv * n;
    if (use_reg && rv16) hipLaunchKernelGGL(select_reg_kernel<16>, grid, dim3(NTR), 0, s, Sl, Hkv, n, kk, w, ip);
    else if (use_reg) hipLaunchKernelGGL(select_reg_kernel<REGV>, grid, dim3(NTR), 0, s, Sl, Hkv, n, kk, w, ip);
    else if (use_cache) hipLaunchKernelGGL((select_kernel<true, true>), grid, dim3(NT), cache, s, Sl, Hkv, n, kk, w, ip);
    else if (vec) hipLaunchKernelGGL((select_kernel<true, false>), grid, dim3(NT), 0, s, Sl, Hkv, n, kk, w, ip);
    else hipLaunchKernelGGL((select_kernel<false, false>), grid, dim3(NT), 0, s, Sl, Hkv, n, kk, w, ip);
  }
  return launch_status("kvc_select_topk");
}
