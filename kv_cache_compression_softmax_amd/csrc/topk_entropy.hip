// Top-k restricted entropy of each final-layer logits row.
//
// [InfoKV] Method and Glossary (top-k restricted entropy): for every token the
// entropy of the model's next-token distribution is taken over its k most likely
// tokens only, renormalised over them.
//
// One wave streams one row from HBM exactly once (16-byte lanes, the next step's
// loads in flight while the current one is filtered) and never waits for another
// wave.  Instead of holding the 256 KB row on chip it keeps a candidate list in its
// own slice of LDS.  All comparisons are in the order of the order-preserving
// integer keys (bit patterns), so they are exact and free of float rounding.
//   * tau is the k-th largest key among the elements seen so far.
//   * Filter: a lane appends its whole 16-byte vector (8 bf16 or 4 float32) when
//     any element's key exceeds tau.  For tau >= +0 that test is a signed max of
//     the raw bit patterns (packed 16-bit for bf16: half an instruction per
//     element); for tau < 0 it is "some element is >= +0, or the unsigned min of
//     the bit patterns is below tau's".  At k ~ 0.2% of the row about one vector
//     in a hundred is appended, so the test, not the appending, sets the pace.
//   * Re-select, when the list passes RESEL: an ordered compaction keeps the keys
//     >= tau (the other elements of appended vectors are dropped here), an exact
//     radix select (8-bit digits, LDS histogram) finds the new tau, and a second
//     compaction rewrites the list as the keys > tau followed by copies of tau,
//     padded to a whole vector with the smallest key.
// The list always holds, besides real elements of the row and padding of the
// smallest key, exactly the top-k multiset of what was seen: an element that is
// not > the current tau never enters the final top-k beyond the copies of tau
// already held, so the final list equals the row's top-k multiset.  Appends and
// compactions are ordered by lane and element index (ballots and prefix sums; no
// atomic decides a position), so the float sums below are deterministic.
// Entropy is float32 over the k survivors, summing -p ln p term by term.
#include "common.h"

namespace kvc {
namespace {

constexpr int NT = 256;      // 4 waves = 4 rows per workgroup

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
constexpr int RESEL = 1536;  // list length that triggers a re-select (>= k rounded up)

typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

template <typename T> struct Tr;
template <> struct Tr<uint16_t> {                 // bf16 bit patterns
  using Raw = uint16_t;
  static constexpr int VEC = 8;
  static constexpr int NV = 2;                    // 16-byte vectors per lane per step
  static constexpr int DIGITS = 2;
  static constexpr Raw kMin = 0xffffu;            // bit pattern of the smallest key (0)
  __device__ static uint32_t key(Raw r) { return bf16_key(r); }
  __device__ static float value(uint32_t k) { return key_bf16(k); }
  __device__ static Raw raw(uint32_t k) {         // canonical bit pattern of a key
    return (k & 0x8000u) ? (Raw)(k & 0x7fffu) : (Raw)(~k & 0xffffu);
  }
  // some element's key > key(t), t = raw(tau): for t with a clear sign bit a
  // signed max of the bit patterns, else "some element >= +0 or the unsigned min
  // of the bit patterns below t"
  __device__ static bool above_pos(const uint4& u, Raw t) {
    const s16x2 a = __builtin_bit_cast(s16x2, u.x), b = __builtin_bit_cast(s16x2, u.y);
    const s16x2 c = __builtin_bit_cast(s16x2, u.z), d = __builtin_bit_cast(s16x2, u.w);
    const s16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                              __builtin_elementwise_max(c, d));
    return max((int)m.x, (int)m.y) > (int)(short)t;
  }
  __device__ static bool above_neg(const uint4& u, Raw t) {
    const s16x2 a = __builtin_bit_cast(s16x2, u.x), b = __builtin_bit_cast(s16x2, u.y);
    const s16x2 c = __builtin_bit_cast(s16x2, u.z), d = __builtin_bit_cast(s16x2, u.w);
    const s16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                              __builtin_elementwise_max(c, d));
    const u16x2 ua = __builtin_bit_cast(u16x2, u.x), ub = __builtin_bit_cast(u16x2, u.y);
    const u16x2 uc = __builtin_bit_cast(u16x2, u.z), ud = __builtin_bit_cast(u16x2, u.w);
    const u16x2 n = __builtin_elementwise_min(__builtin_elementwise_min(ua, ub),
                                              __builtin_elementwise_min(uc, ud));
    return max((int)m.x, (int)m.y) >= 0 || min((int)n.x, (int)n.y) < (int)t;
  }
};
template <> struct Tr<float> {
  using Raw = uint32_t;
  static constexpr int VEC = 4;
  static constexpr int NV = 4;
  static constexpr int DIGITS = 4;
  static constexpr Raw kMin = 0xffffffffu;
  __device__ static uint32_t key(Raw r) { return f32_key(__uint_as_float(r)); }
  __device__ static float value(uint32_t k) { return key_f32(k); }
  __device__ static Raw raw(uint32_t k) { return (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k; }
  __device__ static bool above_pos(const uint4& u, Raw t) {
    return max(max((int)u.x, (int)u.y), max((int)u.z, (int)u.w)) > (int)t;
  }
  __device__ static bool above_neg(const uint4& u, Raw t) {
    const int mx = max(max((int)u.x, (int)u.y), max((int)u.z, (int)u.w));
    return mx >= 0 || min(min(u.x, u.y), min(u.z, u.w)) < t;
  }
};

// Per-wave LDS: CAP candidate bit patterns and a 256-bin histogram.
template <typename Raw, int CAP>
struct WaveSmem {
  uint4 cand4[CAP * sizeof(Raw) / 16];
  int hist[256];
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// lanes strictly below this one that have their bit set in `mask`
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Ordered in-place compaction of cand[0..c): keeps the elements whose key passes
// `keep`, in their order; returns how many.  Lane l of round r reads the 16-byte
// group 64r + l; all reads of a round precede its writes, and an element only
// moves to a lower index.
template <typename T, typename Keep>
__device__ __forceinline__ int compact_keep(typename Tr<T>::Raw* cand, int c, Keep keep) {
  using Raw = typename Tr<T>::Raw;
  constexpr int VEC = Tr<T>::VEC;
  const int lane = threadIdx.x & 63;
  int pos = 0;
  for (int g0 = 0; g0 * VEC < c; g0 += 64) {
    const int g = g0 + lane;
    Raw e[VEC];
    uint32_t bits = 0;
    if (g * VEC < c) {
      const uint4 u = reinterpret_cast<const uint4*>(cand)[g];
      __builtin_memcpy(&e, &u, 16);
#pragma unroll
      for (int i = 0; i < VEC; ++i)
        bits |= (uint32_t)(g * VEC + i < c && keep(Tr<T>::key(e[i]))) << i;
    }
    const int cnt = __builtin_popcount(bits);
    const int incl = wave_inclusive_scan(cnt);
    wave_sync();
    int p = pos + incl - cnt;
#pragma unroll
    for (int i = 0; i < VEC; ++i)
      if (bits & (1u << i)) cand[p++] = e[i];
    pos += __builtin_amdgcn_readlane(incl, 63);   // wave-uniform
    wave_sync();
  }
  return pos;
}

// Re-select over cand[0..count): returns the new tau (the k-th largest key) and
// leaves cand[0..k) = the keys > tau in order, then copies of tau, padded with
// the smallest key to a whole vector; count receives the padded length.
// With have_tau, the elements below the old tau are dropped first (the list
// holds k elements >= it, so none of them can be in the top-k).
template <typename T>
__device__ __forceinline__ uint32_t reselect(typename Tr<T>::Raw* cand, int* hist, int& count,
                                             int k, bool have_tau, uint32_t tau_old) {
  using Raw = typename Tr<T>::Raw;
  constexpr int VEC = Tr<T>::VEC;
  constexpr int DIG = Tr<T>::DIGITS;
  const int lane = threadIdx.x & 63;
  wave_sync();
  int c = count;
  if (have_tau) c = compact_keep<T>(cand, c, [=](uint32_t key) { return key >= tau_old; });
  uint32_t prefix = 0;
  int need = k;                                  // rank of tau among the keys left
#pragma unroll 1
  for (int p = DIG - 1; p >= 0; --p) {
    const int shift = 8 * p;
    const uint32_t hi_mask = (p == DIG - 1) ? 0u : (uint32_t)(~0ull << (shift + 8));
#pragma unroll
    for (int b = 0; b < 4; ++b) hist[lane * 4 + b] = 0;
    wave_sync();
    for (int g0 = 0; g0 * VEC < c; g0 += 64) {
      const int g = g0 + lane;
      if (g * VEC < c) {
        const uint4 u = reinterpret_cast<const uint4*>(cand)[g];
        Raw e[VEC];
        __builtin_memcpy(&e, &u, 16);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const uint32_t key = Tr<T>::key(e[i]);
          if (g * VEC + i < c && (key & hi_mask) == (prefix & hi_mask))
            atomicAdd(&hist[(key >> shift) & 255], 1);
        }
      }
    }
    wave_sync();
    // lane owns bins 255-4*lane ... 252-4*lane (descending); inclusive scan of the
    // lane totals, then the crossing bin is found inside the owning lane
    int cb[4], tot = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) { cb[b] = hist[255 - 4 * lane - b]; tot += cb[b]; }
    const int incl = wave_inclusive_scan(tot);
    int run = incl - tot, dsel = -1, asel = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (dsel < 0 && run + cb[b] >= need) { dsel = 255 - 4 * lane - b; asel = run; }
      run += cb[b];
    }
    const uint64_t who = __ballot(dsel >= 0 && incl - tot < need);
    const int src = __builtin_ctzll(who);
    const int digit = __builtin_amdgcn_readlane(dsel, src);
    const int abv = __builtin_amdgcn_readlane(asel, src);
    prefix |= (uint32_t)digit << shift;
    need -= abv;
    wave_sync();
  }
  const uint32_t tau = prefix;
  const int cgt = compact_keep<T>(cand, c, [=](uint32_t key) { return key > tau; });
  // the cgt keys > tau are now cand[0..cgt), with cgt < k
  const int kr = (k + VEC - 1) / VEC * VEC;
  const Raw traw = Tr<T>::raw(tau);
  for (int i = cgt + lane; i < kr; i += 64) cand[i] = i < k ? traw : Tr<T>::kMin;
  wave_sync();
  count = kr;
  return tau;
}

// One vector of the ragged last step: elements past the row end read as the
// smallest key, which never enters the top-k ahead of a real element.
template <typename T>
__device__ __forceinline__ uint4 load_tail(const T* row, int64_t e0, int64_t vocab, bool vec_ok) {
  using Raw = typename Tr<T>::Raw;
  constexpr int VEC = Tr<T>::VEC;
  const int64_t left = vocab - e0;
  if (left >= VEC && vec_ok) return *reinterpret_cast<const uint4*>(row + e0);
  const Raw* r = reinterpret_cast<const Raw*>(row);
  Raw e[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) e[i] = (i < left) ? r[e0 + i] : Tr<T>::kMin;
  uint4 u;
  __builtin_memcpy(&u, &e, 16);
  return u;
}

// SPLIT waves share a row when rows are few (short row counts would leave most
// of the GPU idle with one wave per row): wave q of a row treats its part, the
// q-th run of whole steps (the last part also takes the ragged end), exactly as
// a row of its own and ends with that part's top-k.  Every element of the row's
// top-k multiset is in its part's top-k, so after a workgroup barrier the
// first wave of the row re-selects the top-k of the SPLIT lists and takes the
// entropy.  The host picks SPLIT so that every part has a whole step (at least
// k elements for the part's first select) and the SPLIT lists fit one list.
template <typename T, int CAP, bool ALIGNED, int SPLIT>
__global__ void __launch_bounds__(NT)
topk_entropy_kernel(const T* __restrict__ logits, int64_t rows, int64_t vocab_all, int64_t stride,
                    int k, float* __restrict__ H) {
  using Raw = typename Tr<T>::Raw;
  constexpr int VEC = Tr<T>::VEC;
  constexpr int NV = Tr<T>::NV;
  constexpr int STEP = 64 * NV * VEC;            // elements per wave per step
  // the first select takes the first step alone, which must hold k elements
  static_assert(STEP >= KVC_MAX_TOPK_ENTROPY, "a step holds at least the largest k");
  static_assert(CAP == RESEL + STEP && CAP % VEC == 0, "list capacity");
  static_assert(SPLIT == 1 || SPLIT == 2 || SPLIT == 4, "waves per row");
  __shared__ WaveSmem<Raw, CAP> smem[NT / 64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x / 64;
  const int64_t rowi = (int64_t)blockIdx.x * (NT / 64 / SPLIT) + wv / SPLIT;
  const int part = wv % SPLIT;
  if constexpr (SPLIT == 1) {
    if (rowi >= rows) return;                    // no block barriers with one wave per row
  }
  const bool live = rowi < rows;                 // with SPLIT > 1 every wave reaches the barrier
  Raw* cand = reinterpret_cast<Raw*>(smem[wv].cand4);
  int* hist = smem[wv].hist;
  const int64_t steps_all = vocab_all / STEP;    // whole steps of the row
  const int64_t per = (steps_all + SPLIT - 1) / SPLIT;
  const int64_t s0 = min((int64_t)part * per, steps_all);
  // this wave's part: whole steps [s0, s0 + nfull), plus the ragged end for the last part
  const T* row = logits + rowi * stride + s0 * STEP;
  const int64_t vocab = (part == SPLIT - 1) ? vocab_all - s0 * STEP : min(per, steps_all - s0) * STEP;
  const int64_t nfull = vocab / STEP;            // steps with every element present

  int count = 0;                                 // list length, a multiple of VEC
  bool exact = false;                            // cand[0..k) is the top-k so far
  uint32_t tau = 0;
  Raw traw = 0;
  bool tpos = true;

  auto append = [&](const uint4& u, bool hit) __attribute__((always_inline)) {  // in lane order, whole vectors
    const uint64_t m = __ballot(hit);
    if (m) {
      if (hit) reinterpret_cast<uint4*>(cand + count)[lanes_below(m)] = u;
      count = __builtin_amdgcn_readfirstlane(count + __builtin_popcountll(m) * VEC);
      exact = false;
    }
  };
  auto select = [&](bool have_tau) __attribute__((always_inline)) {
    tau = __builtin_amdgcn_readfirstlane(reselect<T>(cand, hist, count, k, have_tau, tau));
    count = __builtin_amdgcn_readfirstlane(count);
    traw = (Raw)__builtin_amdgcn_readfirstlane((uint32_t)Tr<T>::raw(tau));
    tpos = !(traw & (Raw)(Tr<T>::kMin ^ (Tr<T>::kMin >> 1)));
    exact = true;
  };
  // the first step: every vector, then the first select (it holds >= k elements)
  auto first = [&](const uint4 (&buf)[NV]) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < NV; ++v) append(buf[v], true);
    select(false);
  };
  // later steps: the vectors holding a key above tau; re-select when long
  auto filter = [&](const uint4 (&buf)[NV]) __attribute__((always_inline)) {
    if (tpos) {
#pragma unroll
      for (int v = 0; v < NV; ++v) append(buf[v], Tr<T>::above_pos(buf[v], traw));
    } else {
#pragma unroll
      for (int v = 0; v < NV; ++v) append(buf[v], Tr<T>::above_neg(buf[v], traw));
    }
    if (count > RESEL) select(true);
  };
  auto load = [&](int64_t c, uint4 (&buf)[NV]) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const T* p = row + c * STEP + (int64_t)(v * 64 + lane) * VEC;
      if constexpr (ALIGNED) {
        buf[v] = ld_stream(p);
      } else {
        const Raw* r = reinterpret_cast<const Raw*>(p);
        Raw e[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) e[i] = r[i];
        __builtin_memcpy(&buf[v], &e, 16);
      }
    }
  };
  auto load_last = [&](uint4 (&buf)[NV]) __attribute__((always_inline)) {       // the ragged last step
#pragma unroll
    for (int v = 0; v < NV; ++v)
      buf[v] = load_tail<T>(row, nfull * STEP + (int64_t)(v * 64 + lane) * VEC, vocab, ALIGNED);
  };
  // Full steps.  The next step's loads are issued before the current step is
  // filtered, and unconditionally (past the end they re-read the last full step,
  // an L2 hit): a load issued on only some paths would make the compiler wait for
  // every outstanding load before each step.
  uint4 ba[NV], bb[NV];
  if (!live) {
  } else if (nfull > 0) {
    const int64_t last = nfull - 1;
    load(0, ba);
    load(min((int64_t)1, last), bb);
    first(ba);
    // whole pairs of steps, no exit in between (an exit between the two halves
    // would also make the compiler wait for the loads in flight at the top)
    int64_t c = 1;                               // bb holds step c
#pragma unroll 1
    for (; c + 1 < nfull; c += 2) {
      load(c + 1, ba);
      filter(bb);
      load(min(c + 2, last), bb);
      filter(ba);
    }
    if (c < nfull) filter(bb);                   // the odd step left over
    if (nfull * STEP < vocab) {
      load_last(ba);
      filter(ba);
    }
  } else {                                       // the row is shorter than a step
    load_last(ba);
    first(ba);
  }
  if (live && !exact) select(true);
  if constexpr (SPLIT > 1) {
    // the row's top-k from its parts' lists (each padded to kr with the
    // smallest key); the first wave of the row gathers them after its own
    const int kr = (k + VEC - 1) / VEC * VEC;
    __syncthreads();
    if (part == 0 && live) {
      for (int q = 1; q < SPLIT; ++q) {
        const Raw* src = reinterpret_cast<const Raw*>(smem[wv + q].cand4);
        for (int i = lane; i < kr; i += 64) cand[q * kr + i] = src[i];
      }
      count = SPLIT * kr;
      select(false);
    }
    if (part != 0 || !live) return;
  }

  // Entropy over the k held keys (float32, fixed reduction order).  With
  // x = t - m <= 0 and Z = sum e^x:  H = ln Z + (1/Z) sum e^x (-x).  A row whose
  // softmax is nearly one-hot has Z = 1 + S with S tiny, and a float32 Z keeps
  // few digits of S: ln Z from it is off by ~6e-8 absolute, which was a 1.7e-3
  // relative error at H = 1.2e-4.  So S is summed apart: the keys equal to m
  // contribute exactly 1 each, one of them is the 1 of Z, and ln Z = log1p(S).
  // Both parts of H are then sums of terms >= 0, accurate to a few ulp.
  float mloc = -INFINITY;
  for (int i = lane; i < k; i += 64) mloc = fmaxf(mloc, Tr<T>::value(Tr<T>::key(cand[i])));
  const float m = wave_max(mloc);
  float sloc = 0.f, hloc = 0.f;
  int ties = 0;
  for (int i = lane; i < k; i += 64) {
    const float t = Tr<T>::value(Tr<T>::key(cand[i]));
    if (t < m) {
      const float e = expf(t - m);
      sloc += e;
      // e = 0 (a -inf logit held because fewer than k are finite, or an
      // underflow) contributes its limit 0, not 0 * inf
      if (e > 0.f) hloc += e * (m - t);
    } else {
      ++ties;
    }
  }
  const float S = wave_sum(sloc) + (float)(wave_sum_int(ties) - 1);
  const float h = log1pf(S) + wave_sum(hloc) / (1.0f + S);
  if (lane == 0) H[rowi] = m == -INFINITY ? NAN : h;   // no finite logit: no entropy
}

template <typename T, int SPLIT>
void launch_split(const void* logits, int64_t rows, int64_t vocab, int64_t stride, int k, float* H,
                  hipStream_t s) {
  constexpr int CAP = RESEL + 64 * Tr<T>::NV * Tr<T>::VEC;
  static_assert(RESEL >= KVC_MAX_TOPK_ENTROPY + 8, "a re-selected list must fit below RESEL");
  constexpr int RPW = NT / 64 / SPLIT;           // rows per workgroup
  const unsigned grid = (unsigned)((rows + RPW - 1) / RPW);
  // every row start is 16-byte aligned iff the base and the row pitch are; a
  // part starts a whole number of 16-byte steps after its row
  const bool aligned = ((uintptr_t)logits % 16 == 0) && ((stride * (int64_t)sizeof(T)) % 16 == 0);
  if (aligned)
    hipLaunchKernelGGL((topk_entropy_kernel<T, CAP, true, SPLIT>), dim3(grid), dim3(NT), 0, s,
                       (const T*)logits, rows, vocab, stride, k, H);
  else
    hipLaunchKernelGGL((topk_entropy_kernel<T, CAP, false, SPLIT>), dim3(grid), dim3(NT), 0, s,
                       (const T*)logits, rows, vocab, stride, k, H);
}

template <typename T>
void launch(const void* logits, int64_t rows, int64_t vocab, int64_t stride, int k, float* H,
            hipStream_t s) {
  constexpr int STEP = 64 * Tr<T>::NV * Tr<T>::VEC;
  constexpr int CAP = RESEL + STEP;
  const int64_t kr = (k + Tr<T>::VEC - 1) / Tr<T>::VEC * Tr<T>::VEC;
  // waves per row: enough for about 16 waves per CU when rows are few, while
  // every part keeps a whole step and the parts' lists fit one list
  auto fits = [&](int sp) { return vocab / STEP >= sp && sp * kr <= CAP; };
  int split = 1;
  if (rows < 4096) split = (rows < 2048 && fits(4)) ? 4 : (fits(2) ? 2 : 1);
  if (split == 4) launch_split<T, 4>(logits, rows, vocab, stride, k, H, s);
  else if (split == 2) launch_split<T, 2>(logits, rows, vocab, stride, k, H, s);
  else launch_split<T, 1>(logits, rows, vocab, stride, k, H, s);
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" int kvc_topk_entropy(const void* logits, int dtype, int64_t rows, int64_t vocab,
                                int64_t row_stride, int topk, float* H_out, void* stream) {
  clear_error();
  if (!dtype_ok(dtype)) return KVC_FAIL(KVC_ERR_DTYPE, "kvc_topk_entropy: dtype %d", dtype);
  KVC_REQUIRE(rows >= 0, "kvc_topk_entropy: rows < 0");
  KVC_REQUIRE(rows <= 0x7fffffffLL * 4, "kvc_topk_entropy: too many rows");
  KVC_REQUIRE(vocab >= 1 && row_stride >= vocab, "kvc_topk_entropy: need 1 <= vocab <= row_stride");
  KVC_REQUIRE(topk >= 1 && topk <= KVC_MAX_TOPK_ENTROPY && topk <= vocab,
              "kvc_topk_entropy: need 1 <= topk <= min(vocab, %d)", KVC_MAX_TOPK_ENTROPY);
  if (rows == 0) return KVC_OK;
  KVC_REQUIRE(logits && H_out, "kvc_topk_entropy: null pointer");
  hipStream_t s = as_stream(stream);
  if (dtype == KVC_BF16) launch<uint16_t>(logits, rows, vocab, row_stride, topk, H_out, s);
  else launch<float>(logits, rows, vocab, row_stride, topk, H_out, s);
  return launch_status("kvc_topk_entropy");
}
