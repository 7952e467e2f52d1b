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
constexpr int NTR = 768;        // threads of the register path (3 waves per SIMD)
constexpr int REGV = 34;        // 16-byte vectors per thread held in registers (REG path)

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
// dynamic LDS, as float4, from the first pass on.  REG (with VEC): [0, n - w) is
// held in registers, REGV vectors per thread.
template <bool VEC, bool CACHE, bool REG = false>
__global__ void __launch_bounds__(REG ? NTR : NT)
select_kernel(const float* __restrict__ S, int Hkv, int64_t n, I64s kk, int w, MutPtrs idx) {
  constexpr int NTB = REG ? NTR : NT;             // threads of this variant
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
  // REG: the thread's vectors t + r * NTB, loaded once, all in flight together
  // (vectors past the row repeat its last one and are never counted)
  // (held as order-preserving keys, converted once)
  uint4 rk[REG ? REGV : 1];
  if constexpr (REG) {
    const int64_t nv = (nb + 3) / 4;
    const float4* row4 = reinterpret_cast<const float4*>(row);
    float4 t[REG ? REGV : 1];
#pragma unroll
    for (int r = 0; r < REGV; ++r) t[r] = row4[min((int64_t)r * NTB + tid, nv - 1)];
#pragma unroll
    for (int r = 0; r < REGV; ++r)
      rk[r] = make_uint4(f32_key(t[r].x), f32_key(t[r].y), f32_key(t[r].z), f32_key(t[r].w));
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
    if constexpr (REG) {
      // element 4 (r NTB + tid) + q is in the row iff 4 r NTB + q < lim: a
      // constant against one register
      const int lim = (int)nb - 4 * tid;
#pragma unroll
      for (int r = 0; r < REGV; ++r) {
        count(rk[r].x, 4 * r * NTB + 0 < lim);
        count(rk[r].y, 4 * r * NTB + 1 < lim);
        count(rk[r].z, 4 * r * NTB + 2 < lim);
        count(rk[r].w, 4 * r * NTB + 3 < lim);
      }
    } else if constexpr (VEC) {
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
  if constexpr (REG) {
    // chunk r of the ordered pass is vector r * NTB + tid of this thread: registers
#pragma unroll
    for (int r = 0; r < REGV; ++r) {
      // 32-bit index arithmetic: n < 2^31
      if (r * NTB * EPT >= (int)nb) break;        // uniform
      const int i0 = r * NTB * EPT + tid * EPT;
      const int lim = (int)nb - 4 * tid;
      const uint32_t k4[EPT] = {rk[r].x, rk[r].y, rk[r].z, rk[r].w};
      uint32_t gt = 0, eq = 0;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const uint32_t key = k4[e];
        const bool in = 4 * r * NTB + e < lim;
        gt |= (uint32_t)(in && key > T) << e;
        eq |= (uint32_t)(in && key == T) << e;
      }
      const int packed = __builtin_popcount(gt) | (__builtin_popcount(eq) << 16);
      int tot;
      const int ex = block_exclusive_scan<NTB>(packed, scan, &tot);
      int gtb = (int)run_gt + (ex & 0xffff), eqb = (int)run_eq + (ex >> 16);
      const int teq = (int)take_eq;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        if (gt & (1u << e)) {
          out[gtb + min(eqb, teq)] = i0 + e;
          ++gtb;
        } else if (eq & (1u << e)) {
          if (eqb < teq) out[gtb + eqb] = i0 + e;
          ++eqb;
        }
      }
      run_gt += tot & 0xffff;
      run_eq += tot >> 16;
    }
    return;
  }
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
    else if (use_reg) hipLaunchKernelGGL((select_kernel<true, false, true>), grid, dim3(NTR), 0, s, Sl, Hkv, n, kk, w, ip);
    else if (vec) hipLaunchKernelGGL((select_kernel<true, false>), grid, dim3(NT), 0, s, Sl, Hkv, n, kk, w, ip);
    else hipLaunchKernelGGL((select_kernel<false, false>), grid, dim3(NT), 0, s, Sl, Hkv, n, kk, w, ip);
  }
  return launch_status("kvc_select_topk");
}
