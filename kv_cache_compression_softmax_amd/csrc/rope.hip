// RoPE re-positioning of the kept keys ([SelKV] section 2, pipeline overview,
// step 6): keys that carry the rotary embedding of their original positions are
// re-embedded at contiguous positions, so the compacted cache reads as a
// sequence without gaps.  A rotation by angle a followed by one by b is the
// rotation by a + b, so each pair only turns by (new - old) times its frequency.
//
// Pairing: element i with element i + d/2 (the half-split layout), frequency
// base^(-2i/d).  The angle delta * frequency reaches ~1e5 rad at long contexts,
// so it is formed and reduced to [-pi, pi] in float64; the sine, cosine and
// rotation run in float32 and bf16 results are rounded to nearest even.
//
// For d = 4 .. 128 (a power of two) a lane turns two neighbouring pairs with
// one 2-element load and one 2-element store per half, and a wave covers
// 128/(d/2) rows per step, eight steps' loads in flight; other shapes take one
// row per wave, one pair per lane at a time.  Either way a row's halves are read and written as contiguous
// segments.
#include "common.h"

namespace kvc {
namespace {

constexpr int NT = 256;

struct RopeTables { MutPtrs K; ConstPtrs pos; };

// two consecutive elements, loaded as one
template <typename T> struct P2T;
template <> struct P2T<uint16_t> { using type = uint32_t; };
template <> struct P2T<float> { using type = float2; };
template <typename T> using P2 = typename P2T<T>::type;
// read once and written once: bf16 pairs use non-temporal loads and stores
__device__ __forceinline__ uint32_t ld_p2(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ float2 ld_p2(const float* p) { return *reinterpret_cast<const float2*>(p); }
__device__ __forceinline__ float p2_lo(uint32_t v) { return bf16_lo(v); }
__device__ __forceinline__ float p2_hi(uint32_t v) { return bf16_hi(v); }
__device__ __forceinline__ float p2_lo(float2 v) { return v.x; }
__device__ __forceinline__ float p2_hi(float2 v) { return v.y; }

template <typename T> __device__ __forceinline__ float ld_el(const T* p);
template <> __device__ __forceinline__ float ld_el<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <> __device__ __forceinline__ float ld_el<float>(const float* p) { return *p; }
__device__ __forceinline__ void st_el(uint16_t* p, float v) { *p = f32_to_bf16_rne(v); }
__device__ __forceinline__ void st_el(float* p, float v) { *p = v; }
// two consecutive elements, stored as one
__device__ __forceinline__ void st_p2(uint16_t* p, float lo, float hi) {
  __builtin_nontemporal_store((uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16),
                              reinterpret_cast<uint32_t*>(p));
}
__device__ __forceinline__ void st_p2(float* p, float lo, float hi) {
  *reinterpret_cast<float2*>(p) = make_float2(lo, hi);
}

constexpr int RPB = 8;         // blocks per (layer, KV head)
constexpr int RW = 8;          // rows per wave step when d <= 128

// One wave per row at a time, looping over the rows of its (layer, KV head); lane
// i turns pairs i, i + 64, ...  The shift new - old is the same for the whole row
// (wave-uniform); for d <= 128 each lane's one frequency is computed once.
template <typename T>
__global__ void __launch_bounds__(NT)
rope_kernel(RopeTables t, int Hkv, int64_t m, int d, int64_t new0, double log2_base, int paired) {
  const int lg = blockIdx.y;                    // (layer, KV head)
  const int l = lg / Hkv, g = lg % Hkv;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = d / 2;
  const int32_t* pos = (const int32_t*)t.pos.p[l] + (int64_t)g * m;
  T* kg = (T*)t.K.p[l] + (int64_t)g * m * d;
  const double inv_two_pi = 0.15915494309189533576888376337251;
  const double two_pi = 6.283185307179586476925286766559;
  // frequency of pair i: base^(-2i/d)
  auto freq = [&](int i) __attribute__((always_inline)) {
    return exp2(-2.0 * (double)i / (double)d * log2_base);
  };
  // (a, b) turned by delta * f: (a cos - b sin, a sin + b cos)
  auto rot = [&](int64_t delta, double f, float a, float b, float& x, float& y) __attribute__((always_inline)) {
    const double ang = (double)delta * f;
    const float r = (float)fma(-two_pi, rint(ang * inv_two_pi), ang);
    // the hardware sine and cosine: on [-pi, pi] their error was measured at
    // most 2.7e-7 (absolute), against the float32 rotation's own rounding
    const float sn = __sinf(r), cs = __cosf(r);
    x = a * cs - b * sn;
    y = a * sn + b * cs;
  };
  auto turn = [&](int64_t delta, int i, double f, float a, float b, T* k) __attribute__((always_inline)) {
    float x, y;
    rot(delta, f, a, b, x, y);
    st_el(k + i, x);
    st_el(k + i + h, y);
  };
  const int64_t nw = (int64_t)gridDim.x * (NT / 64);
  int64_t j = (int64_t)blockIdx.x * (NT / 64) + wv;
  if (paired) {                                 // h a power of two <= 64, rows 8-byte aligned
    // two pairs per lane (elements 2q, 2q + 1 of each half, one 2-element load
    // per half), 128 / h rows per wave step; RW steps' loads issued before any
    // is used
    const int lpr = h / 2;                       // lanes per row
    const int rpw = 64 / lpr;                    // rows per wave step
    const int sub = lane / lpr, q = 2 * (lane % lpr);
    const double f0 = freq(q), f1 = freq(q + 1);
    const int64_t stride = nw * rpw;             // rows between a wave's steps
    for (j = ((int64_t)blockIdx.x * (NT / 64) + wv) * rpw + sub; j < m; j += RW * stride) {
      P2<T> a[RW], b[RW];
      int64_t dl[RW];
#pragma unroll
      for (int u = 0; u < RW; ++u) {
        const int64_t ju = min(j + u * stride, m - 1);      // clamped: loaded, not stored
        dl[u] = new0 + ju - (int64_t)pos[ju];
        const T* k = kg + ju * d;
        a[u] = ld_p2(k + q);
        b[u] = ld_p2(k + q + h);
      }
#pragma unroll
      for (int u = 0; u < RW; ++u) {
        const int64_t ju = j + u * stride;
        if (ju < m) {
          T* k = kg + ju * d;
          float x0, y0, x1, y1;
          rot(dl[u], f0, p2_lo(a[u]), p2_lo(b[u]), x0, y0);
          rot(dl[u], f1, p2_hi(a[u]), p2_hi(b[u]), x1, y1);
          st_p2(k + q, x0, x1);                   // one 2-element store per half
          st_p2(k + q + h, y0, y1);
        }
      }
    }
  } else {
    for (; j < m; j += nw) {
      const int64_t delta = new0 + j - (int64_t)pos[j];
      T* k = kg + j * d;
      for (int i = lane; i < h; i += 64) turn(delta, i, freq(i), ld_el<T>(k + i), ld_el<T>(k + i + h), k);
    }
  }
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" int kvc_rope_reposition(void* const* K, int dtype, const int32_t* const* pos_old,
                                   int64_t new_pos0, double base, int L, int Hkv, int64_t m, int d,
                                   void* stream) {
  clear_error();
  if (!dtype_ok(dtype)) return KVC_FAIL(KVC_ERR_DTYPE, "kvc_rope_reposition: dtype %d", dtype);
  KVC_REQUIRE(L >= 1 && L <= KVC_MAX_LAYERS, "kvc_rope_reposition: need 1 <= L <= %d", KVC_MAX_LAYERS);
  KVC_REQUIRE(Hkv >= 1 && m >= 1 && m <= 0x7fffffffLL, "kvc_rope_reposition: need Hkv >= 1, 1 <= m < 2^31");
  KVC_REQUIRE(d >= 2 && d % 2 == 0 && d <= 4096, "kvc_rope_reposition: need an even 2 <= d <= 4096");
  KVC_REQUIRE(base > 1.0, "kvc_rope_reposition: need base > 1");
  KVC_REQUIRE(new_pos0 >= 0 && new_pos0 <= 0x7fffffffLL, "kvc_rope_reposition: need 0 <= new_pos0 < 2^31");
  KVC_REQUIRE(K && pos_old, "kvc_rope_reposition: null pointer");
  for (int l = 0; l < L; ++l)
    KVC_REQUIRE(K[l] && pos_old[l], "kvc_rope_reposition: null pointer in layer %d", l);
  hipStream_t s = as_stream(stream);
  const double lb = log2(base);
  // two pairs per lane with 2-element loads: h = d/2 a power of two up to 64 (so
  // the lanes of a row divide the wave), every row 8-byte aligned
  const int h = d / 2;
  int paired = h >= 2 && h <= 64 && (h & (h - 1)) == 0;
  for (int l = 0; l < L; ++l) paired = paired && (uintptr_t)K[l] % 8 == 0;
  for (int l0 = 0; l0 < L; l0 += kLayersPerLaunch) {
    const int lc = min(kLayersPerLaunch, L - l0);
    RopeTables t{};
    for (int i = 0; i < lc; ++i) { t.K.p[i] = K[l0 + i]; t.pos.p[i] = pos_old[l0 + i]; }
    KVC_REQUIRE((int64_t)lc * Hkv <= 65535, "kvc_rope_reposition: L * Hkv > 65535");
    const dim3 grid((unsigned)RPB, (unsigned)(lc * Hkv));
    if (dtype == KVC_BF16) hipLaunchKernelGGL(rope_kernel<uint16_t>, grid, dim3(NT), 0, s, t, Hkv, m, d, new_pos0, lb, paired);
    else hipLaunchKernelGGL(rope_kernel<float>, grid, dim3(NT), 0, s, t, Hkv, m, d, new_pos0, lb, paired);
  }
  return launch_status("kvc_rope_reposition");
}
