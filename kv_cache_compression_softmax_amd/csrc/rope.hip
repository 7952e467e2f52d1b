// RoPE re-positioning of the kept keys ([SelKV] section 2, pipeline overview,
// step 6): keys that carry the rotary embedding of their original positions are
// re-embedded at contiguous positions, so the compacted cache reads as a
// sequence without gaps.  A rotation by angle a followed by one by b is the
// rotation by a + b, so each pair only turns by (new - old) times its frequency.
//
// Pairing: element i with element i + d/2 (the half-split layout), frequency
// base^(-2i/d).  The angle delta * frequency reaches ~1e5 rad at long contexts,
// so it is formed and reduced to [-pi, pi] in float64; the rotation itself runs
// in float32 and bf16 results are rounded to nearest even.
//
// One thread per (row, pair): a wave covers the pairs of one row (d = 128), so
// a row's two halves are each read and written as one contiguous segment.
#include "common.h"

namespace kvc {
namespace {

constexpr int NT = 256;

struct RopeTables { MutPtrs K; ConstPtrs pos; };

template <typename T> __device__ __forceinline__ float ld_el(const T* p);
template <> __device__ __forceinline__ float ld_el<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <> __device__ __forceinline__ float ld_el<float>(const float* p) { return *p; }
__device__ __forceinline__ void st_el(uint16_t* p, float v) { *p = f32_to_bf16_rne(v); }
__device__ __forceinline__ void st_el(float* p, float v) { *p = v; }

template <typename T>
__global__ void __launch_bounds__(NT)
rope_kernel(RopeTables t, int lc, int Hkv, int64_t m, int d, int64_t new0, double log2_base) {
  const int h = d / 2;
  const int64_t id = (int64_t)blockIdx.x * NT + threadIdx.x;
  const int64_t rows = (int64_t)lc * Hkv * m;
  if (id >= rows * h) return;
  const int i = (int)(id % h);
  const int64_t row = id / h;                   // (layer, KV head, slot)
  const int64_t j = row % m;
  const int64_t lg = row / m;
  const int l = (int)(lg / Hkv), g = (int)(lg % Hkv);
  const int32_t* pos = (const int32_t*)t.pos.p[l] + (int64_t)g * m;
  T* k = (T*)t.K.p[l] + ((int64_t)g * m + j) * d;
  const double freq = exp2(-2.0 * (double)i / (double)d * log2_base);
  const double ang = (double)(new0 + j - (int64_t)pos[j]) * freq;
  const double two_pi = 6.283185307179586476925286766559;
  const float r = (float)(ang - two_pi * rint(ang / two_pi));
  float sn, cs;
  sincosf(r, &sn, &cs);
  const float a = ld_el<T>(k + i), b = ld_el<T>(k + i + h);
  st_el(k + i, a * cs - b * sn);
  st_el(k + i + h, a * sn + b * cs);
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
  for (int l0 = 0; l0 < L; l0 += kLayersPerLaunch) {
    const int lc = min(kLayersPerLaunch, L - l0);
    RopeTables t{};
    for (int i = 0; i < lc; ++i) { t.K.p[i] = K[l0 + i]; t.pos.p[i] = pos_old[l0 + i]; }
    const int64_t total = (int64_t)lc * Hkv * m * (d / 2);
    KVC_REQUIRE((total + NT - 1) / NT <= 0x7fffffffLL, "kvc_rope_reposition: too many rows");
    const dim3 grid((unsigned)((total + NT - 1) / NT));
    if (dtype == KVC_BF16) hipLaunchKernelGGL(rope_kernel<uint16_t>, grid, dim3(NT), 0, s, t, lc, Hkv, m, d, new_pos0, lb);
    else hipLaunchKernelGGL(rope_kernel<float>, grid, dim3(NT), 0, s, t, lc, Hkv, m, d, new_pos0, lb);
  }
  return launch_status("kvc_rope_reposition");
}
