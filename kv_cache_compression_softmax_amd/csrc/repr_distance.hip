// Layer-wise representation distance D[l, i] = 1 - cos(h_l[i], h_final[i]) + tau.
//
// [InfoKV] Method, Technical detail and Glossary (layer-wise representation
// evolution): the cosine distance between a token's hidden state at layer l and
// at the last layer, plus a small bias tau.
//
// The work is one pass over L+1 hidden-state tensors, so it is bound by HBM.  One
// wave owns one token: it loads the token's final-layer row once into registers
// (hidden/64 elements per lane), then streams the same row of every layer,
// accumulating <a, b> and |a|^2 per lane in float32 and reducing across the wave.
// Loads are 16 bytes per lane and a wave instruction covers 1 KB of one row.  The
// next layer's row is requested before the current one is reduced.
#include "common.h"

namespace kvc {
namespace {

constexpr int NT = 256;          // 4 waves = 4 tokens per workgroup
constexpr int MAXV = 16;         // most 16-byte vectors per lane kept in registers

template <typename T> struct VecT;
template <> struct VecT<uint16_t> { static constexpr int N = 8; };
template <> struct VecT<float> { static constexpr int N = 4; };

template <typename T>
__device__ __forceinline__ void unpack(const uint4& u, float (&x)[VecT<T>::N]);
template <>
__device__ __forceinline__ void unpack<uint16_t>(const uint4& u, float (&x)[8]) {
  x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
  x[4] = bf16_lo(u.z); x[5] = bf16_hi(u.z); x[6] = bf16_lo(u.w); x[7] = bf16_hi(u.w);
}
template <>
__device__ __forceinline__ void unpack<float>(const uint4& u, float (&x)[4]) {
  x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
  x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
}

__device__ __forceinline__ float distance(float dot, float na2, float nb2, float tau) {
  float den = sqrtf(na2) * sqrtf(nb2);
  float c = den > 0.f ? dot / den : 0.f;
  return 1.0f - c + tau;
}

// Fast path: rows 16-byte aligned, hidden a multiple of the vector width and at
// most 64 * V vectors (V = vectors per lane held in registers).
template <typename T, int V>
__global__ void __launch_bounds__(NT)
repr_distance_vec(ConstPtrs h, const T* __restrict__ hf, int L, int64_t n, int64_t hidden,
                  float tau, float* __restrict__ D) {
  constexpr int W = VecT<T>::N;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t tok = (int64_t)blockIdx.x * (NT / kWave) + threadIdx.x / kWave;
  if (tok >= n) return;
  const int nvec = (int)(hidden / W);             // vectors per row
  const int64_t roff = tok * hidden;
  uint4 b[V];
  float nb2 = 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int vi = v * kWave + lane;
    if (vi < nvec) {
      b[v] = *reinterpret_cast<const uint4*>(hf + roff + (int64_t)vi * W);
      float x[W];
      unpack<T>(b[v], x);
#pragma unroll
      for (int e = 0; e < W; ++e) nb2 += x[e] * x[e];
    }
  }
  nb2 = wave_sum(nb2);
  uint4 a[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int vi = v * kWave + lane;
    if (vi < nvec) a[v] = *reinterpret_cast<const uint4*>((const T*)h.p[0] + roff + (int64_t)vi * W);
  }
#pragma unroll 1
  for (int l = 0; l < L; ++l) {
    float dot = 0.f, na2 = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int vi = v * kWave + lane;
      if (vi < nvec) {
        float x[W], y[W];
        unpack<T>(a[v], x);
        unpack<T>(b[v], y);
#pragma unroll
        for (int e = 0; e < W; ++e) { dot += x[e] * y[e]; na2 += x[e] * x[e]; }
      }
    }
    if (l + 1 < L) {                        // next layer's row while this one reduces
      const T* nl = (const T*)h.p[l + 1] + roff;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int vi = v * kWave + lane;
        if (vi < nvec) a[v] = *reinterpret_cast<const uint4*>(nl + (int64_t)vi * W);
      }
    }
    dot = wave_sum(dot);
    na2 = wave_sum(na2);
    if (lane == 0) D[(int64_t)l * n + tok] = distance(dot, na2, nb2, tau);
  }
}

template <typename T> __device__ __forceinline__ float ld(const T* p);
template <> __device__ __forceinline__ float ld<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <> __device__ __forceinline__ float ld<float>(const float* p) { return *p; }

// General path: any alignment and width (element loads, final row re-read per layer).
template <typename T>
__global__ void __launch_bounds__(NT)
repr_distance_any(ConstPtrs h, const T* __restrict__ hf, int L, int64_t n, int64_t hidden,
                  float tau, float* __restrict__ D) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t tok = (int64_t)blockIdx.x * (NT / kWave) + threadIdx.x / kWave;
  if (tok >= n) return;
  const int64_t roff = tok * hidden;
  float nb2 = 0.f;
  for (int64_t j = lane; j < hidden; j += kWave) { float y = ld<T>(hf + roff + j); nb2 += y * y; }
  nb2 = wave_sum(nb2);
  for (int l = 0; l < L; ++l) {
    const T* a = (const T*)h.p[l] + roff;
    float dot = 0.f, na2 = 0.f;
    for (int64_t j = lane; j < hidden; j += kWave) {
      float x = ld<T>(a + j), y = ld<T>(hf + roff + j);
      dot += x * y; na2 += x * x;
    }
    dot = wave_sum(dot);
    na2 = wave_sum(na2);
    if (lane == 0) D[(int64_t)l * n + tok] = distance(dot, na2, nb2, tau);
  }
}

template <typename T>
int launch(const void* const* h_layers, const void* h_final, int L, int64_t n, int64_t hidden,
           float tau, float* D, hipStream_t s) {
  constexpr int W = VecT<T>::N;
  bool vec = (hidden % W == 0) && (hidden / W <= (int64_t)MAXV * kWave) &&
             ((uintptr_t)h_final % 16 == 0);
  for (int l = 0; l < L; ++l) vec = vec && ((uintptr_t)h_layers[l] % 16 == 0);
  const unsigned grid = (unsigned)((n + NT / kWave - 1) / (NT / kWave));
  for (int l0 = 0; l0 < L; l0 += kLayersPerLaunch) {
    const int lc = min(kLayersPerLaunch, L - l0);
    ConstPtrs tab{};
    for (int i = 0; i < lc; ++i) tab.p[i] = h_layers[l0 + i];
    float* Dl = D + (int64_t)l0 * n;
    const int64_t per_lane = (hidden / W + kWave - 1) / kWave;
#define KVC_RD_LAUNCH(VV)                                                                     \
    hipLaunchKernelGGL((repr_distance_vec<T, VV>), dim3(grid), dim3(NT), 0, s, tab,          \
                       (const T*)h_final, lc, n, hidden, tau, Dl)
    if (vec && per_lane <= 1) KVC_RD_LAUNCH(1);
    else if (vec && per_lane <= 2) KVC_RD_LAUNCH(2);
    else if (vec && per_lane <= 4) KVC_RD_LAUNCH(4);
    else if (vec && per_lane <= 6) KVC_RD_LAUNCH(6);
    else if (vec && per_lane <= 8) KVC_RD_LAUNCH(8);
    else if (vec && per_lane <= 12) KVC_RD_LAUNCH(12);
    else if (vec) KVC_RD_LAUNCH(16);
#undef KVC_RD_LAUNCH
    else
      hipLaunchKernelGGL(repr_distance_any<T>, dim3(grid), dim3(NT), 0, s, tab, (const T*)h_final,
                         lc, n, hidden, tau, Dl);
  }
  return launch_status("kvc_repr_distance");
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" int kvc_repr_distance(const void* const* h_layers, const void* h_final, int dtype,
                                 int L, int64_t n, int64_t hidden, float tau, float* D_out,
                                 void* stream) {
  clear_error();
  if (!dtype_ok(dtype)) return KVC_FAIL(KVC_ERR_DTYPE, "kvc_repr_distance: dtype %d", dtype);
  KVC_REQUIRE(L >= 1 && L <= KVC_MAX_LAYERS, "kvc_repr_distance: need 1 <= L <= %d", KVC_MAX_LAYERS);
  KVC_REQUIRE(n >= 0 && hidden >= 1, "kvc_repr_distance: need n >= 0, hidden >= 1");
  KVC_REQUIRE((n + 3) / 4 <= 0x7fffffff, "kvc_repr_distance: n too large");
  if (n == 0) return KVC_OK;
  KVC_REQUIRE(h_layers && h_final && D_out, "kvc_repr_distance: null pointer");
  for (int l = 0; l < L; ++l) KVC_REQUIRE(h_layers[l], "kvc_repr_distance: h_layers[%d] is null", l);
  hipStream_t s = as_stream(stream);
  return dtype == KVC_BF16 ? launch<uint16_t>(h_layers, h_final, L, n, hidden, tau, D_out, s)
                           : launch<float>(h_layers, h_final, L, n, hidden, tau, D_out, s);
}
