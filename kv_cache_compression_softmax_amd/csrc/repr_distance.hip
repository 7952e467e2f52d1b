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
// Loads are 16 bytes per lane and a wave instruction covers 1 KB of one row.  Two
// layer rows are held in turn: the next layer's row is in flight while the current
// one is reduced.  bf16 products go through v_dot2_f32_bf16 (two products and the
// float32 accumulate in one instruction, no unpacking).
#include "common.h"

namespace kvc {
namespace {

constexpr int NT = 256;          // 4 waves = 4 tokens per workgroup
constexpr int MAXV = 16;         // most 16-byte vectors per lane kept in registers

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <typename T> struct VecT;
template <> struct VecT<uint16_t> { static constexpr int N = 8; };
template <> struct VecT<float> { static constexpr int N = 4; };

// acc[j] += <x, y> over the 16-byte vector's elements (4 independent sums)
template <typename T>
__device__ __forceinline__ void dot_acc(const uint4& x, const uint4& y, float (&acc)[4]);
template <>
__device__ __forceinline__ void dot_acc<uint16_t>(const uint4& x, const uint4& y, float (&acc)[4]) {
  acc[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.x),
                                           __builtin_bit_cast(bf16x2, y.x), acc[0], false);
  acc[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.y),
                                           __builtin_bit_cast(bf16x2, y.y), acc[1], false);
  acc[2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.z),
                                           __builtin_bit_cast(bf16x2, y.z), acc[2], false);
  acc[3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.w),
                                           __builtin_bit_cast(bf16x2, y.w), acc[3], false);
}
template <>
__device__ __forceinline__ void dot_acc<float>(const uint4& x, const uint4& y, float (&acc)[4]) {
  acc[0] = fmaf(__uint_as_float(x.x), __uint_as_float(y.x), acc[0]);
  acc[1] = fmaf(__uint_as_float(x.y), __uint_as_float(y.y), acc[1]);
  acc[2] = fmaf(__uint_as_float(x.z), __uint_as_float(y.z), acc[2]);
  acc[3] = fmaf(__uint_as_float(x.w), __uint_as_float(y.w), acc[3]);
}

__device__ __forceinline__ float distance(float dot, float na2, float nb2, float tau) {
  float den = sqrtf(na2) * sqrtf(nb2);
  float c = den > 0.f ? dot / den : 0.f;
  return 1.0f - c + tau;
}

// Fast path: rows 16-byte aligned, hidden a multiple of the vector width and at
// most 64 * V vectors (V = vectors per lane held in registers); FULL: exactly
// 64 * V, so no lane skips a vector.
template <typename T, int V, bool FULL>
__global__ void __launch_bounds__(NT)
repr_distance_vec(ConstPtrs h, const T* __restrict__ hf, int L, int64_t n, int64_t hidden,
                  float tau, float* __restrict__ D) {
  constexpr int W = VecT<T>::N;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t tok = (int64_t)blockIdx.x * (NT / kWave) + threadIdx.x / kWave;
  if (tok >= n) return;
  const int nvec = (int)(hidden / W);             // vectors per row
  const int64_t roff = tok * hidden;
  // The rows are read-only, so the compiler may re-issue a prefetch where its data
  // is used; the empty asm with a memory clobber keeps each load where it stands.
  auto load = [&](const T* row, uint4 (&a)[V]) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int vi = v * kWave + lane;
      if (FULL || vi < nvec) a[v] = ld_stream(row + (int64_t)vi * W);
      else a[v] = make_uint4(0u, 0u, 0u, 0u);      // contributes 0 to every sum
    }
    asm volatile("" ::: "memory");
  };
  uint4 b[V];
  load(hf + roff, b);
  float nb2;
  {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < V; ++v) dot_acc<T>(b[v], b[v], acc);
    nb2 = wave_sum((acc[0] + acc[1]) + (acc[2] + acc[3]));
  }
  // lane l keeps layer l's result (L <= 64 per launch); one store per lane at the
  // end, so the layer loop is a single basic block the scheduler keeps in order
  float mine = 0.f;
  auto layer = [&](int l, const uint4 (&a)[V]) __attribute__((always_inline)) {
    float d4[4] = {0.f, 0.f, 0.f, 0.f}, n4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < V; ++v) { dot_acc<T>(a[v], b[v], d4); dot_acc<T>(a[v], a[v], n4); }
    const float dot = wave_sum((d4[0] + d4[1]) + (d4[2] + d4[3]));
    const float na2 = wave_sum((n4[0] + n4[1]) + (n4[2] + n4[3]));
    float dist = distance(dot, na2, nb2, tau);
    asm volatile("" : "+v"(dist));               // computed by every lane, then selected
    mine = lane == l ? dist : mine;
  };
  // Layers in pairs, two rows in turn.  Inside the loop every load is
  // unconditional and no exit sits between the halves, so the compiler never has
  // to wait for the row that is still in flight.  The loop stops while two or
  // three layers remain, so no load reaches past the last layer (a clamped
  // re-read of it would miss L2: its rows were read non-temporally).
  uint4 a0[V], a1[V];
  load((const T*)h.p[0] + roff, a0);
  if (L > 1) load((const T*)h.p[1] + roff, a1);
  int l = 0;
#pragma unroll 1
  for (; l + 3 < L; l += 2) {
    // the barriers keep each refill behind the last read of its buffer, so the
    // new row lands in the same registers (no copies of rows still in flight)
    layer(l, a0);
    __builtin_amdgcn_sched_barrier(0);
    load((const T*)h.p[l + 2] + roff, a0);
    layer(l + 1, a1);
    __builtin_amdgcn_sched_barrier(0);
    load((const T*)h.p[l + 3] + roff, a1);
  }
  // 1, 2 or 3 layers remain: l, l + 1 (in a1), l + 2 (reloaded into a0)
  layer(l, a0);
  if (l + 2 < L) {
    __builtin_amdgcn_sched_barrier(0);
    load((const T*)h.p[l + 2] + roff, a0);
  }
  if (l + 1 < L) layer(l + 1, a1);
  if (l + 2 < L) layer(l + 2, a0);
  if (lane < L) D[(int64_t)lane * n + tok] = mine;
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
    do {                                                                                      \
      if (hidden / W == (int64_t)(VV) * kWave)                                                \
        hipLaunchKernelGGL((repr_distance_vec<T, VV, true>), dim3(grid), dim3(NT), 0, s, tab, \
                           (const T*)h_final, lc, n, hidden, tau, Dl);                        \
      else                                                                                    \
        hipLaunchKernelGGL((repr_distance_vec<T, VV, false>), dim3(grid), dim3(NT), 0, s, tab,\
                           (const T*)h_final, lc, n, hidden, tau, Dl);                        \
    } while (0)
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
