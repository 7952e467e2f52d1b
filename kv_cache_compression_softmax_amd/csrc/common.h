// Internal helpers shared by the HIP sources of libkvc (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "kvc.h"

namespace kvc {

// ---------------------------------------------------------------- host side
// Per-thread message of the last failure (kvc_last_error).
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

// Returns `status` after recording a message.
#define KVC_FAIL(status, ...) (::kvc::set_error(__VA_ARGS__), (status))
#define KVC_REQUIRE(cond, ...) \
  do { if (!(cond)) return KVC_FAIL(KVC_ERR_ARG, __VA_ARGS__); } while (0)

// Checks hipGetLastError() after launches; returns KVC_OK or KVC_ERR_HIP.
int launch_status(const char* what);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline int dtype_size(int dtype) { return dtype == KVC_F32 ? 4 : 2; }
inline bool dtype_ok(int dtype) { return dtype == KVC_F32 || dtype == KVC_BF16; }

// A launch covers at most this many layers; the host loops over chunks.  Per-layer
// device pointers travel by value in the kernel arguments.
constexpr int kLayersPerLaunch = 32;

struct ConstPtrs { const void* p[kLayersPerLaunch]; };
struct MutPtrs { void* p[kLayersPerLaunch]; };
struct I64s { int64_t v[kLayersPerLaunch]; };

// ------------------------------------------------------------- device side
constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16 bits, round to nearest, ties to even (inputs finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// 16-byte load marked non-temporal, for data read exactly once: a plain streaming
// read reaches up to 7.1 TB/s this way against 6.2-6.3 TB/s with ordinary loads.
// Not for data read again soon (it loses the MALL: window attention's second pass
// over K slows from 1.03 to 1.47 ms with it).
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
// 16-byte store marked non-temporal, for output not read again soon (gathered or
// merged cache rows): the gather of kept rows runs 4-7% faster with it.
__device__ __forceinline__ void st_stream(void* p, uint4 v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = width / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive prefix sum across a block of NT threads (NT a multiple of 64, at most
// 1024).  `tmp` is shared memory of at least NT/64 ints.  Returns the exclusive
// sum; *total receives the block total.  Contains two barriers.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) tmp[wv] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    int s = tmp[i];
    base += (i < wv) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// Block-wide reductions for NT threads; `tmp` holds NT/64 floats.  Fixed order.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* tmp) {
  constexpr int NW = NT / kWave;
  v = wave_sum(v);
  if ((threadIdx.x & (kWave - 1)) == 0) tmp[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) r += tmp[i];
  __syncthreads();
  return r;
}
template <int NT>
__device__ __forceinline__ float block_max(float v, float* tmp) {
  constexpr int NW = NT / kWave;
  v = wave_max(v);
  if ((threadIdx.x & (kWave - 1)) == 0) tmp[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = -INFINITY;
#pragma unroll
  for (int i = 0; i < NW; ++i) r = fmaxf(r, tmp[i]);
  __syncthreads();
  return r;
}

// Order-preserving integer keys: a > b as floats  <=>  key(a) > key(b).
// -0.0 is mapped to the key of +0.0 so that equal floats get equal keys.
__device__ __forceinline__ uint32_t f32_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint32_t bf16_key(uint32_t b) {   // b: 16-bit pattern
  if (b == 0x8000u) b = 0;
  return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u);
}
__device__ __forceinline__ float key_bf16(uint32_t k) {
  uint32_t b = (k & 0x8000u) ? (k & 0x7fffu) : (~k & 0xffffu);
  return __uint_as_float(b << 16);
}

}  // namespace kvc
