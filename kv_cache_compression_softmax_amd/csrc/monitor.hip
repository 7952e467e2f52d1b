// Dropped-attention-mass monitor of a compacted cache ([RECAS] section 2.B,
// error-bounded compression: the formal bound and its periodic full-attention
// probe steps).
//
// At a probe step the decode query is attended twice: over the full cache and
// over the kept rows only (kvc_decode_attn, no bias).  The two log normalisers
// give the evicted tokens' share of the full softmax exactly,
//   delta = 1 - sum_kept p = 1 - exp(lse_kept - lse_full),
// and the bound ||o - o'||_2 <= 2 * V_max * delta needs V_max, the largest value
// norm of the full cache.  One workgroup per (layer, KV head) streams that head's
// V rows once (non-temporal 16-byte loads, several rows in flight per lane),
// keeps the largest squared norm, and then writes delta and the bound for the
// group's query heads.  No workspace, no atomics: the result does not depend on
// the order of the rows.
#include <cmath>

#include "common.h"

namespace kvc {
namespace {

constexpr int NT = 1024;
constexpr int NW = NT / kWave;
constexpr int RU = 4;           // rows per lane group with loads in flight together

struct MonTables {
  ConstPtrs V;
};

// delta and the bound of the group's query heads, from the workgroup's V_max
__device__ __forceinline__ void write_group(float vmax2, int l, int g, int Hq, int G,
                                            const float* lse_kept, const float* lse_full,
                                            float* delta, float* vmax_out, float* bound) {
  const float vmax = sqrtf(vmax2);
  if (threadIdx.x == 0) vmax_out[l * (Hq / G) + g] = vmax;
  if ((int)threadIdx.x < G) {
    const int64_t h = (int64_t)l * Hq + (int64_t)g * G + threadIdx.x;
    // exp(lse_kept - lse_full) is the kept share (<= 1 up to rounding)
    const float dl = fmaxf(-expm1f(lse_kept[h] - lse_full[h]), 0.f);
    delta[h] = dl;
    bound[h] = 2.f * vmax * dl;
  }
}

// Rows of 16-byte multiples: LPR lanes per row (LPR divides 64), 16 bytes each.
template <typename T, int LPR>
__global__ void __launch_bounds__(NT)
vnorm_vec(MonTables t, int l0, int Hq, int Hkv, int64_t n, const float* lse_kept,
          const float* lse_full, float* delta, float* vmax_out, float* bound) {
  __shared__ float red[NW];
  const int u = blockIdx.x;                    // (layer within the launch, KV head)
  const int li = u / Hkv, g = u % Hkv;
  constexpr int RPI = NT / LPR;                // rows per iteration of the workgroup
  const int64_t rowbytes = (int64_t)LPR * 16;
  const char* V = (const char*)t.V.p[li] + (int64_t)g * n * rowbytes;
  const int r = threadIdx.x / LPR, c = threadIdx.x % LPR;
  float best = 0.f;
  for (int64_t j0 = r; j0 < n; j0 += (int64_t)RU * RPI) {
    uint4 x[RU];
#pragma unroll
    for (int i = 0; i < RU; ++i)               // rows past the end read the last row again
      x[i] = ld_stream(V + min(j0 + (int64_t)i * RPI, n - 1) * rowbytes + c * 16);
#pragma unroll
    for (int i = 0; i < RU; ++i) {
      float s = 0.f;
      const uint32_t w[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (sizeof(T) == 2) {
          const float a = bf16_lo(w[e]), b = bf16_hi(w[e]);
          s = fmaf(a, a, s);
          s = fmaf(b, b, s);
        } else {
          const float a = __uint_as_float(w[e]);
          s = fmaf(a, a, s);
        }
      }
      s = group_sum<LPR>(s);
      best = fmaxf(best, s);
    }
  }
  const float m = block_max<NT>(best, red);
  write_group(m, l0 + li, g, Hq, Hq / Hkv, lse_kept, lse_full, delta, vmax_out, bound);
}

// Any row size: one wave per row, lanes stride over its elements.
template <typename T>
__global__ void __launch_bounds__(NT)
vnorm_any(MonTables t, int l0, int Hq, int Hkv, int64_t n, int d, const float* lse_kept,
          const float* lse_full, float* delta, float* vmax_out, float* bound) {
  __shared__ float red[NW];
  const int u = blockIdx.x;
  const int li = u / Hkv, g = u % Hkv;
  const T* V = (const T*)t.V.p[li] + (int64_t)g * n * d;
  const int wv = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  float best = 0.f;
  for (int64_t j = wv; j < n; j += NW) {
    float s = 0.f;
    for (int e = lane; e < d; e += kWave) {
      float a;
      if constexpr (sizeof(T) == 2) a = bf16_to_f32(V[j * d + e]);
      else a = V[j * d + e];
      s = fmaf(a, a, s);
    }
    best = fmaxf(best, wave_sum(s));
  }
  const float m = block_max<NT>(best, red);
  write_group(m, l0 + li, g, Hq, Hq / Hkv, lse_kept, lse_full, delta, vmax_out, bound);
}

template <typename T>
void launch_vec(int lpr, dim3 grid, hipStream_t s, MonTables t, int l0, int Hq, int Hkv,
                int64_t n, const float* lk, const float* lf, float* dl, float* vm, float* bd) {
#define KVC_V(LL) hipLaunchKernelGGL((vnorm_vec<T, LL>), grid, dim3(NT), 0, s, t, l0, Hq, Hkv, n, lk, lf, dl, vm, bd)
  switch (lpr) {
    case 1: KVC_V(1); break;
    case 2: KVC_V(2); break;
    case 4: KVC_V(4); break;
    case 8: KVC_V(8); break;
    case 16: KVC_V(16); break;
    case 32: KVC_V(32); break;
    default: KVC_V(64); break;
  }
#undef KVC_V
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" int kvc_dropped_mass(const float* lse_kept, const float* lse_full,
                                const void* const* V, int dtype, int L, int Hq, int Hkv,
                                int64_t n, int d, float* delta_out, float* vmax_out,
                                float* bound_out, void* stream) {
  clear_error();
  const char* fn = "kvc_dropped_mass";
  if (!dtype_ok(dtype)) return KVC_FAIL(KVC_ERR_DTYPE, "%s: dtype %d", fn, dtype);
  KVC_REQUIRE(L >= 1 && L <= KVC_MAX_LAYERS, "%s: need 1 <= L <= %d", fn, KVC_MAX_LAYERS);
  KVC_REQUIRE(Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0, "%s: need Hq %% Hkv == 0", fn);
  KVC_REQUIRE(Hq / Hkv <= NT, "%s: more than %d query heads per KV head", fn, NT);
  KVC_REQUIRE(n >= 1 && d >= 1 && d <= 4096, "%s: need n >= 1 and 1 <= d <= 4096", fn);
  KVC_REQUIRE((int64_t)kLayersPerLaunch * Hkv <= 0x7fffffffLL, "%s: Hkv too large", fn);
  KVC_REQUIRE(lse_kept && lse_full && V && delta_out && vmax_out && bound_out,
              "%s: null pointer", fn);
  const int rowbytes = d * dtype_size(dtype);
  const int lpr = rowbytes / 16;
  bool vec = rowbytes % 16 == 0 && lpr <= kWave && (lpr & (lpr - 1)) == 0;
  for (int l = 0; l < L; ++l) {
    KVC_REQUIRE(V[l], "%s: null pointer in layer %d", fn, l);
    vec = vec && (uintptr_t)V[l] % 16 == 0;
  }
  hipStream_t s = as_stream(stream);
  for (int l0 = 0; l0 < L; l0 += kLayersPerLaunch) {
    const int lc = min(kLayersPerLaunch, L - l0);
    MonTables t{};
    for (int i = 0; i < lc; ++i) t.V.p[i] = V[l0 + i];
    const dim3 grid((unsigned)(lc * Hkv));
    if (vec) {
      if (dtype == KVC_BF16)
        launch_vec<uint16_t>(lpr, grid, s, t, l0, Hq, Hkv, n, lse_kept, lse_full, delta_out, vmax_out, bound_out);
      else
        launch_vec<float>(lpr, grid, s, t, l0, Hq, Hkv, n, lse_kept, lse_full, delta_out, vmax_out, bound_out);
    } else if (dtype == KVC_BF16) {
      hipLaunchKernelGGL(vnorm_any<uint16_t>, grid, dim3(NT), 0, s, t, l0, Hq, Hkv, n, d, lse_kept,
                         lse_full, delta_out, vmax_out, bound_out);
    } else {
      hipLaunchKernelGGL(vnorm_any<float>, grid, dim3(NT), 0, s, t, l0, Hq, Hkv, n, d, lse_kept,
                         lse_full, delta_out, vmax_out, bound_out);
    }
  }
  return launch_status(fn);
}
