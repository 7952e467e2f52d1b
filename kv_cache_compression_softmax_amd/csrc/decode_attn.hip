// Decode attention of one query per head over a KV cache, with the optional
// compensation bias alpha * ln R on the logits.
//
// [SelKV] section 2, attention compensation: at decode time a merged entry's
// logit is raised by alpha * ln R so that it receives the attention mass of the
// tokens it stands for.  The same kernel over the full and the compacted cache
// gives the outputs compared by [RECAS] section 2.B's dropped-mass bound.
//
// Split over the cache length: a workgroup handles one (layer, KV head, chunk of
// CK keys) for all G query heads of the group, so each key/value row is read
// once per group.  LG lanes hold one row (16 bytes each); per key the G dot
// products are reduced inside the lane group, then an online softmax keeps
// (max, sum, output) per head.  Lane groups, then waves, are merged in a fixed
// order; a second kernel merges the chunks.
#include "common.h"

namespace kvc {
namespace {

constexpr int NT = 256;
constexpr int CK = 1024;          // keys per workgroup
constexpr int MAXG = 8;           // query heads per KV head

template <typename T> struct DE;
template <> struct DE<uint16_t> {
  static constexpr int N = 8;
  __device__ static void unpack(const uint4& u, float (&x)[8]) {
    x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
    x[4] = bf16_lo(u.z); x[5] = bf16_hi(u.z); x[6] = bf16_lo(u.w); x[7] = bf16_hi(u.w);
  }
};
template <> struct DE<float> {
  static constexpr int N = 4;
  __device__ static void unpack(const uint4& u, float (&x)[4]) {
    x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
    x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
  }
};

struct DecTables { ConstPtrs q, K, V, logR; };

// partial layout: [lc, Hq, nchunk] x (m, l, o[d])
template <typename T, int LG, int G>
__global__ void __launch_bounds__(NT)
decode_partial(DecTables t, int Hq, int Hkv, int64_t len, int d, float scale, float alpha_bias,
               int nchunk, float* __restrict__ part) {
  constexpr int W = DE<T>::N;
  constexpr int NG = NT / LG;                    // lane groups per block
  __shared__ float sm_m[NT / 64][G], sm_l[NT / 64][G];
  __shared__ float sm_o[NT / 64][G][256];
  const int lane = threadIdx.x & 63, wv = threadIdx.x / 64;
  const int grp = threadIdx.x / LG, c = threadIdx.x % LG;
  const int64_t bid = blockIdx.x;
  const int ch = (int)(bid % nchunk);
  const int g = (int)((bid / nchunk) % Hkv);
  const int l = (int)(bid / ((int64_t)nchunk * Hkv));
  const T* q = (const T*)t.q.p[l];
  const T* K = (const T*)t.K.p[l] + (int64_t)g * len * d;
  const T* V = (const T*)t.V.p[l] + (int64_t)g * len * d;
  const float* lr = t.logR.p[l] ? (const float*)t.logR.p[l] + (int64_t)g * len : nullptr;

  float qv[G][W];
#pragma unroll
  for (int h = 0; h < G; ++h)
    DE<T>::unpack(*reinterpret_cast<const uint4*>(q + (int64_t)(g * G + h) * d + c * W), qv[h]);
  float m[G], s[G], o[G][W];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY; s[h] = 0.f;
#pragma unroll
    for (int e = 0; e < W; ++e) o[h][e] = 0.f;
  }
  const int64_t j0 = (int64_t)ch * CK, j1 = min(len, j0 + CK);
  for (int64_t j = j0 + grp; j < j1; j += NG) {
    float kx[W], vx[W];
    DE<T>::unpack(*reinterpret_cast<const uint4*>(K + j * d + c * W), kx);
    DE<T>::unpack(*reinterpret_cast<const uint4*>(V + j * d + c * W), vx);
    const float bias = lr ? alpha_bias * lr[j] : 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < W; ++e) dot += qv[h][e] * kx[e];
      dot = group_sum<LG>(dot);
      const float x = dot * scale + bias;
      const float mn = fmaxf(m[h], x);
      const float a = expf(m[h] - mn), p = expf(x - mn);
      s[h] = s[h] * a + p;
#pragma unroll
      for (int e = 0; e < W; ++e) o[h][e] = o[h][e] * a + p * vx[e];
      m[h] = mn;
    }
  }
  // merge the lane groups of a wave (xor over the group bits), fixed order
#pragma unroll
  for (int off = LG; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off, 64), so = __shfl_xor(s[h], off, 64);
      const float mn = fmaxf(m[h], mo);
      const float a = mn > -INFINITY ? expf(m[h] - mn) : 0.f;
      const float b = mn > -INFINITY ? expf(mo - mn) : 0.f;
      s[h] = s[h] * a + so * b;
#pragma unroll
      for (int e = 0; e < W; ++e) {
        const float oo = __shfl_xor(o[h][e], off, 64);
        o[h][e] = o[h][e] * a + oo * b;
      }
      m[h] = mn;
    }
  }
  if (lane < LG) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (lane == 0) { sm_m[wv][h] = m[h]; sm_l[wv][h] = s[h]; }
#pragma unroll
      for (int e = 0; e < W; ++e) sm_o[wv][h][c * W + e] = o[h][e];
    }
  }
  __syncthreads();
  // merge the waves; thread (h, e) writes one output element
  for (int x = threadIdx.x; x < G * d; x += NT) {
    const int h = x / d, e = x % d;
    float M = -INFINITY;
    for (int w2 = 0; w2 < NT / 64; ++w2) M = fmaxf(M, sm_m[w2][h]);
    float S = 0.f, O = 0.f;
    for (int w2 = 0; w2 < NT / 64; ++w2) {
      const float a = M > -INFINITY ? expf(sm_m[w2][h] - M) : 0.f;
      S += sm_l[w2][h] * a;
      O += sm_o[w2][h][e] * a;
    }
    float* p = part + (((int64_t)l * Hq + g * G + h) * nchunk + ch) * (d + 2);
    if (e == 0) { p[0] = M; p[1] = S; }
    p[2 + e] = O;
  }
}

__global__ void decode_combine(const float* __restrict__ part, int nchunk, int d, int64_t nhead,
                               float* __restrict__ o, float* __restrict__ lse) {
  const int64_t hh = blockIdx.x;                 // (layer, query head)
  if (hh >= nhead) return;
  const float* p = part + hh * nchunk * (d + 2);
  float M = -INFINITY;
  for (int c = 0; c < nchunk; ++c) M = fmaxf(M, p[(int64_t)c * (d + 2)]);
  float S = 0.f;
  for (int c = 0; c < nchunk; ++c) {
    const float* pc = p + (int64_t)c * (d + 2);
    S += pc[1] * (M > -INFINITY ? expf(pc[0] - M) : 0.f);
  }
  for (int e = threadIdx.x; e < d; e += blockDim.x) {
    float O = 0.f;
    for (int c = 0; c < nchunk; ++c) {
      const float* pc = p + (int64_t)c * (d + 2);
      O += pc[2 + e] * (M > -INFINITY ? expf(pc[0] - M) : 0.f);
    }
    o[hh * d + e] = O / S;
  }
  if (lse && threadIdx.x == 0) lse[hh] = M + logf(S);
}

template <typename T, int LG>
void launch_g(int G, dim3 grid, hipStream_t s, const DecTables& t, int Hq, int Hkv, int64_t len,
              int d, float scale, float ab, int nchunk, float* part) {
#define KVC_D(GG) hipLaunchKernelGGL((decode_partial<T, LG, GG>), grid, dim3(NT), 0, s, t, Hq, Hkv, len, d, scale, ab, nchunk, part)
  switch (G) {
    case 1: KVC_D(1); break;
    case 2: KVC_D(2); break;
    case 3: KVC_D(3); break;
    case 4: KVC_D(4); break;
    case 5: KVC_D(5); break;
    case 6: KVC_D(6); break;
    case 7: KVC_D(7); break;
    default: KVC_D(8); break;
  }
#undef KVC_D
}

template <typename T>
void launch_dec(int LG, int G, dim3 grid, hipStream_t s, const DecTables& t, int Hq, int Hkv,
                int64_t len, int d, float scale, float ab, int nchunk, float* part) {
  switch (LG) {
    case 4: launch_g<T, 4>(G, grid, s, t, Hq, Hkv, len, d, scale, ab, nchunk, part); break;
    case 8: launch_g<T, 8>(G, grid, s, t, Hq, Hkv, len, d, scale, ab, nchunk, part); break;
    case 16: launch_g<T, 16>(G, grid, s, t, Hq, Hkv, len, d, scale, ab, nchunk, part); break;
    default: launch_g<T, 32>(G, grid, s, t, Hq, Hkv, len, d, scale, ab, nchunk, part); break;
  }
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" size_t kvc_decode_attn_workspace_size(int L, int Hq, int64_t len, int d) {
  if (L < 1 || Hq < 1 || len < 1 || d < 1) return 0;
  const int lc = L < kLayersPerLaunch ? L : kLayersPerLaunch;
  const int64_t nchunk = (len + CK - 1) / CK;
  return (size_t)lc * Hq * nchunk * (d + 2) * sizeof(float) + 256;
}

extern "C" int kvc_decode_attn(const void* const* q, const void* const* K, const void* const* V,
                               int dtype, const float* const* logR, float alpha_bias, int L, int Hq,
                               int Hkv, int64_t len, int d, float scale, float* o_out, float* lse_out,
                               void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  if (!dtype_ok(dtype)) return KVC_FAIL(KVC_ERR_DTYPE, "kvc_decode_attn: dtype %d", dtype);
  KVC_REQUIRE(L >= 1 && L <= KVC_MAX_LAYERS, "kvc_decode_attn: need 1 <= L <= %d", KVC_MAX_LAYERS);
  KVC_REQUIRE(Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0, "kvc_decode_attn: need Hq %% Hkv == 0");
  KVC_REQUIRE(Hq / Hkv <= MAXG, "kvc_decode_attn: more than %d query heads per KV head", MAXG);
  KVC_REQUIRE(len >= 1 && len <= 0x7fffffffLL, "kvc_decode_attn: need 1 <= len < 2^31");
  KVC_REQUIRE(q && K && V && o_out, "kvc_decode_attn: null pointer");
  const int rb = d * dtype_size(dtype);
  KVC_REQUIRE(d <= 256 && rb % 16 == 0 && (rb / 16 == 4 || rb / 16 == 8 || rb / 16 == 16 || rb / 16 == 32),
              "kvc_decode_attn: need d * elsize in {64, 128, 256, 512} bytes and d <= 256");
  const int LG = rb / 16;
  for (int l = 0; l < L; ++l) {
    KVC_REQUIRE(q[l] && K[l] && V[l], "kvc_decode_attn: null pointer in layer %d", l);
    KVC_REQUIRE((uintptr_t)q[l] % 16 == 0 && (uintptr_t)K[l] % 16 == 0 && (uintptr_t)V[l] % 16 == 0,
                "kvc_decode_attn: layer %d tensors not 16-byte aligned", l);
    KVC_REQUIRE(!logR || logR[l], "kvc_decode_attn: logR[%d] is null", l);
  }
  const size_t need = kvc_decode_attn_workspace_size(L, Hq, len, d);
  if (!ws || ws_bytes < need)
    return KVC_FAIL(KVC_ERR_WORKSPACE, "kvc_decode_attn: workspace needs %zu bytes", need);
  float* part = (float*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
  const int nchunk = (int)((len + CK - 1) / CK);
  hipStream_t s = as_stream(stream);
  const int G = Hq / Hkv;
  for (int l0 = 0; l0 < L; l0 += kLayersPerLaunch) {
    const int lc = min(kLayersPerLaunch, L - l0);
    DecTables t{};
    for (int i = 0; i < lc; ++i) {
      t.q.p[i] = q[l0 + i]; t.K.p[i] = K[l0 + i]; t.V.p[i] = V[l0 + i];
      t.logR.p[i] = logR ? logR[l0 + i] : nullptr;
    }
    const dim3 grid((unsigned)((int64_t)lc * Hkv * nchunk));
    if (dtype == KVC_BF16) launch_dec<uint16_t>(LG, G, grid, s, t, Hq, Hkv, len, d, scale, alpha_bias, nchunk, part);
    else launch_dec<float>(LG, G, grid, s, t, Hq, Hkv, len, d, scale, alpha_bias, nchunk, part);
    const int64_t nhead = (int64_t)lc * Hq;
    hipLaunchKernelGGL(decode_combine, dim3((unsigned)nhead), dim3(128), 0, s, (const float*)part, nchunk,
                       d, nhead, o_out + (int64_t)l0 * Hq * d, lse_out ? lse_out + (int64_t)l0 * Hq : nullptr);
  }
  return launch_status("kvc_decode_attn");
}
