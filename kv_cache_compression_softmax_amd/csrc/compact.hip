// Order-preserving gather of the kept K/V rows into the compacted cache.
//
// [InfoKV] Method: each layer retains its selected tokens; the compacted cache
// holds them in their original order, so positions stay monotone.
//
// Pure bandwidth: each kept row (d elements, 256 B for bf16 d = 128) is read once
// and written once.  A workgroup copies ROWS consecutive kept rows of one
// (layer, KV head): 16-byte lanes, rowbytes/16 lanes per row, so one wave moves
// several whole rows per instruction and both the reads and the writes of a row
// are single contiguous segments.  Layers of different k_l (adaptive budget)
// share one launch through a per-layer table of block offsets.
#include "common.h"

namespace kvc {
namespace {

constexpr int NT = 256;
constexpr int ROWS = 64;        // kept rows per workgroup
constexpr int RU = 4;           // rows per thread with loads in flight together (16-byte path)

struct Tables {
  ConstPtrs K, V, idx;
  MutPtrs Ko, Vo;
  I64s k;
  I64s orows;                   // output rows per KV head (the head stride of K_out, V_out)
  I64s blk0;                    // first block of each layer
};

// A kept index outside [0, n) is clamped to n - 1: a bad list gives wrong rows,
// never a read outside the head's rows.
__device__ __forceinline__ int64_t row_in(int32_t i, int64_t n) {
  return min((int64_t)(uint32_t)i, n - 1);
}

// MODE: 0 any row size (2-byte words), 1 rows of 16-byte multiples, 2 four-byte rows
template <int MODE>
__global__ void __launch_bounds__(NT)
compact_kernel(Tables t, int lc, int Hkv, int64_t n, int rowbytes) {
  const int64_t b = blockIdx.x;
  int l = 0;
  while (l + 1 < lc && t.blk0.v[l + 1] <= b) ++l;
  const int64_t k = t.k.v[l];
  const int64_t nbk = (k + ROWS - 1) / ROWS;
  const int64_t local = b - t.blk0.v[l];
  const int g = (int)(local / nbk);
  const int64_t j0 = (local % nbk) * ROWS;
  const int32_t* idx = (const int32_t*)t.idx.p[l] + (int64_t)g * k;
  const char* K = (const char*)t.K.p[l] + (int64_t)g * n * rowbytes;
  const char* V = t.V.p[l] ? (const char*)t.V.p[l] + (int64_t)g * n * rowbytes : nullptr;
  char* Ko = (char*)t.Ko.p[l] + (int64_t)g * t.orows.v[l] * rowbytes;
  char* Vo = V ? (char*)t.Vo.p[l] + (int64_t)g * t.orows.v[l] * rowbytes : nullptr;
  if (MODE == 1) {
    const int lpr = rowbytes / 16;                 // lanes per row
    const int rpi = NT / lpr;                      // rows per iteration
    const int r = threadIdx.x / lpr, c = threadIdx.x % lpr;
    if (r >= rpi) return;
    // RU rows per thread at a time: their indices, then all their K and V loads,
    // then the stores, so a thread has RU rows' loads in flight (with streaming
    // loads and stores, 341 -> 303 us for the 8B shape at 32K tokens, 20% kept).
    // Rows past the workgroup's last are clamped to it (loaded, not stored).
    const int64_t jend = min(k, j0 + ROWS);
    for (int64_t jg = j0 + r; jg < jend; jg += RU * rpi) {
      int64_t src[RU];
#pragma unroll
      for (int u = 0; u < RU; ++u) src[u] = row_in(idx[min(jg + u * rpi, jend - 1)], n);
      uint4 kv[RU], vv[RU];
#pragma unroll
      for (int u = 0; u < RU; ++u) kv[u] = ld_stream(K + src[u] * rowbytes + c * 16);
      if (V) {
#pragma unroll
        for (int u = 0; u < RU; ++u) vv[u] = ld_stream(V + src[u] * rowbytes + c * 16);
      }
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        const int64_t j = jg + u * rpi;
        if (j < jend) {
          st_stream(Ko + j * rowbytes + c * 16, kv[u]);
          if (V) st_stream(Vo + j * rowbytes + c * 16, vv[u]);
        }
      }
    }
  } else if (MODE == 2) {
    // one 4-byte row per thread (per-slot float32 scores)
    const int64_t j = j0 + threadIdx.x;
    if (threadIdx.x < ROWS && j < k) {
      const int64_t src = row_in(idx[j], n);
      *reinterpret_cast<uint32_t*>(Ko + j * 4) = *reinterpret_cast<const uint32_t*>(K + src * 4);
      if (V) *reinterpret_cast<uint32_t*>(Vo + j * 4) = *reinterpret_cast<const uint32_t*>(V + src * 4);
    }
  } else {
    const int half = rowbytes / 2;                 // 2-byte words per row
    for (int64_t j = j0; j < min(k, j0 + ROWS); ++j) {
      const int64_t src = row_in(idx[j], n);
      for (int c = threadIdx.x; c < half; c += NT) {
        ((uint16_t*)(Ko + j * rowbytes))[c] = ((const uint16_t*)(K + src * rowbytes))[c];
        if (V) ((uint16_t*)(Vo + j * rowbytes))[c] = ((const uint16_t*)(V + src * rowbytes))[c];
      }
    }
  }
}

}  // namespace
}  // namespace kvc

using namespace kvc;

namespace {

int compact_impl(const char* fn, const void* const* K, const void* const* V, int dtype, int L,
                 int Hkv, int64_t n, int d, const int32_t* const* idx, const int64_t* k_keep,
                 int64_t out_rows, void* const* K_out, void* const* V_out, void* stream) {
  clear_error();
  if (!dtype_ok(dtype)) return KVC_FAIL(KVC_ERR_DTYPE, "%s: dtype %d", fn, dtype);
  KVC_REQUIRE(L >= 1 && L <= KVC_MAX_LAYERS, "%s: need 1 <= L <= %d", fn, KVC_MAX_LAYERS);
  KVC_REQUIRE(Hkv >= 1 && n >= 1 && d >= 1 && d <= 4096, "%s: need Hkv, n >= 1 and 1 <= d <= 4096", fn);
  KVC_REQUIRE(K && idx && k_keep && K_out, "%s: null pointer", fn);
  KVC_REQUIRE((V == nullptr) == (V_out == nullptr), "%s: V and V_out must both be set or both NULL", fn);
  KVC_REQUIRE((int64_t)kLayersPerLaunch * Hkv * ((n + ROWS - 1) / ROWS) <= 0x7fffffffLL,
              "%s: too many rows for one launch", fn);
  const int rowbytes = d * dtype_size(dtype);
  bool vec = rowbytes % 16 == 0 && rowbytes / 16 <= NT;
  bool word = rowbytes == 4;
  for (int l = 0; l < L; ++l) {
    KVC_REQUIRE(K[l] && idx[l] && K_out[l], "%s: null pointer in layer %d", fn, l);
    KVC_REQUIRE(!V || (V[l] && V_out[l]), "%s: null V pointer in layer %d", fn, l);
    KVC_REQUIRE(k_keep[l] >= 1 && k_keep[l] <= n, "%s: k_keep[%d] outside [1, n]", fn, l);
    KVC_REQUIRE(out_rows <= 0 || k_keep[l] <= out_rows, "%s: k_keep[%d] > out_rows", fn, l);
    vec = vec && (uintptr_t)K[l] % 16 == 0 && (uintptr_t)K_out[l] % 16 == 0;
    if (V) vec = vec && (uintptr_t)V[l] % 16 == 0 && (uintptr_t)V_out[l] % 16 == 0;
    word = word && (uintptr_t)K[l] % 4 == 0 && (uintptr_t)K_out[l] % 4 == 0;
    if (V) word = word && (uintptr_t)V[l] % 4 == 0 && (uintptr_t)V_out[l] % 4 == 0;
  }
  hipStream_t s = as_stream(stream);
  for (int l0 = 0; l0 < L; l0 += kLayersPerLaunch) {
    const int lc = min(kLayersPerLaunch, L - l0);
    Tables t{};
    int64_t blocks = 0;
    for (int i = 0; i < lc; ++i) {
      t.K.p[i] = K[l0 + i];
      t.V.p[i] = V ? V[l0 + i] : nullptr;
      t.idx.p[i] = idx[l0 + i];
      t.Ko.p[i] = K_out[l0 + i];
      t.Vo.p[i] = V ? V_out[l0 + i] : nullptr;
      t.k.v[i] = k_keep[l0 + i];
      t.orows.v[i] = out_rows > 0 ? out_rows : k_keep[l0 + i];
      t.blk0.v[i] = blocks;
      blocks += (int64_t)Hkv * ((k_keep[l0 + i] + ROWS - 1) / ROWS);
    }
    if (vec) hipLaunchKernelGGL(compact_kernel<1>, dim3((unsigned)blocks), dim3(NT), 0, s, t, lc, Hkv, n, rowbytes);
    else if (word) hipLaunchKernelGGL(compact_kernel<2>, dim3((unsigned)blocks), dim3(ROWS), 0, s, t, lc, Hkv, n, rowbytes);
    else hipLaunchKernelGGL(compact_kernel<0>, dim3((unsigned)blocks), dim3(NT), 0, s, t, lc, Hkv, n, rowbytes);
  }
  return launch_status(fn);
}

}  // namespace

extern "C" int kvc_compact(const void* const* K, const void* const* V, int dtype, int L, int Hkv,
                           int64_t n, int d, const int32_t* const* idx, const int64_t* k_keep,
                           void* const* K_out, void* const* V_out, void* stream) {
  return compact_impl("kvc_compact", K, V, dtype, L, Hkv, n, d, idx, k_keep, 0, K_out, V_out, stream);
}

extern "C" int kvc_compact_into(const void* const* K, const void* const* V, int dtype, int L,
                                int Hkv, int64_t n, int d, const int32_t* const* idx,
                                const int64_t* k_keep, int64_t out_rows, void* const* K_out,
                                void* const* V_out, void* stream) {
  if (out_rows < 1) {
    clear_error();
    return KVC_FAIL(KVC_ERR_ARG, "kvc_compact_into: out_rows < 1");
  }
  return compact_impl("kvc_compact_into", K, V, dtype, L, Hkv, n, d, idx, k_keep, out_rows, K_out,
                      V_out, stream);
}
