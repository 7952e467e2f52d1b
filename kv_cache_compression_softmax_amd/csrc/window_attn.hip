// Observation-window attention A (group mean, or per query head).
//
// [InfoKV] Method and Technical detail: the attention each cached token receives
// from the queries of the last w positions of layer l, averaged over the window
// (and, for GQA, over the query heads sharing the KV head).  [SelKV] section 2,
// pipeline step 1 uses the per-head form for its VATP score.
//
// Layout: q_win[l] is [Hq, w, d], k[l] is [Hkv, n, d].  For KV head g the window
// queries of its G heads form the rows of an M x d matrix; each head's w rows are
// padded to a multiple of 32 so that every 32-row "tile" belongs to one head.
//
// A needs each row's softmax normaliser before any column can be summed, so the
// bf16 path runs two passes over K (the second usually hits the 256 MB MALL when
// the layer chunk is small):
//   pass 1  per 32-key block, S^T = K * Q^T on MFMA (keys on M, queries on N);
//           each lane keeps an online (max, sum) of exp2 for one query row;
//           one partial per (wave task, row) goes to the workspace;
//   combine fixed-order merge of the partials into c_r = log2 of the row's
//           normaliser (max + log2 sum);
//   pass 2  S = Q * K^T on MFMA (queries on M, keys on N): each lane owns one key
//           column, so exp2(s - c_r) summed over the lane's 16 rows plus its
//           partner lane gives the column sum with no atomics.
// Both passes read every key row as 16-byte vectors straight into MFMA operand
// registers: lane (row i, half hf) holds d/2 contiguous elements, and the
// contraction index k of step s maps to element hf*d/2 + 8s + e, the same map
// for Q and K (the contraction does not depend on the order of k).
#include "common.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int NTW = 256;        // threads per workgroup (4 waves, one task each)
constexpr int MAX_TILES = 8;    // G * ceil(w/32)
constexpr int MAX_TG = 4;       // tiles held in registers per launch
constexpr int KPW = 512;        // keys per wave task (multiple of 32)
constexpr float LOG2E = 1.4426950408889634f;

struct Geo {
  int Hq, Hkv, G, w, d, tph, ntiles;   // tiles per head, tiles per group
  int64_t n;
  int nb;                              // wave tasks per (layer, KV head)
};

__device__ __forceinline__ int tile_row_pos(const Geo& g, int tile, int i) {
  // window position of row i of a tile, or -1 for a padding row
  const int rr = (tile % g.tph) * 32 + i;
  return rr < g.w ? (int)(g.n - g.w) + rr : -1;
}

template <int D>
__device__ __forceinline__ void load_q(const uint16_t* q, const Geo& g, int kvh, int tile, int lane,
                                       bf16x8 (&qf)[D / 16]) {
  const int i = lane & 31, hf = lane >> 5;
  const int head = kvh * g.G + tile / g.tph;
  const int rr = (tile % g.tph) * 32 + i;
  if (rr < g.w) {
    const uint16_t* p = q + ((int64_t)head * g.w + rr) * D + hf * (D / 2);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(p + 8 * s);
  } else {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = bf16x8{};
  }
}

template <int D>
__device__ __forceinline__ void load_k(const uint16_t* k, const Geo& g, int kvh, int64_t j0, int lane,
                                       bf16x8 (&kf)[D / 16]) {
  const int i = lane & 31, hf = lane >> 5;
  const int64_t key = j0 + i;
  if (key < g.n) {
    const uint16_t* p = k + ((int64_t)kvh * g.n + key) * D + hf * (D / 2);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) kf[s] = *reinterpret_cast<const bf16x8*>(p + 8 * s);
  } else {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) kf[s] = bf16x8{};
  }
}

// row (M index) of accumulator element v held by a lane of half hf
__device__ __forceinline__ int acc_row(int v, int hf) { return 8 * (v >> 2) + 4 * hf + (v & 3); }

// ---------------------------------------------------------------- pass 1
template <int D, int TG>
__global__ void __launch_bounds__(NTW)
win_pass1(ConstPtrs qs, ConstPtrs ks, Geo g, int tile0, int lc, float scale_log2,
          float2* __restrict__ part) {
  const int lane = threadIdx.x & 63, hf = lane >> 5, qi = lane & 31;
  const int64_t task = (int64_t)blockIdx.x * (NTW / 64) + threadIdx.x / 64;
  const int64_t ntask = (int64_t)lc * g.Hkv * g.nb;
  if (task >= ntask) return;
  const int b = (int)(task % g.nb);
  const int kvh = (int)((task / g.nb) % g.Hkv);
  const int l = (int)(task / ((int64_t)g.nb * g.Hkv));
  const uint16_t* q = (const uint16_t*)qs.p[l];
  const uint16_t* k = (const uint16_t*)ks.p[l];

  bf16x8 qf[TG][D / 16];
  int pos[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    load_q<D>(q, g, kvh, tile0 + t, lane, qf[t]);
    pos[t] = tile_row_pos(g, tile0 + t, qi);
  }
  float m[TG], s[TG];
#pragma unroll
  for (int t = 0; t < TG; ++t) { m[t] = -INFINITY; s[t] = 0.f; }

  const int64_t jb = (int64_t)b * KPW;
  const int64_t je = min(g.n, jb + KPW);
  bf16x8 kf[D / 16], kn[D / 16];
  load_k<D>(k, g, kvh, jb, lane, kf);
#pragma unroll 1
  for (int64_t j0 = jb; j0 < je; j0 += 32) {
    if (j0 + 32 < je) load_k<D>(k, g, kvh, j0 + 32, lane, kn);
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      f32x16 acc = {};
#pragma unroll
      for (int st = 0; st < D / 16; ++st)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[t][st], acc, 0, 0, 0);
      float x[16];
      float bm = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t key = j0 + acc_row(v, hf);
        x[v] = (key <= pos[t] && key < g.n) ? acc[v] * scale_log2 : -INFINITY;
        bm = fmaxf(bm, x[v]);
      }
      if (bm > -INFINITY) {
        const float mn = fmaxf(m[t], bm);
        float sum = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) sum += exp2f(x[v] - mn);
        s[t] = s[t] * exp2f(m[t] - mn) + sum;
        m[t] = mn;
      }
    }
#pragma unroll
    for (int st = 0; st < D / 16; ++st) kf[st] = kn[st];
  }
  // merge the two halves (lanes i and i+32 hold the same query row)
#pragma unroll
  for (int t = 0; t < TG; ++t) {
    const float mo = __shfl_xor(m[t], 32, 64), so = __shfl_xor(s[t], 32, 64);
    const float M = fmaxf(m[t], mo);
    float S = 0.f;
    if (M > -INFINITY) S = s[t] * exp2f(m[t] - M) + so * exp2f(mo - M);
    if (hf == 0) {
      const int64_t row = (int64_t)(tile0 + t) * 32 + qi;
      part[(((int64_t)l * g.Hkv + kvh) * g.nb + b) * (g.ntiles * 32) + row] = make_float2(M, S);
    }
  }
}

// ---------------------------------------------------------------- combine
// c[l, g, row] = log2 of the row's softmax normaliser in exp2 units (+inf for a
// row with no visible key, i.e. a padding row).  Fixed order over the tasks.
__global__ void __launch_bounds__(256)
win_combine(const float2* __restrict__ part, int nb, int rows, int64_t ngroups, float* __restrict__ c) {
  const int64_t gi = blockIdx.x;              // (layer, KV head)
  if (gi >= ngroups) return;
  for (int r = threadIdx.x; r < rows; r += blockDim.x) {
    const float2* p = part + gi * nb * rows + r;
    float M = -INFINITY;
    for (int b = 0; b < nb; ++b) M = fmaxf(M, p[(int64_t)b * rows].x);
    float out = INFINITY;
    if (M > -INFINITY) {
      float S = 0.f;
      for (int b = 0; b < nb; ++b) {
        const float2 v = p[(int64_t)b * rows];
        if (v.x > -INFINITY) S += v.y * exp2f(v.x - M);
      }
      out = M + log2f(S);
    }
    c[gi * rows + r] = out;
  }
}

// ---------------------------------------------------------------- pass 2
template <int D, int TG>
__global__ void __launch_bounds__(NTW)
win_pass2(ConstPtrs qs, ConstPtrs ks, Geo g, int tile0, int lc, float scale_log2,
          const float* __restrict__ cfin, int per_head, float* __restrict__ A) {
  __shared__ float csh[NTW / 64][MAX_TG * 32];
  const int lane = threadIdx.x & 63, hf = lane >> 5, qi = lane & 31, wv = threadIdx.x / 64;
  const int64_t ntask = (int64_t)lc * g.Hkv * g.nb;
  const int64_t task0 = (int64_t)blockIdx.x * (NTW / 64) + wv;
  const bool active = task0 < ntask;
  const int64_t task = active ? task0 : 0;
  const int b = (int)(task % g.nb);
  const int kvh = (int)((task / g.nb) % g.Hkv);
  const int l = (int)(task / ((int64_t)g.nb * g.Hkv));
  const uint16_t* q = (const uint16_t*)qs.p[l];
  const uint16_t* k = (const uint16_t*)ks.p[l];
  const int rows = g.ntiles * 32;

  // each wave stages the row normalisers of its (layer, KV head) tiles in LDS
  const float* cg = cfin + ((int64_t)l * g.Hkv + kvh) * rows + tile0 * 32;
  for (int r = lane; r < TG * 32; r += 64) csh[wv][r] = cg[r];
  __syncthreads();                 // the only barrier; idle waves leave after it
  if (!active) return;
  bf16x8 qf[TG][D / 16];
#pragma unroll
  for (int t = 0; t < TG; ++t) load_q<D>(q, g, kvh, tile0 + t, lane, qf[t]);

  // head of each tile, and the window position of each of this lane's rows
  const int64_t jb = (int64_t)b * KPW;
  const int64_t je = min(g.n, jb + KPW);
  const float inv_group = 1.0f / (float)(g.G * g.w), inv_w = 1.0f / (float)g.w;
  bf16x8 kf[D / 16], kn[D / 16];
  load_k<D>(k, g, kvh, jb, lane, kf);
#pragma unroll 1
  for (int64_t j0 = jb; j0 < je; j0 += 32) {
    if (j0 + 32 < je) load_k<D>(k, g, kvh, j0 + 32, lane, kn);
    const int64_t key = j0 + qi;               // this lane's key column
    float total = 0.f;                         // group mode: over all tiles
    float hsum = 0.f;                          // head mode: current head
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      f32x16 acc = {};
#pragma unroll
      for (int st = 0; st < D / 16; ++st)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[t][st], kf[st], acc, 0, 0, 0);
      float colsum = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = acc_row(v, hf);
        const int p = tile_row_pos(g, tile0 + t, r);
        const float e = exp2f(acc[v] * scale_log2 - csh[wv][t * 32 + r]);
        colsum += (key <= p && key < g.n) ? e : 0.f;
      }
      colsum += __shfl_xor(colsum, 32, 64);
      total += colsum;
      if (per_head) {
        hsum += colsum;
        const int tile = tile0 + t;
        const bool last_of_head = (t == TG - 1) || ((tile + 1) % g.tph == 0);
        if (last_of_head) {
          if (hf == 0 && key < g.n) {
            const int head = kvh * g.G + tile / g.tph;
            float* dst = A + ((int64_t)l * g.Hq + head) * g.n + key;
            const bool first_in_launch = (tile % g.tph) <= t;   // head started in this launch
            *dst = first_in_launch ? hsum * inv_w : *dst + hsum * inv_w;
          }
          hsum = 0.f;
        }
      }
    }
    if (!per_head && hf == 0 && key < g.n) {
      float* dst = A + ((int64_t)l * g.Hkv + kvh) * g.n + key;
      *dst = tile0 == 0 ? total * inv_group : *dst + total * inv_group;
    }
#pragma unroll
    for (int st = 0; st < D / 16; ++st) kf[st] = kn[st];
  }
}

// ---------------------------------------------------------------- float32 path
// Plain vector-ALU version for float32 inputs (small shapes).  Rows are indexed
// (head in group, window row) without padding.
constexpr int NTF = 256;

__global__ void __launch_bounds__(NTF)
win_f32_stats(ConstPtrs qs, ConstPtrs ks, Geo g, float scale_log2, float* __restrict__ c) {
  __shared__ float qsh[256];
  __shared__ float red[NTF / 64];
  const int R = g.G * g.w;
  const int64_t id = blockIdx.x;               // (l, kvh, row)
  const int r = (int)(id % R);
  const int kvh = (int)((id / R) % g.Hkv);
  const int l = (int)(id / ((int64_t)R * g.Hkv));
  const float* q = (const float*)qs.p[l] + ((int64_t)(kvh * g.G + r / g.w) * g.w + r % g.w) * g.d;
  const float* k = (const float*)ks.p[l] + (int64_t)kvh * g.n * g.d;
  for (int e = threadIdx.x; e < g.d; e += NTF) qsh[e] = q[e];
  __syncthreads();
  const int64_t p = g.n - g.w + r % g.w;
  float m = -INFINITY, s = 0.f;
  for (int64_t j = threadIdx.x; j <= p; j += NTF) {
    float dot = 0.f;
    for (int e = 0; e < g.d; ++e) dot += qsh[e] * k[j * g.d + e];
    const float x = dot * scale_log2;
    const float mn = fmaxf(m, x);
    s = s * exp2f(m - mn) + exp2f(x - mn);
    m = mn;
  }
  const float M = block_max<NTF>(m, red);
  const float S = block_sum<NTF>(m > -INFINITY ? s * exp2f(m - M) : 0.f, red);
  if (threadIdx.x == 0) c[id] = M + log2f(S);
}

__global__ void __launch_bounds__(NTF)
win_f32_accum(ConstPtrs qs, ConstPtrs ks, Geo g, float scale_log2, const float* __restrict__ c,
              int per_head, float* __restrict__ A) {
  extern __shared__ float qall[];              // [R, d]
  const int R = g.G * g.w;
  const int64_t nblk = (g.n + NTF - 1) / NTF;
  const int64_t id = blockIdx.x;
  const int kvh = (int)((id / nblk) % g.Hkv);
  const int l = (int)(id / (nblk * g.Hkv));
  const int64_t j = (id % nblk) * NTF + threadIdx.x;
  const float* q = (const float*)qs.p[l] + (int64_t)kvh * g.G * g.w * g.d;
  for (int e = threadIdx.x; e < R * g.d; e += NTF) qall[e] = q[e];
  __syncthreads();
  if (j >= g.n) return;
  const float* kr = (const float*)ks.p[l] + ((int64_t)kvh * g.n + j) * g.d;
  const float* cr = c + ((int64_t)l * g.Hkv + kvh) * R;
  float total = 0.f;
  for (int h = 0; h < g.G; ++h) {
    float hs = 0.f;
    for (int rr = 0; rr < g.w; ++rr) {
      if (j > g.n - g.w + rr) continue;
      const float* qr = qall + (h * g.w + rr) * g.d;
      float dot = 0.f;
      for (int e = 0; e < g.d; ++e) dot += qr[e] * kr[e];
      hs += exp2f(dot * scale_log2 - cr[h * g.w + rr]);
    }
    if (per_head) A[((int64_t)l * g.Hq + kvh * g.G + h) * g.n + j] = hs / (float)g.w;
    total += hs;
  }
  if (!per_head) A[((int64_t)l * g.Hkv + kvh) * g.n + j] = total / (float)(g.G * g.w);
}

// ---------------------------------------------------------------- host
struct Plan {
  Geo g;
  bool mfma;
  size_t part_bytes, c_bytes;
};

int make_plan(int L, int Hq, int Hkv, int64_t n, int w, int d, int dtype, Plan* P) {
  Geo g{};
  g.Hq = Hq; g.Hkv = Hkv; g.G = Hq / Hkv; g.w = w; g.d = d; g.n = n;
  g.tph = (w + 31) / 32;
  g.ntiles = g.G * g.tph;
  g.nb = (int)((n + KPW - 1) / KPW);
  const int lc = L < kLayersPerLaunch ? L : kLayersPerLaunch;
  P->g = g;
  P->mfma = (dtype == KVC_BF16);
  if (P->mfma) {
    P->part_bytes = (size_t)lc * Hkv * g.nb * g.ntiles * 32 * sizeof(float2);
    P->c_bytes = (size_t)lc * Hkv * g.ntiles * 32 * sizeof(float);
  } else {
    P->part_bytes = 0;
    P->c_bytes = (size_t)lc * Hkv * g.G * w * sizeof(float);
  }
  return KVC_OK;
}

template <int D, int TG>
void launch_tiles(const ConstPtrs& qt, const ConstPtrs& kt, const Geo& g, int tile0, int lc,
                  float sl2, float2* part, float* cfin, int per_head, float* A, hipStream_t s,
                  bool stats) {
  const int64_t ntask = (int64_t)lc * g.Hkv * g.nb;
  const unsigned grid = (unsigned)((ntask + 3) / 4);
  if (stats)
    hipLaunchKernelGGL((win_pass1<D, TG>), dim3(grid), dim3(NTW), 0, s, qt, kt, g, tile0, lc, sl2, part);
  else
    hipLaunchKernelGGL((win_pass2<D, TG>), dim3(grid), dim3(NTW), 0, s, qt, kt, g, tile0, lc, sl2,
                       (const float*)cfin, per_head, A);
}

template <int D>
void launch_group(int tg, const ConstPtrs& qt, const ConstPtrs& kt, const Geo& g, int tile0, int lc,
                  float sl2, float2* part, float* cfin, int per_head, float* A, hipStream_t s,
                  bool stats) {
  switch (tg) {
    case 1: launch_tiles<D, 1>(qt, kt, g, tile0, lc, sl2, part, cfin, per_head, A, s, stats); break;
    case 2: launch_tiles<D, 2>(qt, kt, g, tile0, lc, sl2, part, cfin, per_head, A, s, stats); break;
    case 3: launch_tiles<D, 3>(qt, kt, g, tile0, lc, sl2, part, cfin, per_head, A, s, stats); break;
    default: launch_tiles<D, 4>(qt, kt, g, tile0, lc, sl2, part, cfin, per_head, A, s, stats); break;
  }
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" size_t kvc_score_window_attn_workspace_size(int L, int Hq, int Hkv, int64_t n, int w,
                                                       int d, int dtype) {
  if (L < 1 || Hkv < 1 || Hq < Hkv || n < 1 || w < 1 || d < 1) return 0;
  Plan P;
  make_plan(L, Hq, Hkv, n, w, d, dtype, &P);
  return P.part_bytes + P.c_bytes + 256;
}

extern "C" int kvc_score_window_attn(const void* const* q_win, const void* const* k, int dtype,
                                     int L, int Hq, int Hkv, int64_t n, int w, int d, float scale,
                                     int per_query_head, float* A_out, void* ws, size_t ws_bytes,
                                     void* stream) {
  clear_error();
  if (!dtype_ok(dtype)) return KVC_FAIL(KVC_ERR_DTYPE, "kvc_score_window_attn: dtype %d", dtype);
  KVC_REQUIRE(L >= 1 && L <= KVC_MAX_LAYERS, "kvc_score_window_attn: need 1 <= L <= %d", KVC_MAX_LAYERS);
  KVC_REQUIRE(Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0, "kvc_score_window_attn: need Hq %% Hkv == 0");
  KVC_REQUIRE(n >= 1 && w >= 1 && w <= n, "kvc_score_window_attn: need 1 <= w <= n");
  KVC_REQUIRE(n <= 0x7fffffffLL, "kvc_score_window_attn: n > 2^31-1");
  KVC_REQUIRE(per_query_head == 0 || per_query_head == 1, "kvc_score_window_attn: per_query_head");
  KVC_REQUIRE(q_win && k && A_out, "kvc_score_window_attn: null pointer");
  for (int l = 0; l < L; ++l)
    KVC_REQUIRE(q_win[l] && k[l], "kvc_score_window_attn: null pointer in layer %d", l);
  Plan P;
  make_plan(L, Hq, Hkv, n, w, d, dtype, &P);
  const Geo& g = P.g;
  if (P.mfma) {
    KVC_REQUIRE(d == 64 || d == 128, "kvc_score_window_attn: bf16 needs d in {64, 128}");
    KVC_REQUIRE(g.ntiles <= MAX_TILES, "kvc_score_window_attn: (Hq/Hkv)*ceil(w/32) > %d", MAX_TILES);
    for (int l = 0; l < L; ++l)
      KVC_REQUIRE((uintptr_t)q_win[l] % 16 == 0 && (uintptr_t)k[l] % 16 == 0,
                  "kvc_score_window_attn: bf16 tensors must be 16-byte aligned");
  } else {
    KVC_REQUIRE(d >= 1 && d <= 256, "kvc_score_window_attn: float32 needs d <= 256");
    KVC_REQUIRE((int64_t)g.G * w * d * 4 <= 64 * 1024,
                "kvc_score_window_attn: float32 path needs (Hq/Hkv)*w*d*4 <= 64 KB");
  }
  const size_t need = P.part_bytes + P.c_bytes;
  if (!ws || ws_bytes < need)
    return KVC_FAIL(KVC_ERR_WORKSPACE, "kvc_score_window_attn: workspace needs %zu bytes", need);
  char* base = (char*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
  if ((size_t)(base - (char*)ws) + need > ws_bytes)
    return KVC_FAIL(KVC_ERR_WORKSPACE, "kvc_score_window_attn: workspace needs %zu bytes", need + 256);
  float2* part = (float2*)base;
  float* cfin = (float*)(base + P.part_bytes);
  hipStream_t s = as_stream(stream);
  const float sl2 = scale * LOG2E;
  const int Aheads = per_query_head ? Hq : Hkv;

  for (int l0 = 0; l0 < L; l0 += kLayersPerLaunch) {
    const int lc = min(kLayersPerLaunch, L - l0);
    ConstPtrs qt{}, kt{};
    for (int i = 0; i < lc; ++i) { qt.p[i] = q_win[l0 + i]; kt.p[i] = k[l0 + i]; }
    float* A = A_out + (int64_t)l0 * Aheads * n;
    if (P.mfma) {
      const int64_t ngroups = (int64_t)lc * Hkv;
      for (int t0 = 0; t0 < g.ntiles; t0 += MAX_TG) {
        const int tg = min(MAX_TG, g.ntiles - t0);
        if (d == 64) launch_group<64>(tg, qt, kt, g, t0, lc, sl2, part, cfin, per_query_head, A, s, true);
        else launch_group<128>(tg, qt, kt, g, t0, lc, sl2, part, cfin, per_query_head, A, s, true);
      }
      hipLaunchKernelGGL(win_combine, dim3((unsigned)ngroups), dim3(256), 0, s, (const float2*)part,
                         g.nb, g.ntiles * 32, ngroups, cfin);
      for (int t0 = 0; t0 < g.ntiles; t0 += MAX_TG) {
        const int tg = min(MAX_TG, g.ntiles - t0);
        if (d == 64) launch_group<64>(tg, qt, kt, g, t0, lc, sl2, part, cfin, per_query_head, A, s, false);
        else launch_group<128>(tg, qt, kt, g, t0, lc, sl2, part, cfin, per_query_head, A, s, false);
      }
    } else {
      const int R = g.G * w;
      hipLaunchKernelGGL(win_f32_stats, dim3((unsigned)((int64_t)lc * Hkv * R)), dim3(NTF), 0, s,
                         qt, kt, g, sl2, cfin);
      const int64_t nblk = (n + NTF - 1) / NTF;
      hipLaunchKernelGGL(win_f32_accum, dim3((unsigned)(lc * Hkv * nblk)), dim3(NTF),
                         (size_t)R * d * sizeof(float), s, qt, kt, g, sl2, (const float*)cfin,
                         per_query_head, A);
    }
  }
  return launch_status("kvc_score_window_attn");
}
