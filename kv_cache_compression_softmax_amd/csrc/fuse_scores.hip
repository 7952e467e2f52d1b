// Importance fusion S = alpha * A + (1 - alpha) * softmax_tokens(D * H), and the
// layer's mean entropy score Ebar.
//
// [InfoKV] Contributions, Method and Technical detail: the layer entropy score
// E_i = D_i * H_i is normalised by a softmax over the tokens of the layer and
// mixed with the window attention; [InfoKV] Method / Glossary (adaptive budget):
// the layer's share of the total entropy score drives the adaptive budget.
//
// Two small kernels, both deterministic:
//   stats  one block per (layer, chunk of tokens) computes max E, sum exp(E - max)
//          and sum E over its chunk; the chunk partials are merged in index order
//          by a second tiny launch into (max, sum, Ebar) per layer;
//   apply  elementwise over [L, Hkv, n], recomputing E from D and H (cheaper than
//          storing it).
#include "common.h"

namespace kvc {
namespace {

constexpr int NT = 256;
constexpr int CHUNK = 1024;     // tokens per stats block (4 per thread, held in registers)
constexpr int PER = CHUNK / NT;
static_assert(CHUNK % NT == 0, "whole tokens per thread");

struct Part { float m, s, e; };

__global__ void __launch_bounds__(NT)
fuse_stats(const float* __restrict__ D, const float* __restrict__ H, int64_t n, int nchunk,
           Part* __restrict__ part) {
  __shared__ float red[NT / 64];
  const int l = blockIdx.y, c = blockIdx.x;
  const int64_t i0 = (int64_t)c * CHUNK, i1 = min(n, i0 + CHUNK);
  const float* Dl = D + (int64_t)l * n;
  float e[PER];
  float m = -INFINITY, esum = 0.f;
#pragma unroll
  for (int u = 0; u < PER; ++u) {                // this thread's tokens, read once
    const int64_t i = i0 + threadIdx.x + (int64_t)u * NT;
    e[u] = i < i1 ? Dl[i] * H[i] : 0.f;
    if (i < i1) { m = fmaxf(m, e[u]); esum += e[u]; }
  }
  const float M = block_max<NT>(m, red);
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if (i0 + threadIdx.x + (int64_t)u * NT < i1) s += expf(e[u] - M);
  const float S = block_sum<NT>(s, red);
  const float ES = block_sum<NT>(esum, red);
  if (threadIdx.x == 0) part[(int64_t)l * nchunk + c] = Part{M, S, ES};
}

__global__ void fuse_stats_merge(const Part* __restrict__ part, int nchunk, int L, int64_t n,
                                 float2* __restrict__ stats, float* __restrict__ Ebar) {
  const int l = blockIdx.x * blockDim.x + threadIdx.x;
  if (l >= L) return;
  const Part* p = part + (int64_t)l * nchunk;
  float M = -INFINITY;
  for (int c = 0; c < nchunk; ++c) M = fmaxf(M, p[c].m);
  float S = 0.f, ES = 0.f;
  for (int c = 0; c < nchunk; ++c) { S += p[c].s * expf(p[c].m - M); ES += p[c].e; }
  stats[l] = make_float2(M, 1.0f / S);
  if (Ebar) Ebar[l] = ES / (float)n;
}

__global__ void __launch_bounds__(NT)
fuse_apply(const float* __restrict__ A, const float* __restrict__ D, const float* __restrict__ H,
           const float2* __restrict__ stats, int Hkv, int64_t n, float alpha,
           float* __restrict__ S) {
  const int64_t row = blockIdx.y;               // (layer, KV head)
  const int l = (int)(row / Hkv);
  const float2 st = stats[l];
  const float* Dl = D + (int64_t)l * n;
  const float* Ar = A + row * n;
  float* Sr = S + row * n;
  const float beta = 1.0f - alpha;
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) {
    const float sigma = expf(Dl[i] * H[i] - st.x) * st.y;
    Sr[i] = alpha * Ar[i] + beta * sigma;
  }
}

// The same with 16-byte accesses, for rows a multiple of 4 long (16-byte
// aligned); the per-element arithmetic is the same.
__global__ void __launch_bounds__(NT)
fuse_apply4(const float4* __restrict__ A, const float* __restrict__ D, const float* __restrict__ H,
            const float2* __restrict__ stats, int Hkv, int64_t n, float alpha,
            float4* __restrict__ S) {
  const int64_t row = blockIdx.y;               // (layer, KV head)
  const int l = (int)(row / Hkv);
  const float2 st = stats[l];
  const int64_t n4 = n / 4;
  const float4* Dl = reinterpret_cast<const float4*>(D + (int64_t)l * n);
  const float4* H4 = reinterpret_cast<const float4*>(H);
  const float4* Ar = A + row * n4;
  float4* Sr = S + row * n4;
  const float beta = 1.0f - alpha;
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n4; i += (int64_t)gridDim.x * NT) {
    const float4 a = Ar[i], d = Dl[i], h = H4[i];
    float4 r;
    r.x = alpha * a.x + beta * (expf(d.x * h.x - st.x) * st.y);
    r.y = alpha * a.y + beta * (expf(d.y * h.y - st.x) * st.y);
    r.z = alpha * a.z + beta * (expf(d.z * h.z - st.x) * st.y);
    r.w = alpha * a.w + beta * (expf(d.w * h.w - st.x) * st.y);
    Sr[i] = r;
  }
}

// ---- cache slots: one entropy score per (layer, KV head, slot) ----------------
// After a compaction each KV head holds its own token set, so E is a row per
// (layer, KV head) and the softmax runs over that row.

__global__ void __launch_bounds__(NT)
slot_stats(const float* __restrict__ E, int64_t n, int nchunk, Part* __restrict__ part) {
  __shared__ float red[NT / 64];
  const int64_t row = blockIdx.y;
  const int c = blockIdx.x;
  const int64_t i0 = (int64_t)c * CHUNK, i1 = min(n, i0 + CHUNK);
  const float* Er = E + row * n;
  float e[PER];
  float m = -INFINITY, esum = 0.f;
#pragma unroll
  for (int u = 0; u < PER; ++u) {                // this thread's tokens, read once
    const int64_t i = i0 + threadIdx.x + (int64_t)u * NT;
    e[u] = i < i1 ? Er[i] : 0.f;
    if (i < i1) { m = fmaxf(m, e[u]); esum += e[u]; }
  }
  const float M = block_max<NT>(m, red);
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if (i0 + threadIdx.x + (int64_t)u * NT < i1) s += expf(e[u] - M);
  const float S = block_sum<NT>(s, red);
  const float ES = block_sum<NT>(esum, red);
  if (threadIdx.x == 0) part[row * nchunk + c] = Part{M, S, ES};
}

// one thread per row merges its chunks in index order; one thread per layer sums
// its rows' E in (head, chunk) order for Ebar
__global__ void slot_stats_merge(const Part* __restrict__ part, int nchunk, int L, int Hkv,
                                 int64_t n, float2* __restrict__ stats, float* __restrict__ Ebar) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < L * Hkv) {
    const Part* p = part + (int64_t)r * nchunk;
    float M = -INFINITY;
    for (int c = 0; c < nchunk; ++c) M = fmaxf(M, p[c].m);
    float S = 0.f;
    for (int c = 0; c < nchunk; ++c) S += p[c].s * expf(p[c].m - M);
    stats[r] = make_float2(M, 1.0f / S);
  }
  if (Ebar && r < L) {
    const Part* p = part + (int64_t)r * Hkv * nchunk;
    float ES = 0.f;
    for (int c = 0; c < Hkv * nchunk; ++c) ES += p[c].e;
    Ebar[r] = ES / ((float)Hkv * (float)n);
  }
}

__global__ void __launch_bounds__(NT)
slot_apply(const float* __restrict__ A, const float* __restrict__ E, const float2* __restrict__ stats,
           int64_t n, float alpha, float* __restrict__ S) {
  const int64_t row = blockIdx.y;               // (layer, KV head)
  const float2 st = stats[row];
  const float* Ar = A + row * n;
  const float* Er = E + row * n;
  float* Sr = S + row * n;
  const float beta = 1.0f - alpha;
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT)
    Sr[i] = alpha * Ar[i] + beta * (expf(Er[i] - st.x) * st.y);
}

// E[l, g, offset + i] = D[l, i] * H[i] for every KV head g
__global__ void __launch_bounds__(NT)
slot_append(const float* __restrict__ D, const float* __restrict__ H, int Hkv, int64_t t,
            int64_t cap, int64_t offset, float* __restrict__ E) {
  const int64_t row = blockIdx.y;               // (layer, KV head)
  const int64_t l = row / Hkv;
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < t; i += (int64_t)gridDim.x * NT)
    E[row * cap + offset + i] = D[l * t + i] * H[i];
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" size_t kvc_fuse_scores_workspace_size(int L, int64_t n) {
  if (L < 1 || n < 1) return 0;
  const int64_t nchunk = (n + CHUNK - 1) / CHUNK;
  return (size_t)L * nchunk * sizeof(Part) + (size_t)L * sizeof(float2) + 256;
}

extern "C" int kvc_fuse_scores(const float* A, const float* D, const float* H, int L, int Hkv,
                               int64_t n, float alpha_fuse, float* S_out, float* Ebar_out,
                               void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  KVC_REQUIRE(L >= 1 && L <= KVC_MAX_LAYERS, "kvc_fuse_scores: need 1 <= L <= %d", KVC_MAX_LAYERS);
  KVC_REQUIRE(Hkv >= 1 && n >= 1, "kvc_fuse_scores: need Hkv >= 1 and n >= 1");
  KVC_REQUIRE(alpha_fuse >= 0.f && alpha_fuse <= 1.f, "kvc_fuse_scores: alpha_fuse outside [0, 1]");
  KVC_REQUIRE(A && D && H && S_out, "kvc_fuse_scores: null pointer");
  const int64_t nchunk = (n + CHUNK - 1) / CHUNK;
  KVC_REQUIRE(nchunk <= 0x7fffffff, "kvc_fuse_scores: n too large");
  const int64_t rows = (int64_t)L * Hkv;
  KVC_REQUIRE(rows <= 65535, "kvc_fuse_scores: L * Hkv > 65535");
  const size_t need = kvc_fuse_scores_workspace_size(L, n);
  if (!ws || ws_bytes < need)
    return KVC_FAIL(KVC_ERR_WORKSPACE, "kvc_fuse_scores: workspace needs %zu bytes", need);
  char* base = (char*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
  Part* part = (Part*)base;
  float2* stats = (float2*)(base + (size_t)L * nchunk * sizeof(Part));
  hipStream_t s = as_stream(stream);
  hipLaunchKernelGGL(fuse_stats, dim3((unsigned)nchunk, (unsigned)L), dim3(NT), 0, s, D, H, n,
                     (int)nchunk, part);
  hipLaunchKernelGGL(fuse_stats_merge, dim3((L + 63) / 64), dim3(64), 0, s, (const Part*)part,
                     (int)nchunk, L, n, stats, Ebar_out);
  const bool vec = n % 4 == 0 && ((uintptr_t)A | (uintptr_t)D | (uintptr_t)H | (uintptr_t)S_out) % 16 == 0;
  if (vec) {
    const int64_t gx64 = (n / 4 + NT - 1) / NT;  // one 16-byte group per thread
    const unsigned gx = (unsigned)(gx64 < 1024 ? gx64 : 1024);
    hipLaunchKernelGGL(fuse_apply4, dim3(gx, (unsigned)rows), dim3(NT), 0, s, (const float4*)A, D, H,
                       (const float2*)stats, Hkv, n, alpha_fuse, (float4*)S_out);
  } else {
    const int64_t gx64 = (n + NT * 4 - 1) / (NT * 4);
    const unsigned gx = (unsigned)(gx64 < 1024 ? gx64 : 1024);
    hipLaunchKernelGGL(fuse_apply, dim3(gx, (unsigned)rows), dim3(NT), 0, s, A, D, H,
                       (const float2*)stats, Hkv, n, alpha_fuse, S_out);
  }
  return launch_status("kvc_fuse_scores");
}

extern "C" size_t kvc_fuse_scores_slots_workspace_size(int L, int Hkv, int64_t n) {
  if (L < 1 || Hkv < 1 || n < 1) return 0;
  const int64_t nchunk = (n + CHUNK - 1) / CHUNK;
  return (size_t)L * Hkv * nchunk * sizeof(Part) + (size_t)L * Hkv * sizeof(float2) + 256;
}

extern "C" int kvc_fuse_scores_slots(const float* A, const float* E, int L, int Hkv, int64_t n,
                                     float alpha_fuse, float* S_out, float* Ebar_out, void* ws,
                                     size_t ws_bytes, void* stream) {
  clear_error();
  KVC_REQUIRE(L >= 1 && L <= KVC_MAX_LAYERS, "kvc_fuse_scores_slots: need 1 <= L <= %d", KVC_MAX_LAYERS);
  KVC_REQUIRE(Hkv >= 1 && n >= 1, "kvc_fuse_scores_slots: need Hkv >= 1 and n >= 1");
  KVC_REQUIRE(alpha_fuse >= 0.f && alpha_fuse <= 1.f, "kvc_fuse_scores_slots: alpha_fuse outside [0, 1]");
  KVC_REQUIRE(A && E && S_out, "kvc_fuse_scores_slots: null pointer");
  const int64_t nchunk = (n + CHUNK - 1) / CHUNK;
  const int64_t rows = (int64_t)L * Hkv;
  KVC_REQUIRE(rows <= 65535 && nchunk <= 0x7fffffff, "kvc_fuse_scores_slots: L * Hkv > 65535");
  const size_t need = kvc_fuse_scores_slots_workspace_size(L, Hkv, n);
  if (!ws || ws_bytes < need)
    return KVC_FAIL(KVC_ERR_WORKSPACE, "kvc_fuse_scores_slots: workspace needs %zu bytes", need);
  char* base = (char*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
  Part* part = (Part*)base;
  float2* stats = (float2*)(base + (size_t)rows * nchunk * sizeof(Part));
  hipStream_t s = as_stream(stream);
  hipLaunchKernelGGL(slot_stats, dim3((unsigned)nchunk, (unsigned)rows), dim3(NT), 0, s, E, n,
                     (int)nchunk, part);
  const int64_t nt = rows > L ? rows : L;
  hipLaunchKernelGGL(slot_stats_merge, dim3((unsigned)((nt + 63) / 64)), dim3(64), 0, s,
                     (const Part*)part, (int)nchunk, L, Hkv, n, stats, Ebar_out);
  const int64_t gx64 = (n + NT * 4 - 1) / (NT * 4);
  const unsigned gx = (unsigned)(gx64 < 1024 ? gx64 : 1024);
  hipLaunchKernelGGL(slot_apply, dim3(gx, (unsigned)rows), dim3(NT), 0, s, A, E,
                     (const float2*)stats, n, alpha_fuse, S_out);
  return launch_status("kvc_fuse_scores_slots");
}

extern "C" int kvc_append_entropy_scores(const float* D, const float* H, int L, int Hkv, int64_t t,
                                         float* E, int64_t cap, int64_t offset, void* stream) {
  clear_error();
  KVC_REQUIRE(L >= 1 && L <= KVC_MAX_LAYERS, "kvc_append_entropy_scores: need 1 <= L <= %d", KVC_MAX_LAYERS);
  KVC_REQUIRE(Hkv >= 1 && t >= 1 && (int64_t)L * Hkv <= 65535, "kvc_append_entropy_scores: need Hkv, t >= 1");
  KVC_REQUIRE(offset >= 0 && offset + t <= cap, "kvc_append_entropy_scores: need 0 <= offset and offset + t <= cap");
  KVC_REQUIRE(D && H && E, "kvc_append_entropy_scores: null pointer");
  const int64_t gx64 = (t + NT - 1) / NT;
  const unsigned gx = (unsigned)(gx64 < 1024 ? gx64 : 1024);
  hipLaunchKernelGGL(slot_append, dim3(gx, (unsigned)((int64_t)L * Hkv)), dim3(NT), 0,
                     as_stream(stream), D, H, Hkv, t, cap, offset, E);
  return launch_status("kvc_append_entropy_scores");
}
