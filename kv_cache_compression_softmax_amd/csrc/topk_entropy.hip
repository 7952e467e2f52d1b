// Top-k restricted entropy of each final-layer logits row.
//
// [InfoKV] Method and Glossary (top-k restricted entropy): for every token the
// entropy of the model's next-token distribution is taken over its k most likely
// tokens only, renormalised over them.
//
// One workgroup streams one row from HBM exactly once.  Instead of holding the
// 256 KB row on chip, it keeps a small candidate set in LDS:
//   * after the first chunk it knows tau = the k-th largest key seen so far;
//   * every later element is compared with tau and only strictly larger ones are
//     appended (an element equal to tau can never add to the top-k multiset:
//     enough copies of tau are already held);
//   * when the candidate set grows past RESEL, an exact radix select over the
//     candidates (8-bit digits of the order-preserving key) recomputes tau and
//     shrinks the set back to exactly k (all keys > tau, then copies of tau).
// Any element of the final top-k is >= every intermediate tau, so nothing it
// needs is ever dropped.  For random rows the filter passes a few hundred
// elements per row, so the kernel runs at the speed of the row stream.
// Appends use an ordered block scan (no atomics decide positions), so the
// candidate order, and with it every float sum, is deterministic.
#include "common.h"

namespace kvc {
namespace {

constexpr int NT = 256;      // threads per workgroup
constexpr int NV = 2;        // 16-byte vectors per thread per chunk
constexpr int CAP = 8192;    // candidate capacity (keys)
constexpr int RESEL = 2048;  // re-select once more candidates than this are held

template <typename T> struct Tr;
template <> struct Tr<uint16_t> {                 // bf16 bit patterns
  using Key = uint16_t;
  static constexpr int VEC = 8;
  static constexpr int DIGITS = 2;
  __device__ static Key key(uint16_t raw) { return (Key)bf16_key(raw); }
  __device__ static float value(Key k) { return key_bf16(k); }
};
template <> struct Tr<float> {
  using Key = uint32_t;
  static constexpr int VEC = 4;
  static constexpr int DIGITS = 4;
  __device__ static Key key(float raw) { return f32_key(raw); }
  __device__ static float value(Key k) { return key_f32(k); }
};

template <typename T>
struct Smem {
  typename Tr<T>::Key cand[CAP];
  typename Tr<T>::Key stage[KVC_MAX_TOPK_ENTROPY];
  int hist[256];
  int wtot[2][NT / kWave];
  int scan[NT / kWave];
  int pick[2];
  float red[NT / kWave];
};

// Exact k-th largest key of cand[0..count) and the number of keys above it.
// Then rewrites cand[0..k) as (keys > tau in their current order, then k - cgt
// copies of tau).  Called by all threads; returns the new count (= k).
template <typename T>
__device__ int reselect(Smem<T>& sm, int count, int k) {
  using Key = typename Tr<T>::Key;
  constexpr int DIG = Tr<T>::DIGITS;
  const int tid = threadIdx.x;
  uint32_t prefix = 0;
  int above = 0, need = k;
#pragma unroll 1
  for (int p = DIG - 1; p >= 0; --p) {
    const int shift = 8 * p;
    const uint32_t hi_mask = (p == DIG - 1) ? 0u : (uint32_t)(~0ull << (shift + 8));
    sm.hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < count; i += NT) {
      uint32_t key = sm.cand[i];
      if ((key & hi_mask) == (prefix & hi_mask)) atomicAdd(&sm.hist[(key >> shift) & 255], 1);
    }
    __syncthreads();
    // thread t owns bin 255 - t: inclusive scan from the top bin down
    const int c = sm.hist[255 - tid];
    int tot;
    const int incl = block_exclusive_scan<NT>(c, sm.scan, &tot) + c;
    if (incl >= need && incl - c < need) { sm.pick[0] = 255 - tid; sm.pick[1] = incl - c; }
    __syncthreads();
    prefix |= (uint32_t)sm.pick[0] << shift;
    above += sm.pick[1];
    need -= sm.pick[1];
    __syncthreads();
  }
  const Key tau = (Key)prefix;
  const int cgt = above;
  // ordered compaction of keys > tau into stage[0..cgt)
  const int seg = (count + NT - 1) / NT;
  const int b = min(count, tid * seg), e = min(count, b + seg);
  int mine = 0;
  for (int i = b; i < e; ++i) mine += sm.cand[i] > tau;
  int tot;
  int pos = block_exclusive_scan<NT>(mine, sm.scan, &tot);
  for (int i = b; i < e; ++i) {
    Key key = sm.cand[i];
    if (key > tau) sm.stage[pos++] = key;
  }
  for (int i = cgt + tid; i < k; i += NT) sm.stage[i] = tau;
  __syncthreads();
  for (int i = tid; i < k; i += NT) sm.cand[i] = sm.stage[i];
  __syncthreads();
  return k;
}

template <typename T>
__device__ __forceinline__ void load_vec(const T* row, int64_t e0, int64_t vocab, bool vec_ok,
                                         T (&out)[Tr<T>::VEC], int& nvalid) {
  constexpr int VEC = Tr<T>::VEC;
  int64_t left = vocab - e0;
  nvalid = left >= VEC ? VEC : (left > 0 ? (int)left : 0);
  if (nvalid == VEC && vec_ok) {
    uint4 u = *reinterpret_cast<const uint4*>(row + e0);
    __builtin_memcpy(&out, &u, 16);
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) out[e] = (e < nvalid) ? row[e0 + e] : T(0);
  }
}

template <typename T>
__global__ void __launch_bounds__(NT)
topk_entropy_kernel(const T* __restrict__ logits, int64_t vocab, int64_t stride, int k,
                    float* __restrict__ H) {
  using Key = typename Tr<T>::Key;
  constexpr int VEC = Tr<T>::VEC;
  constexpr int E = NV * VEC;
  constexpr int CHUNK = NT * E;
  __shared__ Smem<T> sm;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int64_t rowi = blockIdx.x;
  const T* row = logits + rowi * stride;
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(row) & 15) == 0);
  const int64_t nchunks = (vocab + CHUNK - 1) / CHUNK;

  T cur[NV][VEC], nxt[NV][VEC];
  int ncur[NV], nnxt[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) load_vec<T>(row, (int64_t)(v * NT + tid) * VEC, vocab, vec_ok, cur[v], ncur[v]);

  int count = 0, parity = 0;
  bool have_tau = false;
  Key tau = 0;
#pragma unroll 1
  for (int64_t c = 0; c < nchunks; ++c) {
    if (c + 1 < nchunks) {
#pragma unroll
      for (int v = 0; v < NV; ++v)
        load_vec<T>(row, (c + 1) * CHUNK + (int64_t)(v * NT + tid) * VEC, vocab, vec_ok, nxt[v], nnxt[v]);
    }
    Key keys[E];
    uint32_t pass = 0;
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        Key kk = Tr<T>::key(cur[v][e]);
        keys[v * VEC + e] = kk;
        bool p = (e < ncur[v]) && (!have_tau || kk > tau);
        pass |= (uint32_t)p << (v * VEC + e);
      }
    const int cnt = __builtin_popcount(pass);
    const int incl = wave_inclusive_scan(cnt);
    if (lane == kWave - 1) sm.wtot[parity][wv] = incl;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / kWave; ++i) {
      int s = sm.wtot[parity][i];
      base += (i < wv) ? s : 0;
      tot += s;
    }
    if (pass) {
      int pos = count + base + incl - cnt;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (pass & (1u << e)) sm.cand[pos++] = keys[e];
    }
    count += tot;
    parity ^= 1;
    if (!have_tau || count > RESEL) {
      __syncthreads();
      count = reselect<T>(sm, count, k);
      tau = sm.cand[k - 1];   // the copies of tau sit at the end
      // the smallest key held is tau (all others are > tau)
      have_tau = true;
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      ncur[v] = nnxt[v];
#pragma unroll
      for (int e = 0; e < VEC; ++e) cur[v][e] = nxt[v][e];
    }
  }
  __syncthreads();
  if (count > k) count = reselect<T>(sm, count, k);

  // entropy over the k held keys (float32, fixed reduction order)
  float mloc = -INFINITY;
  for (int i = tid; i < k; i += NT) mloc = fmaxf(mloc, Tr<T>::value(sm.cand[i]));
  const float m = block_max<NT>(mloc, sm.red);
  float zloc = 0.f;
  for (int i = tid; i < k; i += NT) zloc += expf(Tr<T>::value(sm.cand[i]) - m);
  const float Z = block_sum<NT>(zloc, sm.red);
  const float lnZ = logf(Z), invZ = 1.0f / Z;
  float hloc = 0.f;
  for (int i = tid; i < k; i += NT) {
    float t = Tr<T>::value(sm.cand[i]);
    hloc += expf(t - m) * invZ * ((m - t) + lnZ);   // -p ln p, every term >= 0
  }
  const float h = block_sum<NT>(hloc, sm.red);
  if (tid == 0) H[rowi] = h;
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" int kvc_topk_entropy(const void* logits, int dtype, int64_t rows, int64_t vocab,
                                int64_t row_stride, int topk, float* H_out, void* stream) {
  clear_error();
  if (!dtype_ok(dtype)) return KVC_FAIL(KVC_ERR_DTYPE, "kvc_topk_entropy: dtype %d", dtype);
  KVC_REQUIRE(rows >= 0, "kvc_topk_entropy: rows < 0");
  KVC_REQUIRE(rows <= 0x7fffffff, "kvc_topk_entropy: rows > 2^31-1");
  KVC_REQUIRE(vocab >= 1 && row_stride >= vocab, "kvc_topk_entropy: need 1 <= vocab <= row_stride");
  KVC_REQUIRE(topk >= 1 && topk <= KVC_MAX_TOPK_ENTROPY && topk <= vocab,
              "kvc_topk_entropy: need 1 <= topk <= min(vocab, %d)", KVC_MAX_TOPK_ENTROPY);
  if (rows == 0) return KVC_OK;
  KVC_REQUIRE(logits && H_out, "kvc_topk_entropy: null pointer");
  hipStream_t s = as_stream(stream);
  if (dtype == KVC_BF16)
    hipLaunchKernelGGL(topk_entropy_kernel<uint16_t>, dim3((unsigned)rows), dim3(NT), 0, s,
                       (const uint16_t*)logits, vocab, row_stride, topk, H_out);
  else
    hipLaunchKernelGGL(topk_entropy_kernel<float>, dim3((unsigned)rows), dim3(NT), 0, s,
                       (const float*)logits, vocab, row_stride, topk, H_out);
  return launch_status("kvc_topk_entropy");
}
