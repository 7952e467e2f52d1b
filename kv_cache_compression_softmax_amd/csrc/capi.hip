// Host-side parts of the C ABI: status strings, per-thread error text, and the
// two host-only budget calls of [InfoKV] (uniform and adaptive layer budgets).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "common.h"

namespace kvc {

static thread_local char g_last_error[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

void clear_error() { g_last_error[0] = 0; }

int launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return KVC_FAIL(KVC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return KVC_OK;
}

}  // namespace kvc

using namespace kvc;

extern "C" int kvc_version(void) { return 100; }   // 0.1.0

extern "C" const char* kvc_status_string(int status) {
  switch (status) {
    case KVC_OK: return "ok";
    case KVC_ERR_ARG: return "invalid argument";
    case KVC_ERR_DTYPE: return "unsupported dtype";
    case KVC_ERR_WORKSPACE: return "workspace missing or too small";
    case KVC_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

extern "C" const char* kvc_last_error(void) { return g_last_error; }

// [InfoKV] Contributions, Technical detail: the default budget keeps the same
// number of tokens in every layer.
extern "C" int kvc_uniform_budget(double keep_fraction, int64_t n, int w, int64_t* k_out) {
  clear_error();
  KVC_REQUIRE(k_out, "kvc_uniform_budget: null pointer");
  KVC_REQUIRE(n >= 1 && w >= 0 && w <= n, "kvc_uniform_budget: need n >= 1, 0 <= w <= n");
  KVC_REQUIRE(keep_fraction >= 0.0 && keep_fraction <= 1.0,
              "kvc_uniform_budget: keep_fraction outside [0, 1]");
  int64_t k = (int64_t)floor(keep_fraction * (double)n);
  if (k < w) k = w;
  if (k < 1) k = 1;
  if (k > n) k = n;
  *k_out = k;
  return KVC_OK;
}

// [InfoKV] Method; Glossary (adaptive budget allocation): the total budget B is
// split across layers in proportion to each layer's mean entropy score.
extern "C" int kvc_adaptive_budget(const float* Ebar, int L, int64_t B, int w, int64_t n,
                                   int64_t* k_out) {
  clear_error();
  KVC_REQUIRE(Ebar && k_out, "kvc_adaptive_budget: null pointer");
  KVC_REQUIRE(L >= 1 && L <= KVC_MAX_LAYERS, "kvc_adaptive_budget: need 1 <= L <= %d", KVC_MAX_LAYERS);
  KVC_REQUIRE(n >= 1 && w >= 0 && w <= n && B >= 0, "kvc_adaptive_budget: bad n, w or B");
  double sum = 0.0;
  for (int l = 0; l < L; ++l) {
    KVC_REQUIRE(Ebar[l] > 0.0f && isfinite(Ebar[l]), "kvc_adaptive_budget: Ebar[%d] not > 0", l);
    sum += (double)Ebar[l];
  }
  int64_t used = 0;
  for (int l = 0; l < L; ++l) {
    k_out[l] = (int64_t)floor((double)Ebar[l] / sum * (double)B);
    used += k_out[l];
  }
  int64_t left = B - used;
  for (int l = 0; l < L && left > 0; ++l, --left) k_out[l] += 1;
  for (int l = 0; l < L; ++l) {
    if (k_out[l] < w) k_out[l] = w;
    if (k_out[l] < 1) k_out[l] = 1;
    if (k_out[l] > n) k_out[l] = n;
  }
  return KVC_OK;
}
