// Status strings, thread-local error detail and launch profiling.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>
#include "common.hpp"

namespace moeq {

static thread_local char g_err[512] = "";

void set_error(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

moeq_status fail(moeq_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

moeq_status check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MOEQ_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return MOEQ_OK;
}

// ---- profiling: events recorded around launches when enabled.  Events
// come from a pool created up front so that recording costs one
// hipEventRecord per boundary.
struct ProfRec {
  const char *name;
  int a, b;   // pool indices
};
static bool g_prof = false;
static std::vector<hipEvent_t> g_pool;
static size_t g_used = 0;
static std::vector<ProfRec> g_recs;
static std::vector<int> g_pending;   // begin events waiting for their end

static int prof_event(hipStream_t s) {
  if (g_used == g_pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return -1;
    g_pool.push_back(e);
  }
  const int i = (int)g_used++;
  (void)hipEventRecord(g_pool[i], s);
  return i;
}

void prof_begin(const char *name, hipStream_t s) {
  (void)name;
  if (!g_prof) return;
  g_pending.push_back(prof_event(s));
}

void prof_end(const char *name, hipStream_t s) {
  if (!g_prof || g_pending.empty()) return;
  const int b = prof_event(s);
  const int a = g_pending.back();
  g_pending.pop_back();
  if (a >= 0 && b >= 0) g_recs.push_back(ProfRec{name, a, b});
}

static void prof_clear() {
  g_recs.clear();
  g_pending.clear();
  g_used = 0;
}

static void prof_reserve(size_t n) {
  while (g_pool.size() < n) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) break;
    g_pool.push_back(e);
  }
}

}  // namespace moeq

using namespace moeq;

MOEQ_API const char *moeq_status_string(moeq_status s) {
  switch (s) {
    case MOEQ_OK: return "MOEQ_OK";
    case MOEQ_ERR_INVALID: return "MOEQ_ERR_INVALID";
    case MOEQ_ERR_UNSUPPORTED: return "MOEQ_ERR_UNSUPPORTED";
    case MOEQ_ERR_WORKSPACE: return "MOEQ_ERR_WORKSPACE";
    case MOEQ_ERR_HIP: return "MOEQ_ERR_HIP";
  }
  return "MOEQ_ERR_UNKNOWN";
}

MOEQ_API const char *moeq_last_error(void) { return g_err; }

MOEQ_API int32_t moeq_abi_version(void) { return 1; }

MOEQ_API moeq_status moeq_profile_enable(int32_t on) {
  if (g_prof && !g_recs.empty()) {
    // events of the previous session may still be pending on a stream
    if (hipEventSynchronize(g_pool[g_recs.back().b]) != hipSuccess)
      return fail(MOEQ_ERR_HIP, "profile_enable: event sync failed");
  }
  prof_clear();
  g_prof = on != 0;
  if (g_prof) prof_reserve(4096);
  return MOEQ_OK;
}

MOEQ_API moeq_status moeq_profile_read(int32_t max_kernels, const char **names, int32_t *launches,
                                       double *total_ms, int32_t *n_kernels) {
  if (!n_kernels) return fail(MOEQ_ERR_INVALID, "profile_read: null n_kernels");
  std::vector<const char *> nm;
  std::vector<int32_t> cnt;
  std::vector<double> ms;
  for (auto &r : g_recs) {
    if (hipEventSynchronize(g_pool[r.b]) != hipSuccess) return fail(MOEQ_ERR_HIP, "profile_read: event sync failed");
    float t = 0.f;
    if (hipEventElapsedTime(&t, g_pool[r.a], g_pool[r.b]) != hipSuccess)
      return fail(MOEQ_ERR_HIP, "profile_read: elapsed time failed");
    size_t i = 0;
    for (; i < nm.size(); ++i) if (std::strcmp(nm[i], r.name) == 0) break;
    if (i == nm.size()) { nm.push_back(r.name); cnt.push_back(0); ms.push_back(0.0); }
    cnt[i] += 1;
    ms[i] += t;
  }
  *n_kernels = (int32_t)nm.size();
  for (int32_t i = 0; i < (int32_t)nm.size() && i < max_kernels; ++i) {
    if (names) names[i] = nm[i];
    if (launches) launches[i] = cnt[i];
    if (total_ms) total_ms[i] = ms[i];
  }
  return MOEQ_OK;
}
