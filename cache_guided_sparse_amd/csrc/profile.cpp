// Event-based kernel timing behind cgs_profile_start / cgs_profile_result.
#include "profile.hpp"

#include <string.h>

#include <string>
#include <vector>

#include "../../include/cgs.h"

namespace cgs {
namespace {

struct Profile {
  bool active = false;
  std::string filter;
  std::vector<hipEvent_t> ev;  // pairs: start, stop
  std::vector<const char*> site;  // site of each pair (static strings)
  size_t used = 0;             // events recorded
  bool overflow = false;
  bool open = false;           // a start event waits for its stop
};

Profile g_prof;

bool matches(const char* site) {
  return g_prof.active && strstr(site, g_prof.filter.c_str()) != nullptr;
}

}  // namespace

void prof_begin(const char* site, hipStream_t s) {
  if (!matches(site)) return;
  // a launch being captured into a graph is not timed (no event enters the graph)
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
  if (g_prof.used + 2 > g_prof.ev.size()) { g_prof.overflow = true; return; }
  hipEventRecord(g_prof.ev[g_prof.used], s);
  g_prof.site[g_prof.used / 2] = site;
  g_prof.open = true;
}

void prof_end(const char* site, hipStream_t s) {
  if (!matches(site) || !g_prof.open) return;
  hipEventRecord(g_prof.ev[g_prof.used + 1], s);
  g_prof.used += 2;
  g_prof.open = false;
}

}  // namespace cgs

using cgs::g_prof;

extern "C" int cgs_profile_start(const char* site_filter, int max_launches) {
  if (!site_filter || max_launches <= 0) return CGS_ERR_ARG;
  for (hipEvent_t e : g_prof.ev) hipEventDestroy(e);
  g_prof = cgs::Profile{};
  g_prof.ev.resize(2 * static_cast<size_t>(max_launches));
  g_prof.site.resize(static_cast<size_t>(max_launches));
  for (auto& e : g_prof.ev)
    if (hipEventCreate(&e) != hipSuccess) return CGS_ERR_LAUNCH;
  g_prof.filter = site_filter;
  g_prof.active = true;
  return CGS_OK;
}

extern "C" int cgs_profile_stop(void) {
  g_prof.active = false;
  return CGS_OK;
}

extern "C" int cgs_profile_result(const char* site, double* total_ms, int* launches) {
  if (!total_ms || !launches) return CGS_ERR_ARG;
  double t = 0.0;
  int n = 0;
  for (size_t i = 0; i + 1 < g_prof.used; i += 2) {
    if (site && strstr(g_prof.site[i / 2], site) == nullptr) continue;
    if (hipEventSynchronize(g_prof.ev[i + 1]) != hipSuccess) return CGS_ERR_LAUNCH;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_prof.ev[i], g_prof.ev[i + 1]) != hipSuccess) return CGS_ERR_LAUNCH;
    t += ms;
    ++n;
  }
  *total_ms = t;
  *launches = n;
  return g_prof.overflow ? CGS_ERR_SHAPE : CGS_OK;
}
