// Optional per-kernel timing with HIP events (used by benchmarks).
//
// While a profile is active, every launch whose site name contains the filter
// string is bracketed by two events recorded on its own stream (unless the
// stream is being captured); the result query waits for them and sums the
// elapsed times.  Inactive: one branch per launch.  Not thread-safe: start,
// launch and query from one host thread.
#pragma once

#include <hip/hip_runtime.h>

namespace cgs {

void prof_begin(const char* site, hipStream_t s);
void prof_end(const char* site, hipStream_t s);

// Brackets the launches in its scope.
struct ProfScope {
  const char* site;
  hipStream_t stream;
  ProfScope(const char* n, hipStream_t s) : site(n), stream(s) { prof_begin(site, stream); }
  ~ProfScope() { prof_end(site, stream); }
};

}  // namespace cgs
