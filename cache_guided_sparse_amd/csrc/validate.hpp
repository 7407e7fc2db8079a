// Opt-in checks of documented device-data preconditions (validate.hip).
// Each returns CGS_OK when checking is off or the data passes, CGS_ERR_DATA
// when it does not (after waiting for the check on the stream), or
// CGS_ERR_LAUNCH.
#pragma once

#include "common.hpp"

namespace cgs {

bool validate_on();
// idx[0..n) strictly ascending and in [0, limit).
int validate_index(const int32_t* idx, int n, int limit, hipStream_t s);
// a[0..n) finite with |a| <= bound (dtype CGS_BF16 or CGS_F32).
int validate_abs(const void* a, size_t n, int dtype, float bound, hipStream_t s);
// a[0..n) finite (and, with nonneg, not negative).
int validate_finite_f64(const double* a, int n, hipStream_t s, bool nonneg = false);

}  // namespace cgs
