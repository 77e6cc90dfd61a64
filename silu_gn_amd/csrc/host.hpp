// Host-side argument checks and error reporting shared by the C entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "silugn.h"

namespace sgn {

void set_error(const char* fmt, ...);
void clear_error();

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Byte ranges [a, a+na) and [b, b+nb) intersect.
inline bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

// Positive dims, C % 8 == 0, and an element count that fits int64 comfortably.
bool dims_ok(sgn_dims d, const char* fn);

// Checks hipGetLastError after a launch; records the HIP message on failure.
bool launch_ok(const char* what);

// GroupNorm statistics from per-block partial sums (gn.hip): ws holds, for every sample n
// and group g, nblk sums S then nblk sums Q at ws[((n * groups + g) * 2) * nblk]; stats
// receives mean = S / length and the biased variance Q / length - mean^2 per (n, g).
bool launch_gn_finalize(const double* ws, int nblk, int groups, int64_t n, double length,
                        double* stats, hipStream_t stream);

}  // namespace sgn
