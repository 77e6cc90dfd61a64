// Host part of the C ABI: thread-local error messages, shape checks, and the
// (host-side) preparation of the nearest-x2 phase weights.
#include <hip/hip_runtime.h>
#include <math.h>
#include <new>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "host.hpp"
#include "silugn.h"

namespace sgn {

static thread_local char g_error[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof g_error, fmt, ap);
  va_end(ap);
}

void clear_error() { g_error[0] = 0; }

bool dims_ok(sgn_dims d, const char* fn) {
  if (d.n <= 0 || d.t <= 0 || d.h <= 0 || d.w <= 0 || d.c <= 0) {
    set_error("%s: dims must be positive (n=%lld t=%lld h=%lld w=%lld c=%lld)", fn, (long long)d.n,
              (long long)d.t, (long long)d.h, (long long)d.w, (long long)d.c);
    return false;
  }
  if (d.c % 8 != 0) {
    set_error("%s: C=%lld must be a multiple of 8", fn, (long long)d.c);
    return false;
  }
  if (d.n > 65535 || d.t > (1 << 20) || d.h > 32767 || d.w > 32767 || d.c > 65536) {
    set_error("%s: dims out of the supported range", fn);
    return false;
  }
  const double elems = (double)d.n * d.t * d.h * d.w * d.c;
  if (elems > 4.0e12) {
    set_error("%s: tensor of %.3g elements is too large", fn, elems);
    return false;
  }
  return true;
}

bool launch_ok(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: launch failed: %s", what, hipGetErrorString(e));
    return false;
  }
  return true;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN -> quiet NaN).
static uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

}  // namespace sgn

using namespace sgn;

extern "C" const char* sgn_last_error(void) { return g_error; }

// Phase weights of nearest-x2 + 3x3 (binding.cpp page, prepare()): for output phase a
// along H, 3x3 row tap r lands on low-resolution row floor((a + r - 1) / 2) relative
// to the output's low-resolution row, i.e. phase tap u = floor((a + r - 1) / 2) - a + 1
// (a = 0: r 0 -> u 0, r 1,2 -> u 1; a = 1: r 0,1 -> u 0, r 2 -> u 1); the same for
// columns. The taps of a phase tap are summed in fp32 and rounded once to bf16.
extern "C" int upsample2x_prepare_weights(const uint16_t* w3x3, int k, int c, uint16_t* w_phase) {
  clear_error();
  if (!w3x3 || !w_phase || k <= 0 || c <= 0) {
    set_error("upsample2x_prepare_weights: w3x3, w_phase and positive k, c are required");
    return SGN_EINVAL;
  }
  const size_t in_bytes = (size_t)k * 9 * c * 2, out_bytes = (size_t)k * 16 * c * 2;
  if (overlap(w3x3, in_bytes, w_phase, out_bytes)) {
    set_error("upsample2x_prepare_weights: w_phase overlaps w3x3");
    return SGN_EALIAS;
  }
  // tap_of[a][r]: phase tap (0/1) that 3x3 tap r feeds for output phase a.
  int tap_of[2][3];
  for (int a = 0; a < 2; ++a)
    for (int r = 0; r < 3; ++r) {
      const int num = a + r - 1;
      const int fl = num < 0 ? -1 : num / 2;
      tap_of[a][r] = fl - a + 1;
    }
  float* acc = new (std::nothrow) float[(size_t)c];
  if (!acc) {
    set_error("upsample2x_prepare_weights: cannot allocate %d floats of host memory", c);
    return SGN_EINVAL;
  }
  for (int a = 0; a < 2; ++a)
    for (int b = 0; b < 2; ++b)
      for (int kk = 0; kk < k; ++kk)
        for (int u = 0; u < 2; ++u)
          for (int v = 0; v < 2; ++v) {
            for (int ci = 0; ci < c; ++ci) acc[ci] = 0.0f;
            for (int r = 0; r < 3; ++r) {
              if (tap_of[a][r] != u) continue;
              for (int s = 0; s < 3; ++s) {
                if (tap_of[b][s] != v) continue;
                const uint16_t* src = w3x3 + (((size_t)kk * 3 + r) * 3 + s) * c;
                for (int ci = 0; ci < c; ++ci) acc[ci] += bf16_to_f32(src[ci]);
              }
            }
            uint16_t* dst = w_phase + ((((size_t)(a * 2 + b) * k + kk) * 2 + u) * 2 + v) * c;
            for (int ci = 0; ci < c; ++ci) dst[ci] = f32_to_bf16(acc[ci]);
          }
  delete[] acc;
  return SGN_OK;
}

// Winograd F(4x4,3x3) weights (binding.cpp page, prepare(): the 6x3 matrix G; each of the 36
// components keeps the 3 frame taps; sums formed in fp32, stored in bf16):
//   u[a * 6 + b][k][dt][c] = RNE_bf16( fp32 sum over the taps (r, s) with G[a][r] G[b][s] != 0
//                                      of w[k][dt][r][s][c] * (G[a][r] G[b][s]) ).
extern "C" int winograd_prepare_weights(const uint16_t* w, int k, int c, uint16_t* u) {
  clear_error();
  if (!w || !u || k <= 0 || c <= 0) {
    set_error("winograd_prepare_weights: w, u and positive k, c are required");
    return SGN_EINVAL;
  }
  const size_t in_bytes = (size_t)k * 27 * c * 2, out_bytes = (size_t)36 * k * 3 * c * 2;
  if (overlap(w, in_bytes, u, out_bytes)) {
    set_error("winograd_prepare_weights: u overlaps w");
    return SGN_EALIAS;
  }
  static const float G[6][3] = {{0.25f, 0.0f, 0.0f},
                                {-1.0f / 6, -1.0f / 6, -1.0f / 6},
                                {-1.0f / 6, 1.0f / 6, -1.0f / 6},
                                {1.0f / 24, 1.0f / 12, 1.0f / 6},
                                {1.0f / 24, -1.0f / 12, 1.0f / 6},
                                {0.0f, 0.0f, 1.0f}};
  float* acc = new (std::nothrow) float[(size_t)c];
  if (!acc) {
    set_error("winograd_prepare_weights: cannot allocate %d floats of host memory", c);
    return SGN_EINVAL;
  }
  for (int a = 0; a < 6; ++a)
    for (int b = 0; b < 6; ++b)
      for (int kk = 0; kk < k; ++kk)
        for (int dt = 0; dt < 3; ++dt) {
          for (int ci = 0; ci < c; ++ci) acc[ci] = 0.0f;
          for (int r = 0; r < 3; ++r)
            for (int s = 0; s < 3; ++s) {
              const float coef = G[a][r] * G[b][s];
              if (coef == 0.0f) continue;
              const uint16_t* src = w + ((((size_t)kk * 3 + dt) * 3 + r) * 3 + s) * c;
              for (int ci = 0; ci < c; ++ci) acc[ci] += bf16_to_f32(src[ci]) * coef;
            }
          uint16_t* dst = u + (((size_t)(a * 6 + b) * k + kk) * 3 + dt) * c;
          for (int ci = 0; ci < c; ++ci) dst[ci] = f32_to_bf16(acc[ci]);
        }
  delete[] acc;
  return SGN_OK;
}
