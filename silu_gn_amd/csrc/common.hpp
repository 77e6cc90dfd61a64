// Device helpers shared by the GroupNorm and convolution kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgn {

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// bf16 halves of a packed dword -> exact fp32.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Two fp32 -> packed bf16x2, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// silu(z) = z / (1 + e^-z) in fp32 for z >= -80 (e^-z stays finite): hardware
// exp2 and reciprocal, each within 1 ulp, so the result is within a few fp32
// ulps -- far inside the half bf16 ulp that the single output rounding allows.
__device__ __forceinline__ float silu_fast(float z) {
  const float kNegLog2e = -1.4426950408889634f;
  float t = __builtin_amdgcn_exp2f(z * kNegLog2e);
  return z * __builtin_amdgcn_rcpf(1.0f + t);
}

// silu for any finite z: with t = e^-|z| in (0, 1] nothing overflows;
// z * t / (1 + t) for z < 0, z / (1 + t) otherwise; library exp and IEEE division.
__device__ __noinline__ float silu_precise(float z) {
  float t = expf(-fabsf(z));
  float num = z >= 0.0f ? z : z * t;
  return num / (1.0f + t);
}

// Per-channel affine of GroupNorm in fp64: z = x * s + b with
// s = gamma / sqrt(var + eps) and b = beta - mean * s.
struct Affine {
  double s, b;
};

__device__ __forceinline__ Affine channel_affine(const double* stats, const float* gamma,
                                                 const float* beta, double eps, int groups,
                                                 int cg, int n, int c) {
  const double mean = stats[((int64_t)n * groups + c / cg) * 2 + 0];
  const double var = stats[((int64_t)n * groups + c / cg) * 2 + 1];
  const double s = (double)gamma[c] / sqrt(var + eps);
  Affine a;
  a.s = s;
  a.b = fma(-mean, s, (double)beta[c]);
  return a;
}

// silu(group_norm) of one 16-byte packet (8 channels) with the channels' affines.
// The pre-activation is formed in fp64 (x is exact in fp64; one fma), rounded
// to fp32, activated in fp32 and rounded once to bf16. Lanes holding a very
// negative pre-activation take the overflow-free path.
__device__ __forceinline__ uint4 activate_packet(uint4 v, const Affine* a) {
  float z[8];
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    z[2 * i] = (float)fma((double)bf16_lo(d[i]), a[2 * i].s, a[2 * i].b);
    z[2 * i + 1] = (float)fma((double)bf16_hi(d[i]), a[2 * i + 1].s, a[2 * i + 1].b);
  }
  float lo = z[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) lo = fminf(lo, z[i]);
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = silu_fast(z[i]);
  if (__builtin_expect(lo < -80.0f, 0)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = silu_precise(z[i]);
  }
  uint4 r;
  r.x = pack_bf16x2(o[0], o[1]);
  r.y = pack_bf16x2(o[2], o[3]);
  r.z = pack_bf16x2(o[4], o[5]);
  r.w = pack_bf16x2(o[6], o[7]);
  return r;
}

// Thread-local error state of the host API.
void set_error(const char* fmt, ...);

}  // namespace sgn
