// Ceiling probes for the benchmark (libsgnprobe.so, separate from the C ABI in libsilugn.so):
// what this GPU sustains for the two resources the hot path is bound by.
// - bf16 MFMA: v_mfma_f32_32x32x16_bf16 back to back, 16 accumulators per wave, operands
//   re-read from LDS every 16 MFMAs (as in the convolution's inner loop), with random or
//   constant operand bits. The rate with random bits is the one real data sees: MFMA power
//   grows with operand toggling and the clock drops to hold the board's power limit.
// - HBM: a streaming read (16-byte non-temporal loads, xor-reduced) and a streaming copy.
// Built by silu_gn_amd/build.py into bench_probe/libsgnprobe.so; only bench.py loads it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

template <bool RANDOM>
__global__ __launch_bounds__(256) void mfma_probe(float* out, int iters) {
  __shared__ __attribute__((aligned(16))) char buf[32768];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 32768 / 16; i += 256) {
    unsigned h = (unsigned)(i + blockIdx.x * 7919) * 2654435761u;
    h ^= h >> 15;
    h *= 2246822519u;
    h ^= h >> 13;
    // bf16 pairs near +-1 with random mantissas and signs, or all 1.0
    const unsigned a = RANDOM ? ((h & 0x807f807fu) | 0x3f003f00u) : 0x3f803f80u;
    const unsigned b = RANDOM ? (((h * 3u) & 0x807f807fu) | 0x3f003f00u) : 0x3f803f80u;
    reinterpret_cast<u32x4*>(buf)[i] = u32x4{a, b, a ^ 0x00010001u, b ^ 0x00020002u};
  }
  __syncthreads();
  f32x16 acc[4][4];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j)
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  bf16x8 a[2][4], b[2][4];
  for (int i = 0; i < 4; ++i) {
    a[0][i] = *reinterpret_cast<const bf16x8*>(buf + i * 1024 + lane * 16);
    b[0][i] = *reinterpret_cast<const bf16x8*>(buf + 4096 + i * 1024 + lane * 16);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
      const int cur = ph, nxt = ph ^ 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[nxt][i] = *reinterpret_cast<const bf16x8*>(buf + ((wave * 8 + i + it + ph) & 31) * 1024 + lane * 16);
        b[nxt][i] = *reinterpret_cast<const bf16x8*>(buf + ((wave * 8 + 4 + i + 3 * it + ph) & 31) * 1024 + lane * 16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][i], b[cur][j], acc[i][j], 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float s = 0;
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j)
      for (int r = 0; r < 16; ++r) s += acc[i][j][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Each workgroup streams one contiguous slice (as the GroupNorm kernels do: whole DRAM
// pages per workgroup), 8 packets in flight per thread.
constexpr int kU = 8;

__global__ __launch_bounds__(256) void read_probe(const u32x4* src, size_t n, u32x4* out) {
  const size_t per = (n + gridDim.x - 1) / gridDim.x;
  const size_t beg = (size_t)blockIdx.x * per, end = beg + per < n ? beg + per : n;
  u32x4 acc = {0, 0, 0, 0};
  size_t i = beg + threadIdx.x;
  for (; i + (kU - 1) * 256 < end; i += kU * 256) {
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < kU; ++u) acc ^= v[u];
  }
  for (; i < end; i += 256) acc ^= __builtin_nontemporal_load(src + i);
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// The copy sweeps grid-wide (pass k of workgroup b covers packets (k * grid + b) * 1024 ..
// + 1023, 4 in flight per thread), as the GroupNorm apply does: with whole slices per
// workgroup the copy ran at about 4.9 TB/s, swept at about 5.7.
constexpr int kCopyU = 4;
constexpr int kCopyBlocks = 8192;
__global__ __launch_bounds__(256) void copy_probe(const u32x4* src, u32x4* dst, size_t n) {
  const size_t step = (size_t)gridDim.x * 256 * kCopyU;
  for (size_t base = (size_t)blockIdx.x * 256 * kCopyU; base < n; base += step) {
    u32x4 v[kCopyU];
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
      const size_t i = base + u * 256 + threadIdx.x;
      if (i < n) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
      const size_t i = base + u * 256 + threadIdx.x;
      if (i < n) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

constexpr int kProbeBlocks = 1792;   // 7 per CU on 256 CUs: one round

}  // namespace

// MFMA probe: `blocks` workgroups of 4 waves, `iters` x 32 MFMAs per wave; out holds
// blocks x 256 floats. FLOPs = 2 * 32 * 32 * 16 * 32 * 4 * blocks * iters.
extern "C" int sgn_probe_mfma(float* out, int blocks, int iters, int random_operands, hipStream_t s) {
  if (!out || blocks <= 0 || iters <= 0) return -1;
  if (random_operands)
    mfma_probe<true><<<blocks, 256, 0, s>>>(out, iters);
  else
    mfma_probe<false><<<blocks, 256, 0, s>>>(out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Streaming read of `bytes` (a multiple of 16) from src; out holds 2048 x 256 x 16 bytes.
extern "C" int sgn_probe_read(const void* src, size_t bytes, void* out, hipStream_t s) {
  if (!src || !out || bytes % 16) return -1;
  read_probe<<<kProbeBlocks, 256, 0, s>>>(static_cast<const u32x4*>(src), bytes / 16, static_cast<u32x4*>(out));
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Streaming copy of `bytes` (a multiple of 16) from src to dst (non-overlapping).
extern "C" int sgn_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  if (!src || !dst || bytes % 16) return -1;
  copy_probe<<<kCopyBlocks, 256, 0, s>>>(static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
