// GroupNorm + SiLU on channels-last bf16 activations (gfx950).
//
// Statistics (gn_silu_stats): one read of x in 16-byte packets. Each thread keeps a
// fixed packet column (8 channels) and walks positions, accumulating every value and
// its exact square in fp64 (one add and one fma per value).
// Threads of a block are combined through LDS in a fixed order into one fp64
// partial per (block, group); a second kernel sums the partials of each group in a
// fixed order and forms mean = S/L and the biased variance Q/L - mean^2. The same
// inputs and launch always give the same bits.
//
// Apply (gn_silu_apply): one read and one write; each thread forms the fp64 affine of
// its 8 channels once and then streams packets through activate_packet().
//
// Pages: WanGP group_norm_silu.py (module docstring: exact partial sums reduced in
// fp64 in a fixed order, one rounding to the output dtype; its apply kernel: biased
// variance, rstd = 1/sqrt(var + eps), y * sigmoid(y)). The pages' second, centred pass
// over x is replaced by the fp64 sum of exact squares, which saves one full read.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "common.hpp"
#include "silugn.h"
#include "host.hpp"

namespace sgn {

constexpr int kThreads = 256;
constexpr int kMaxStatBlocks = 2048;  // partial-sum blocks over the whole grid (workspace bound)

// x and y are streamed once per pass: loads and stores are non-temporal (they do not
// displace what other work keeps in the caches). Measured on MI355X at the full-resolution
// shape: statistics 5.7 -> 6.5 TB/s with non-temporal loads, 4 packets in flight per thread;
// apply 4.8 -> 5.0 TB/s with 8 packets in flight.
constexpr int kStatsUnroll = 4;
constexpr int kApplyUnroll = 8;

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store_stream(uint4* p, uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

// Packet decomposition shared by the stats and apply kernels: Cp packets per
// position; ncol = Cp threads form one position row, rstep rows per pass.
struct PacketGrid {
  int cp;         // packets per position (C / 8), <= 256
  int rstep;      // rows (positions) covered by one pass of the block
  int active;     // rstep * cp threads of the block take part
  int64_t rows_per_block;
  int blocks;     // blocks per sample
};

static PacketGrid packet_grid(int64_t positions, int c, int n, int min_iters, int max_blocks) {
  PacketGrid g;
  g.cp = c / 8;
  g.rstep = kThreads / g.cp;
  g.active = g.rstep * g.cp;
  int64_t want = max_blocks / (n > 0 ? n : 1);
  if (want < 1) want = 1;
  int64_t cap = (positions + (int64_t)g.rstep * min_iters - 1) / ((int64_t)g.rstep * min_iters);
  if (cap < 1) cap = 1;
  int64_t blocks = want < cap ? want : cap;
  int64_t rows = (positions + blocks - 1) / blocks;
  rows = (rows + g.rstep - 1) / g.rstep * g.rstep;     // whole passes per block
  g.rows_per_block = rows;
  g.blocks = (int)((positions + rows - 1) / rows);
  return g;
}

// Workgroups of kThreads that the device holds at once for `kernel` (all CUs at full
// occupancy), at most kMaxStatBlocks: a grid of that many runs in one round, with no tail
// of late workgroups on a mostly idle chip. Cached per device and kernel.
static int resident_blocks(const void* kernel) {
  struct Entry {
    int dev;
    const void* fn;
    int blocks;
  };
  static thread_local Entry cache[16];
  static thread_local int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return kMaxStatBlocks;
  for (int i = 0; i < used; ++i)
    if (cache[i].dev == dev && cache[i].fn == kernel) return cache[i].blocks;
  int cus = 0, per_cu = 0;
  int blocks = kMaxStatBlocks;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) == hipSuccess &&
      cus > 0 && per_cu > 0)
    blocks = cus * per_cu < kMaxStatBlocks ? cus * per_cu : kMaxStatBlocks;
  if (used < 16) cache[used++] = Entry{dev, kernel, blocks};
  return blocks;
}

// Adds the two bf16 values of dword i of a packet to their groups' fp64 sums: x is exact
// in fp64 and x*x (16 significant bits) is exact inside the fma, so each value costs one
// rounding of a running fp64 sum and one of a running fp64 sum of squares.
template <int GPP>
__device__ __forceinline__ void accumulate(uint32_t d, int i, double* s, double* q) {
  const double a = (double)bf16_lo(d), b = (double)bf16_hi(d);
  const int sa = (GPP == 1) ? 0 : (GPP == 2) ? (i >> 1) : (GPP == 4) ? i : 2 * i;
  const int sb = (GPP == 8) ? sa + 1 : sa;
  s[sa] += a;
  q[sa] = fma(a, a, q[sa]);
  s[sb] += b;
  q[sb] = fma(b, b, q[sb]);
}

// GPP = groups inside one packet (1 when C/G >= 8, else 8 / (C/G)).
template <int GPP>
__global__ __launch_bounds__(kThreads) void gn_stats_partial(const uint4* __restrict__ x,
                                                             int64_t positions, int cp, int rstep,
                                                             int64_t rows_per_block, int cg,
                                                             int groups, double* __restrict__ ws) {
  __shared__ double red[kThreads][GPP][2];
  const int tid = threadIdx.x;
  const int blk = blockIdx.x, nblk = gridDim.x, n = blockIdx.y;
  const int active = rstep * cp;
  const int col = tid % cp;
  const int row0 = tid / cp;
  double s[GPP], q[GPP];
#pragma unroll
  for (int i = 0; i < GPP; ++i) s[i] = q[i] = 0.0;

  if (tid < active) {
    const int64_t start = (int64_t)blk * rows_per_block;
    int64_t end = start + rows_per_block;
    if (end > positions) end = positions;
    const uint4* base = x + (int64_t)n * positions * cp + col;
    constexpr int U = kStatsUnroll;
    int64_t p = start + row0;
    for (; p + (U - 1) * rstep < end; p += U * rstep) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = load_stream(base + (p + u * rstep) * cp);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t d[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) accumulate<GPP>(d[i], i, s, q);
      }
    }
    for (; p < end; p += rstep) {
      const uint4 v = load_stream(base + p * cp);
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) accumulate<GPP>(d[i], i, s, q);
    }
  }
#pragma unroll
  for (int i = 0; i < GPP; ++i) {
    red[tid][i][0] = s[i];
    red[tid][i][1] = q[i];
  }
  __syncthreads();
  // One thread per group adds its contributors in a fixed order: rows, then columns.
  const int pk_per_group = (GPP == 1) ? cg / 8 : 1;
  for (int g = tid; g < groups; g += kThreads) {
    const int col0 = (GPP == 1) ? g * pk_per_group : (g * cg) / 8;
    const int slot = (GPP == 1) ? 0 : g - col0 * GPP;
    double S = 0.0, Q = 0.0;
    for (int r = 0; r < rstep; ++r)
      for (int k = 0; k < pk_per_group; ++k) {
        const int t = r * cp + col0 + k;
        S += red[t][slot][0];
        Q += red[t][slot][1];
      }
    double* o = ws + (((int64_t)n * groups + g) * 2) * nblk;
    o[blk] = S;
    o[nblk + blk] = Q;
  }
}

// One block per (group, sample): fixed-order sum of the block partials.
__global__ __launch_bounds__(kThreads) void gn_stats_finalize(const double* __restrict__ ws,
                                                              int nblk, int groups, double length,
                                                              double* __restrict__ stats) {
  __shared__ double rs[kThreads], rq[kThreads];
  const int g = blockIdx.x, n = blockIdx.y, tid = threadIdx.x;
  const double* src = ws + (((int64_t)n * groups + g) * 2) * nblk;
  double S = 0.0, Q = 0.0;
  for (int b = tid; b < nblk; b += kThreads) {
    S += src[b];
    Q += src[nblk + b];
  }
  rs[tid] = S;
  rq[tid] = Q;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) {
      rs[tid] += rs[tid + w];
      rq[tid] += rq[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double mean = rs[0] / length;
    double var = rq[0] / length - mean * mean;
    if (var < 0.0) var = 0.0;
    stats[((int64_t)n * groups + g) * 2 + 0] = mean;
    stats[((int64_t)n * groups + g) * 2 + 1] = var;
  }
}

// y = silu(group_norm(x)) -- same packet decomposition as the statistics.
__global__ __launch_bounds__(kThreads) void gn_apply_kernel(
    const uint4* x, uint4* y, int64_t positions, int cp, int rstep,
    int64_t rows_per_block, const double* __restrict__ stats, const float* __restrict__ gamma,
    const float* __restrict__ beta, double eps, int groups, int cg) {
  const int tid = threadIdx.x;
  const int n = blockIdx.y;
  const int active = rstep * cp;
  if (tid >= active) return;
  const int col = tid % cp;
  Affine a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = channel_affine(stats, gamma, beta, eps, groups, cg, n, col * 8 + i);
  const int64_t start = (int64_t)blockIdx.x * rows_per_block;
  int64_t end = start + rows_per_block;
  if (end > positions) end = positions;
  const int64_t off = (int64_t)n * positions * cp + col;
  const uint4* src = x + off;
  uint4* dst = y + off;
  constexpr int U = kApplyUnroll;
  int64_t p = start + tid / cp;
  for (; p + (U - 1) * rstep < end; p += U * rstep) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = load_stream(src + (p + u * rstep) * cp);
#pragma unroll
    for (int u = 0; u < U; ++u) store_stream(dst + (p + u * rstep) * cp, activate_packet(v[u], a));
  }
  for (; p < end; p += rstep) store_stream(dst + p * cp, activate_packet(load_stream(src + p * cp), a));
}

static bool gn_shape_ok(sgn_dims d, int groups, const char* fn) {
  if (!dims_ok(d, fn)) return false;
  if (groups <= 0 || d.c % groups != 0) {
    set_error("%s: groups=%d must divide C=%lld", fn, groups, (long long)d.c);
    return false;
  }
  const int64_t cg = d.c / groups;
  if (!(cg == 1 || cg == 2 || cg == 4 || cg % 8 == 0)) {
    set_error("%s: C/groups=%lld must be 1, 2, 4 or a multiple of 8", fn, (long long)cg);
    return false;
  }
  if (d.c > 2048) {
    set_error("%s: C=%lld exceeds 2048", fn, (long long)d.c);
    return false;
  }
  return true;
}

}  // namespace sgn

using namespace sgn;

extern "C" size_t gn_silu_stats_workspace(sgn_dims d, int groups) {
  if (!gn_shape_ok(d, groups, "gn_silu_stats_workspace")) return 0;
  const int64_t positions = d.t * d.h * d.w;
  PacketGrid g = packet_grid(positions, (int)d.c, (int)d.n, 8, kMaxStatBlocks);
  return (size_t)d.n * groups * 2 * g.blocks * sizeof(double);
}

extern "C" int gn_silu_stats(const uint16_t* x, sgn_dims d, int groups, double* stats, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (!gn_shape_ok(d, groups, "gn_silu_stats")) return SGN_EINVAL;
  if (!x || !stats) {
    set_error("gn_silu_stats: x and stats are required");
    return SGN_EINVAL;
  }
  if (!aligned16(x) || ((uintptr_t)stats & 7)) {
    set_error("gn_silu_stats: x must be 16-byte and stats 8-byte aligned");
    return SGN_EALIGN;
  }
  const int64_t positions = d.t * d.h * d.w;
  const int cg = (int)(d.c / groups);
  const int gpp = cg >= 8 ? 1 : 8 / cg;
  const void* partial = gpp == 1   ? (const void*)gn_stats_partial<1>
                        : gpp == 2 ? (const void*)gn_stats_partial<2>
                        : gpp == 4 ? (const void*)gn_stats_partial<4>
                                   : (const void*)gn_stats_partial<8>;
  PacketGrid g = packet_grid(positions, (int)d.c, (int)d.n, 8, resident_blocks(partial));
  const size_t need = (size_t)d.n * groups * 2 * g.blocks * sizeof(double);
  if (!ws || ws_bytes < need) {
    set_error("gn_silu_stats: workspace of %zu bytes required, got %zu", need, ws ? ws_bytes : 0);
    return SGN_EWORKSPACE;
  }
  if (!aligned16(ws)) {
    set_error("gn_silu_stats: workspace must be 16-byte aligned");
    return SGN_EALIGN;
  }
  dim3 grid(g.blocks, (unsigned)d.n);
  const uint4* xp = reinterpret_cast<const uint4*>(x);
  double* w = static_cast<double*>(ws);
  switch (gpp) {
    case 1: gn_stats_partial<1><<<grid, kThreads, 0, stream>>>(xp, positions, g.cp, g.rstep, g.rows_per_block, cg, groups, w); break;
    case 2: gn_stats_partial<2><<<grid, kThreads, 0, stream>>>(xp, positions, g.cp, g.rstep, g.rows_per_block, cg, groups, w); break;
    case 4: gn_stats_partial<4><<<grid, kThreads, 0, stream>>>(xp, positions, g.cp, g.rstep, g.rows_per_block, cg, groups, w); break;
    default: gn_stats_partial<8><<<grid, kThreads, 0, stream>>>(xp, positions, g.cp, g.rstep, g.rows_per_block, cg, groups, w); break;
  }
  if (!launch_ok("gn_silu_stats (partial)")) return SGN_ELAUNCH;
  const double length = (double)positions * cg;
  gn_stats_finalize<<<dim3(groups, (unsigned)d.n), kThreads, 0, stream>>>(w, g.blocks, groups, length, stats);
  if (!launch_ok("gn_silu_stats (finalize)")) return SGN_ELAUNCH;
  return SGN_OK;
}

bool sgn::launch_gn_finalize(const double* ws, int nblk, int groups, int64_t n, double length,
                        double* stats, hipStream_t stream) {
  gn_stats_finalize<<<dim3(groups, (unsigned)n), kThreads, 0, stream>>>(ws, nblk, groups, length, stats);
  return launch_ok("GroupNorm statistics (finalize)");
}

extern "C" int gn_silu_apply(const uint16_t* x, sgn_dims d, int groups, const double* stats,
                             const float* gamma, const float* beta, float eps, uint16_t* y,
                             hipStream_t stream) {
  clear_error();
  if (!gn_shape_ok(d, groups, "gn_silu_apply")) return SGN_EINVAL;
  if (!x || !stats || !gamma || !beta || !y) {
    set_error("gn_silu_apply: x, stats, gamma, beta and y are required");
    return SGN_EINVAL;
  }
  if (!(eps > 0.0f) || !isfinite(eps)) {
    set_error("gn_silu_apply: eps must be a positive finite number");
    return SGN_EINVAL;
  }
  if (!aligned16(x) || !aligned16(y) || ((uintptr_t)stats & 7) || ((uintptr_t)gamma & 3) ||
      ((uintptr_t)beta & 3)) {
    set_error("gn_silu_apply: x, y must be 16-byte aligned (stats 8, gamma/beta 4)");
    return SGN_EALIGN;
  }
  const size_t bytes = (size_t)(d.n * d.t * d.h * d.w * d.c) * 2;
  if ((const void*)x != (const void*)y && overlap(x, bytes, y, bytes)) {
    set_error("gn_silu_apply: y partially overlaps x (only y == x is allowed)");
    return SGN_EALIAS;
  }
  const int64_t positions = d.t * d.h * d.w;
  PacketGrid g = packet_grid(positions, (int)d.c, (int)d.n, 4, resident_blocks((const void*)gn_apply_kernel));
  const int cg = (int)(d.c / groups);
  gn_apply_kernel<<<dim3(g.blocks, (unsigned)d.n), kThreads, 0, stream>>>(
      reinterpret_cast<const uint4*>(x), reinterpret_cast<uint4*>(y), positions, g.cp, g.rstep,
      g.rows_per_block, stats, gamma, beta, (double)eps, groups, cg);
  if (!launch_ok("gn_silu_apply")) return SGN_ELAUNCH;
  return SGN_OK;
}
