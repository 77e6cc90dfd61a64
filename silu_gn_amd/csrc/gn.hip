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
// RMS norm + SiLU (rms_silu): the decoder's per-position norm, one read and one write,
// the same activate_packet() with the affine gain * rstd; rms_silu_rstd runs the same
// kernel writing each position's rstd instead (for a convolution that applies the norm in
// its operand load).
//
// Pages: WanGP group_norm_silu.py (module docstring: exact partial sums reduced in
// fp64 in a fixed order, one rounding to the output dtype; its apply kernel: biased
// variance, rstd = 1/sqrt(var + eps), y * sigmoid(y)). The pages' second, centred pass
// over x is replaced by the fp64 sum of exact squares, which saves one full read.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "common.hpp"
#include "silugn.h"
#include "host.hpp"

namespace sgn {

constexpr int kThreads = 256;
constexpr int kMaxStatBlocks = 2048;  // partial-sum blocks over the whole grid (workspace bound)

// x and y are streamed once per pass: loads and stores are non-temporal (they do not
// displace what other work keeps in the caches). Measured on MI355X at the full-resolution
// shape: statistics 5.7 -> 6.5 TB/s with non-temporal loads, 4 packets in flight per thread,
// each workgroup reading its own contiguous range of positions (a grid-wide sweep, as the
// apply's, read at 6.0 TB/s); apply 4.8 -> 5.0 TB/s with 8 packets in flight over contiguous
// ranges, 5.7 TB/s with 4 in flight in a grid-wide sweep of 8192 workgroups.
constexpr int kStatsUnroll = 4;
constexpr int kApplyUnroll = 4;
constexpr int kApplyBlocks = 8192;     // workgroups of the apply's grid-wide sweep (over all samples)

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

// y = silu(group_norm(x)) -- the packet decomposition of the statistics (thread = a fixed
// packet column, rstep position rows per pass of the block), swept grid-wide: pass k of block b
// covers rows (k * grid + b) * rstep * U .. + rstep * U - 1, so that all workgroups advance
// through x and y together (measured at the full-resolution shape: 0.72 ms with a contiguous
// range of rows per workgroup, against about 0.63 ms for an interleaved copy sweep).
__global__ __launch_bounds__(kThreads) void gn_apply_kernel(
    const uint4* x, uint4* y, int64_t positions, int cp, int rstep, const double* __restrict__ stats,
    const float* __restrict__ gamma, const float* __restrict__ beta, double eps, int groups, int cg) {
  const int tid = threadIdx.x;
  const int n = blockIdx.y;
  const int active = rstep * cp;
  if (tid >= active) return;
  const int col = tid % cp;
  const int row0 = tid / cp;
  Affine a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = channel_affine(stats, gamma, beta, eps, groups, cg, n, col * 8 + i);
  const int64_t off = (int64_t)n * positions * cp + col;
  const uint4* src = x + off;
  uint4* dst = y + off;
  constexpr int U = kApplyUnroll;
  const int64_t chunk = (int64_t)rstep * U;
  for (int64_t r0 = (int64_t)blockIdx.x * chunk; r0 < positions; r0 += (int64_t)gridDim.x * chunk) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t p = r0 + u * rstep + row0;
      if (p < positions) v[u] = load_stream(src + p * cp);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t p = r0 + u * rstep + row0;
      if (p < positions) store_stream(dst + p * cp, activate_packet(v[u], a));
    }
  }
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


// ---------------------------------------------------------------- RMS norm + SiLU
// Per position (no statistics across positions): z = x * gain / sqrt(mean_c x^2 + eps),
// out = RNE_bf16(z * sigmoid(z)). LPP lanes (a power of two, >= C/8 up to 64) share one
// position, each holding PPL packets of 8 channels (lanes past C/8 hold none); a wave covers
// 64 / LPP positions, U groups of them per iteration (U x PPL packets in flight per lane).
// Each lane sums the exact squares of its values in fp64 (x*x has 16 significant bits) and
// the LPP lanes add their sums by a xor butterfly: the same order for every position. The
// pre-activation x * (gain * rstd) is formed in fp64 and the SiLU in fp32 by
// activate_packet, as in gn_silu_apply. RSTD: the same launch writes each position's rstd
// (fp64) instead of y -- the bits the activation would have used (rms_silu_rstd).
template <int LPP, int PPL, int U, bool RSTD = false>
__global__ __launch_bounds__(kThreads) void rms_silu_kernel(const uint4* __restrict__ x, uint4* __restrict__ y,
                                                            int64_t positions, int cp,
                                                            const float* __restrict__ gain, double eps,
                                                            double channels, double* __restrict__ rstd_out) {
  constexpr int PPW = 64 / LPP;                      // positions per wave
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPP, li = lane % LPP;
  float g[PPL][8];
#pragma unroll
  for (int j = 0; j < PPL; ++j) {
    const int col = li + j * LPP;
#pragma unroll
    for (int i = 0; i < 8; ++i) g[j][i] = !RSTD && col < cp ? gain[col * 8 + i] : 0.0f;
  }
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t stride = (int64_t)gridDim.x * (kThreads / 64) * U * PPW;
  for (int64_t base = wave * U * PPW; base < positions; base += stride) {
    uint4 v[U][PPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t pos = base + u * PPW + sub;
#pragma unroll
      for (int j = 0; j < PPL; ++j) {
        const int col = li + j * LPP;
        v[u][j] = pos < positions && col < cp ? load_stream(x + pos * cp + col) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t pos = base + u * PPW + sub;
      double ss = 0.0;
#pragma unroll
      for (int j = 0; j < PPL; ++j) {
        const uint32_t d[4] = {v[u][j].x, v[u][j].y, v[u][j].z, v[u][j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const double a = (double)bf16_lo(d[i]), b = (double)bf16_hi(d[i]);
          ss = fma(a, a, ss);
          ss = fma(b, b, ss);
        }
      }
#pragma unroll
      for (int o = LPP / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
      const double rstd = 1.0 / sqrt(ss / channels + eps);
      if constexpr (RSTD) {
        if (li == 0 && pos < positions) rstd_out[pos] = rstd;
        continue;
      }
#pragma unroll
      for (int j = 0; j < PPL; ++j) {
        const int col = li + j * LPP;
        Affine a[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          a[i].s = (double)g[j][i] * rstd;
          a[i].b = 0.0;
        }
        if (pos < positions && col < cp) store_stream(y + pos * cp + col, activate_packet(v[u][j], a));
      }
    }
  }
}

}  // namespace sgn

using namespace sgn;

extern "C" int gn_silu_eligible(sgn_dims d, int groups) {
  clear_error();
  return gn_shape_ok(d, groups, "gn_silu_eligible") ? 1 : 0;
}

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
  const size_t xb = (size_t)(d.n * positions * d.c) * 2, sb = (size_t)d.n * groups * 2 * sizeof(double);
  if (overlap(ws, need, x, xb) || overlap(stats, sb, x, xb) || overlap(ws, need, stats, sb)) {
    set_error("gn_silu_stats: x, stats and the workspace must not overlap");
    return SGN_EALIAS;
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

// ---------------------------------------------------------------- statistics without a workspace
// The per-block partial sums of gn_silu_stats_noalloc live in this file-scope array (one copy
// per GPU, held until the process ends). Host code never passes the array's name to a kernel:
// it is a host-side stand-in, not the device address. The address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr int64_t kScratchDoubles = 1 << 19;      // 4 MiB
static __device__ __align__(256) double scratch[kScratchDoubles];

namespace sgn {

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];       // per device ordinal, null until first looked up

static double* scratch_for_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return static_cast<double*>(g_scratch_ptr[dev]);
}

}  // namespace sgn

extern "C" int gn_silu_stats_noalloc(const uint16_t* x, sgn_dims d, int groups, double* stats,
                                     hipStream_t stream) {
  const char* fn = "gn_silu_stats_noalloc";
  clear_error();
  if (!gn_shape_ok(d, groups, fn)) return SGN_EINVAL;
  if (!x || !stats) {
    set_error("%s: x and stats are required", fn);
    return SGN_EINVAL;
  }
  if (!aligned16(x) || ((uintptr_t)stats & 7)) {
    set_error("%s: x must be 16-byte and stats 8-byte aligned", fn);
    return SGN_EALIGN;
  }
  // Every (sample, group) needs at least one partial (S, Q) pair in the scratch array.
  if ((double)d.n * groups * 2 > (double)kScratchDoubles) {
    set_error("%s: N x groups = %lld exceeds the %lld (sample, group) pairs the scratch holds", fn,
              (long long)(d.n * groups), (long long)(kScratchDoubles / 2));
    return SGN_EINVAL;
  }
  const int64_t positions = d.t * d.h * d.w;
  const size_t xb = (size_t)(d.n * positions * d.c) * 2, sb = (size_t)d.n * groups * 2 * sizeof(double);
  if (overlap(stats, sb, x, xb)) {
    set_error("%s: stats must not overlap x", fn);
    return SGN_EALIAS;
  }
  double* ws = scratch_for_current_device();
  if (!ws) {
    set_error("%s: cannot look up the scratch array's device address", fn);
    return SGN_ELAUNCH;
  }
  const int cg = (int)(d.c / groups);
  const int gpp = cg >= 8 ? 1 : 8 / cg;
  const void* partial = gpp == 1   ? (const void*)gn_stats_partial<1>
                        : gpp == 2 ? (const void*)gn_stats_partial<2>
                        : gpp == 4 ? (const void*)gn_stats_partial<4>
                                   : (const void*)gn_stats_partial<8>;
  // As gn_silu_stats, with the partial-sum blocks capped so that they fit the scratch array
  // (with 32 groups the cap is above the resident grid: the same blocks, the same bits).
  int max_blocks = resident_blocks(partial);
  const int64_t fit = kScratchDoubles / ((int64_t)groups * 2);
  if (max_blocks > fit) max_blocks = (int)fit;
  PacketGrid g = packet_grid(positions, (int)d.c, (int)d.n, 8, max_blocks);
  if ((int64_t)d.n * groups * 2 * g.blocks > kScratchDoubles) {
    set_error("%s: internal: %d partial blocks per sample do not fit the scratch", fn, g.blocks);
    return SGN_EINVAL;
  }
  dim3 grid(g.blocks, (unsigned)d.n);
  const uint4* xp = reinterpret_cast<const uint4*>(x);
  switch (gpp) {
    case 1: gn_stats_partial<1><<<grid, kThreads, 0, stream>>>(xp, positions, g.cp, g.rstep, g.rows_per_block, cg, groups, ws); break;
    case 2: gn_stats_partial<2><<<grid, kThreads, 0, stream>>>(xp, positions, g.cp, g.rstep, g.rows_per_block, cg, groups, ws); break;
    case 4: gn_stats_partial<4><<<grid, kThreads, 0, stream>>>(xp, positions, g.cp, g.rstep, g.rows_per_block, cg, groups, ws); break;
    default: gn_stats_partial<8><<<grid, kThreads, 0, stream>>>(xp, positions, g.cp, g.rstep, g.rows_per_block, cg, groups, ws); break;
  }
  if (!launch_ok("gn_silu_stats_noalloc (partial)")) return SGN_ELAUNCH;
  gn_stats_finalize<<<dim3(groups, (unsigned)d.n), kThreads, 0, stream>>>(ws, g.blocks, groups,
                                                                          (double)positions * cg, stats);
  if (!launch_ok("gn_silu_stats_noalloc (finalize)")) return SGN_ELAUNCH;
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
  // Passes of rstep x kApplyUnroll rows; up to kApplyBlocks workgroups in all sweep them.
  const int cp = (int)(d.c / 8), rstep = kThreads / cp;
  const int64_t passes = (positions + (int64_t)rstep * kApplyUnroll - 1) / ((int64_t)rstep * kApplyUnroll);
  int64_t blocks = kApplyBlocks / d.n;
  if (blocks < 1) blocks = 1;
  if (blocks > passes) blocks = passes;
  const int cg = (int)(d.c / groups);
  gn_apply_kernel<<<dim3((unsigned)blocks, (unsigned)d.n), kThreads, 0, stream>>>(
      reinterpret_cast<const uint4*>(x), reinterpret_cast<uint4*>(y), positions, cp, rstep, stats, gamma, beta,
      (double)eps, groups, cg);
  if (!launch_ok("gn_silu_apply")) return SGN_ELAUNCH;
  return SGN_OK;
}

// rms_silu (rstd_out == null) or rms_silu_rstd (rstd_out != null): the same kernel and
// launch shape, so the rstd the second writes is the one the first applies.
static void launch_rms(const uint16_t* x, sgn_dims d, const float* gain, float eps, uint16_t* y,
                       double* rstd_out, hipStream_t stream) {
  const int64_t positions = d.n * d.t * d.h * d.w;
  const int cp = (int)(d.c / 8);
  const uint4* xp = reinterpret_cast<const uint4*>(x);
  uint4* yp = reinterpret_cast<uint4*>(y);
  const double e = (double)eps, c = (double)d.c;
  // LPP = the power of two >= C/8 (8 .. 64), then PPL packets per lane past 64 lanes;
  // per block: 4 waves x (64 / LPP positions) x U groups.
  // The grid sweeps the positions as the GroupNorm apply does (up to kApplyBlocks workgroups).
  auto launch = [&](auto plain, auto rstd_only, int64_t per_block) {
    int64_t blocks = (positions + per_block - 1) / per_block;
    if (blocks > kApplyBlocks) blocks = kApplyBlocks;
    if (rstd_out)
      rstd_only<<<dim3((unsigned)blocks), kThreads, 0, stream>>>(xp, yp, positions, cp, gain, e, c, rstd_out);
    else
      plain<<<dim3((unsigned)blocks), kThreads, 0, stream>>>(xp, yp, positions, cp, gain, e, c, rstd_out);
  };
  if (cp <= 8) launch(rms_silu_kernel<8, 1, 4>, rms_silu_kernel<8, 1, 4, true>, 4 * 8 * 4);
  else if (cp <= 16) launch(rms_silu_kernel<16, 1, 4>, rms_silu_kernel<16, 1, 4, true>, 4 * 4 * 4);
  else if (cp <= 32) launch(rms_silu_kernel<32, 1, 4>, rms_silu_kernel<32, 1, 4, true>, 4 * 2 * 4);
  else if (cp <= 64) launch(rms_silu_kernel<64, 1, 4>, rms_silu_kernel<64, 1, 4, true>, 4 * 1 * 4);
  else if (cp <= 128) launch(rms_silu_kernel<64, 2, 2>, rms_silu_kernel<64, 2, 2, true>, 4 * 1 * 2);
  else if (cp <= 256) launch(rms_silu_kernel<64, 4, 1>, rms_silu_kernel<64, 4, 1, true>, 4);
  else launch(rms_silu_kernel<64, 8, 1>, rms_silu_kernel<64, 8, 1, true>, 4);
}

extern "C" int rms_silu(const uint16_t* x, sgn_dims d, const float* gain, float eps, uint16_t* y,
                        hipStream_t stream) {
  clear_error();
  if (!dims_ok(d, "rms_silu")) return SGN_EINVAL;
  if (d.c % 64 != 0 || d.c > 4096) {
    set_error("rms_silu: C=%lld must be a multiple of 64, at most 4096", (long long)d.c);
    return SGN_EINVAL;
  }
  if (!x || !gain || !y) {
    set_error("rms_silu: x, gain and y are required");
    return SGN_EINVAL;
  }
  if (!(eps > 0.0f) || !isfinite(eps)) {
    set_error("rms_silu: eps must be a positive finite number");
    return SGN_EINVAL;
  }
  if (!aligned16(x) || !aligned16(y) || ((uintptr_t)gain & 3)) {
    set_error("rms_silu: x, y must be 16-byte aligned (gain 4)");
    return SGN_EALIGN;
  }
  const size_t bytes = (size_t)(d.n * d.t * d.h * d.w * d.c) * 2;
  if ((const void*)x != (const void*)y && overlap(x, bytes, y, bytes)) {
    set_error("rms_silu: y partially overlaps x (only y == x is allowed)");
    return SGN_EALIAS;
  }
  launch_rms(x, d, gain, eps, y, nullptr, stream);
  if (!launch_ok("rms_silu")) return SGN_ELAUNCH;
  return SGN_OK;
}

extern "C" int rms_silu_rstd(const uint16_t* x, sgn_dims d, float eps, double* rstd, hipStream_t stream) {
  const char* fn = "rms_silu_rstd";
  clear_error();
  if (!dims_ok(d, fn)) return SGN_EINVAL;
  if (d.c % 64 != 0 || d.c > 4096) {
    set_error("%s: C=%lld must be a multiple of 64, at most 4096", fn, (long long)d.c);
    return SGN_EINVAL;
  }
  if (!x || !rstd) {
    set_error("%s: x and rstd are required", fn);
    return SGN_EINVAL;
  }
  if (!(eps > 0.0f) || !isfinite(eps)) {
    set_error("%s: eps must be a positive finite number", fn);
    return SGN_EINVAL;
  }
  if (!aligned16(x) || ((uintptr_t)rstd & 7)) {
    set_error("%s: x must be 16-byte and rstd 8-byte aligned", fn);
    return SGN_EALIGN;
  }
  const int64_t positions = d.n * d.t * d.h * d.w;
  if (overlap(x, (size_t)(positions * d.c) * 2, rstd, (size_t)positions * 8)) {
    set_error("%s: rstd overlaps x", fn);
    return SGN_EALIAS;
  }
  launch_rms(x, d, nullptr, eps, nullptr, rstd, stream);
  if (!launch_ok(fn)) return SGN_ELAUNCH;
  return SGN_OK;
}
