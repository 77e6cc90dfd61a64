// Implicit-GEMM convolutions on bf16 MFMA (gfx950): the causal 3x3x3 convolution with
// its 2-frame cache, the nearest-x2 upsample as four 2x2 phase convolutions (optionally
// with an up block's DupUp3D shortcut), an up block's causal 3x1x1 temporal x2, and the
// output head with its 2x2 depth-to-space. Epilogues can also emit the next GroupNorm's
// statistics or apply the next RMS norm + SiLU.
//
// GEMM view (per sample, per upsample phase):
//   D[k][m] = sum_{tap, c} W[k][tap][c] * P[src(m, tap)][c]
// with m an output position, k an output channel and src(m, tap) the input position a
// tap reads (or a zero row for padding). A workgroup of 4 waves computes a BN x BM tile
// of D with v_mfma_f32_32x32x16_bf16, its operands staged through a ring of LDS buffers
// (conv_kernel below describes the pipeline). With GroupNorm fused, position rows go
// through VGPRs instead of straight to LDS: loaded, activated by the same
// activate_packet() as gn_silu_apply (so the result is bitwise that of
// apply-then-convolve), and written to the same swizzled slots; the decoder's RMS norm is
// applied the same way from a per-position rstd (rms_silu's arithmetic).
//
// Pages: FastVideo wan22_vae_decode binding.cpp -- Decoder::conv (causal front padding
// of kt-1 frames from the cache, 1-pixel spatial zero padding, the cache keeps the last
// 2 frames of the padded input, bias and residual in the epilogue), prepare() and
// Decoder::up (the four 2x2 phase convolutions of nearest-x2 + 3x3, interleaved with the
// bias), Decoder::output_head (the head convolution to 12 = 3 x 2 x 2 channels, bias,
// clamp) and decode_video's write of the 2x2-unfolded RGB video; Decoder::up_block (the
// temporal x2 after the resnets, the DupUp3D shortcut in the resampler's last pass),
// Decoder's `prepared` edge (the next norm applied by the producing convolution) and
// norm_pad (the RMS norm + SiLU of a convolution's input).
#include <math.h>
#include <stdio.h>

#include "common.hpp"
#include "host.hpp"
#include "silugn.h"

namespace sgn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kCMax = 4096;      // largest C

// An int as a type, for compile-time arguments of generic lambdas.
template <int V>
struct IC {
  static constexpr int value = V;
};

enum Mode { kCausal = 0, kPhase = 1, kHead = 2, kTime = 3, kWino = 4 };

struct ConvParams {
  const uint16_t* x;
  const uint16_t* cache;     // (N,2,H,W,C) or null
  const uint16_t* w;         // (K,taps,C), or for phases (4,K,4,C)
  const float* bias;         // [K] or null
  const uint16_t* res;       // (N,T,H,W,K) or null
  uint16_t* y;
  const double* stats;       // fused GroupNorm (null when not fused)
  const float* gamma;
  const float* beta;
  double eps;
  int groups;
  int T, H, W, C, K;
  int tiles_f, tiles_n;      // tiles per frame (M), tiles along K (N)
  int64_t mper;              // output positions per sample (and per phase)
  int nblocks;
  int clamp;
  // Statistics of y for the next GroupNorm (causal, staged epilogue), or nws == null:
  // partial sums S, Q of every (sample, group, tile) in the layout gn_stats_finalize reads.
  double* nws;
  int ngroups, ncg;          // groups over K, channels per group (a multiple of 8 dividing BN)
  // Temporal x2 (kTime): x holds Tx frames per sample and the convolution reads them from
  // frame x0 on; y holds To frames per sample, and output frame first + 2 t + s takes
  // channels s K/2 .. (s + 1) K/2 - 1 of the convolution's frame t.
  int Tx, x0, To, first;
  // DupUp3D shortcut added by the phase epilogue, or sc == null: the block input, sc_T
  // frames of sc_C channels per sample at the phase convolution's H x W; time factor sc_ft,
  // sc_first = the first ft - 1 output frames are dropped.
  const uint16_t* sc;
  int sc_T, sc_C, sc_ft, sc_first;
  // The next RMS norm + SiLU written by the causal epilogue, or act == null: act =
  // silu(y * gain / sqrt(mean_k y^2 + eps)) per position over the K channels of the tile
  // (one N tile holds all of them); y itself is stored only if y != null.
  uint16_t* act;
  const float* rms_gain;
  double rms_eps;
  // Winograd products (kWino): sample n of the launch is component n / wino_n (of 36) of
  // sample n % wino_n; its weights start at w + component * K * 3 * C, and the fp32 products
  // go to yf (N x T frames of H x W positions -- the tiles -- by K channels).
  int wino_n;
  float* yf;
  // The RMS norm + SiLU applied in the operand load (conv_kernel with FUSE == kFuseRms):
  // rstd[n][t][h][w] of x (fp64, as rms_silu forms it), the gain in gamma.
  const double* rstd;
};

// What conv_kernel applies to x while loading it: nothing, silu(group_norm(x)) or
// silu(rms_norm(x)).
enum Fuse { kFuseNone = 0, kFuseGn = 1, kFuseRms = 2 };


constexpr int kRsrcFlags = 0x00020000;   // descriptor dword 3 (gfx9 raw buffer, 32-bit data)
constexpr uint32_t kOOB = 0x80000000u;   // an offset past every descriptor built here

typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcFlags);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Workgroup barrier without the memory fence of __syncthreads (which would also wait for
// every outstanding LDS move); LDS-move completion is handled by the counted waits.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Epilogue shared by the convolution kernels. Lane l of a 32x32 accumulator tile holds
// column m = l % 32 and rows k = 8 * (r / 4) + 4 * (l / 32) + r % 4 of element r; the
// tile's k rows start at kbase + 32 * i, its m columns at m0 + wm * WTM + 32 * j; columns
// at or past mlimit (the end of the tile's frame) are not stored.
// bias (+ residual) in fp32, one round to bf16, stored NDHWC (causal), interleaved at
// (2h + a, 2w + b) (phases), or unfolded 2x2 into the channels-first video (head).
// The bias comes from LDS (lbias: the workgroup's BN entries, zeros without a bias), and
// every residual load is issued before the first store: vmcnt counts stores as well as
// loads, so a load issued after stores would make its use wait for those stores. A wave
// whose whole tile lies inside the frame and K takes a path without per-lane conditions.
template <int MODE, int TN, int TM, int WTM, int WTN>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[TN][TM], const ConvParams& p, int n,
                                           int64_t m0, int64_t mlimit, int kbase, int wm, int lane,
                                           int phase, const float* lbias) {
  const int K = p.K, H = p.H, W = p.W, T = p.T;
  const int pa = phase >> 1, pb = phase & 1;
  auto body = [&](auto full_c) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_c)::value;
    uint2 rv[MODE == kCausal ? TM : 1][TN][4];
    if (MODE == kCausal && p.res) {
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int64_t m = m0 + wm * WTM + j * 32 + (lane & 31);
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int k0 = kbase + i * 32 + 8 * q + 4 * (lane >> 5);
            const uint2* src = reinterpret_cast<const uint2*>(p.res + ((int64_t)n * p.mper + m) * K + k0);
            rv[MODE == kCausal ? j : 0][i][q] = FULL || (m < mlimit && k0 < K) ? *src : make_uint2(0, 0);
          }
      }
    }
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int64_t m = m0 + wm * WTM + j * 32 + (lane & 31);
      if (!FULL && m >= mlimit) continue;
      const int w_ = (int)(m % W);
      const int64_t th = m / W;
      const int h_ = (int)(th % H);
      const int t_ = (int)(th / H);
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kr = i * 32 + 8 * q + 4 * (lane >> 5);      // row within the wave's tile
          const int k0 = kbase + kr;
          if (!FULL && k0 >= K) continue;
          const float4 b = *reinterpret_cast<const float4*>(lbias + kr);
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * q + r];
          v[0] += b.x;
          v[1] += b.y;
          v[2] += b.z;
          v[3] += b.w;
          if (MODE == kCausal) {
            const int64_t off = ((int64_t)n * p.mper + m) * K + k0;
            if (p.res) {
              const uint2 rr = rv[MODE == kCausal ? j : 0][i][q];
              v[0] += bf16_lo(rr.x);
              v[1] += bf16_hi(rr.x);
              v[2] += bf16_lo(rr.y);
              v[3] += bf16_hi(rr.y);
            }
            uint2 o;
            o.x = pack_bf16x2(v[0], v[1]);
            o.y = pack_bf16x2(v[2], v[3]);
            *reinterpret_cast<uint2*>(p.y + off) = o;
          } else if (MODE == kPhase) {
            const int64_t yy = 2 * h_ + pa, xx = 2 * w_ + pb;
            const int64_t off = ((((int64_t)n * T + t_) * (2 * H) + yy) * (2 * W) + xx) * K + k0;
            uint2 o;
            o.x = pack_bf16x2(v[0], v[1]);
            o.y = pack_bf16x2(v[2], v[3]);
            *reinterpret_cast<uint2*>(p.y + off) = o;
          } else {
            // K = 12: k0 = 4c, the four values are (dy, dx) = (0,0), (0,1), (1,0), (1,1).
            if (p.clamp) {
#pragma unroll
              for (int r = 0; r < 4; ++r) v[r] = fminf(fmaxf(v[r], -1.0f), 1.0f);
            }
            const int c = k0 >> 2;
            const int64_t W2 = 2 * (int64_t)W;
            const int64_t base = (((int64_t)n * 3 + c) * T + t_) * (2 * (int64_t)H) * W2;
            *reinterpret_cast<uint32_t*>(p.y + base + (2 * h_) * W2 + 2 * w_) = pack_bf16x2(v[0], v[1]);
            *reinterpret_cast<uint32_t*>(p.y + base + (2 * h_ + 1) * W2 + 2 * w_) = pack_bf16x2(v[2], v[3]);
          }
        }
    }
  };
  const bool full = m0 + wm * WTM + TM * 32 <= mlimit && kbase + TN * 32 <= K;
  if (full)
    body(IC<1>{});
  else
    body(IC<0>{});
}

// Epilogue through LDS, for the causal and phase forms: one store instruction of the direct
// form above writes 8 bytes per lane to 64 cache lines (the 32 positions of a fragment are
// K channels apart), and a wave's 64 of them queue behind the CU's address unit. Here each
// wave stages fp32 (acc + bias) of 32 positions x its WTN channels in its own LDS area
// (after a workgroup barrier: the area held operand stages), reads it back as 8 channels
// per lane and adds the residual, loaded 16 contiguous bytes per lane before the first
// store. A store instruction then covers 64 / (WTN / 8) positions x WTN channels: 8 lines.
// Loads and stores go through raw-buffer descriptors over the tile's output (and residual)
// frame, so rows past the frame read zeros and drop their stores without a branch.
// Numerics as in store_tile: one rounding of acc + bias (+ residual). Used when K % 8 == 0,
// so that every 16-byte access is aligned.
// Staging layout: row r (position) of WTN * 4 bytes; the 16-byte chunk c (4 channels) sits
// at c ^ (r & SWZ), SWZ = min(15, WTN / 4 - 1), so 8 consecutive rows at one chunk, and 8
// chunks of one row, hit distinct bank groups.
struct Sums {
  double s, q;
};

template <int MODE, int TN, int TM, int WTM, int WTN, bool SC>
__device__ __forceinline__ Sums store_tile_staged(const f32x16 (&acc)[TN][TM], const ConvParams& p, int n,
                                                  int t, int pos0, int kbase, int wm, int lane,
                                                  int phase, const float* lbias, char* stage) {
  static_assert(MODE == kCausal || MODE == kPhase || MODE == kTime, "staged epilogue modes");
  constexpr int ROW = WTN * 4;                       // staging row bytes
  constexpr int LPR = WTN / 8;                       // lanes per row on the way out
  constexpr int RPI = 64 / LPR;                      // rows per instruction
  constexpr int NI = 32 / RPI;                       // instructions per 32 rows
  static_assert(LPR * RPI == 64 && RPI * NI == 32, "staging shape");
  constexpr int SWZ = WTN / 4 < 16 ? WTN / 4 - 1 : 15;   // chunk swizzle stays inside the row
  const int K = p.K, H = p.H, W = p.W, T = p.T;
  const int HW = H * W;
  const int pa = phase >> 1, pb = phase & 1;
  const int g = lane % LPR;                          // 8-channel group of this lane
  const int k0 = kbase + 8 * g;
  // The tile's span of y: one frame of HW positions (causal) or 2H x 2W (phases), K channels
  // each; for the temporal x2 the two output frames first + 2t, first + 2t + 1 of K / 2
  // channels (same bytes), channel k0 going to the second when k0 >= K / 2.
  const int64_t fpos = MODE == kPhase ? 4 * (int64_t)HW : (int64_t)HW;
  const int64_t fidx = (int64_t)n * T + t;
  const int KH = K / 2;
  const int sub = MODE == kTime && k0 >= KH ? 1 : 0;
  const int64_t ybase = MODE == kTime ? ((int64_t)n * p.To + p.first + 2 * t) * HW * KH : fidx * fpos * K;
  const Rsrc ys = make_rsrc(p.y + ybase, (uint32_t)(fpos * K * 2));
  const bool kfull = kbase + WTN <= K;               // wave-uniform: no channel tail
  auto out_off = [&](int ml) -> uint32_t {           // ml: position within the frame
    if (MODE == kCausal) return (uint32_t)(((int64_t)ml * K + k0) * 2);
    if (MODE == kTime)                               // past the frame: dropped (not the next frame)
      return ml < HW ? (uint32_t)((((int64_t)sub * HW + ml) * KH + k0 - sub * KH) * 2) : kOOB;
    const int h_ = ml / W, w_ = ml - h_ * W;
    return (uint32_t)(((((int64_t)(2 * h_ + pa)) * (2 * W) + 2 * w_ + pb) * K + k0) * 2);
  };
  // DupUp3D shortcut (phases): output channel c of phase (pa, pb) in output frame t reads
  // source channel (c F + o) / rep of frame (t + first (ft - 1)) / ft, with F = 4 ft,
  // o = (a 2 + pa) 2 + pb, a = (t + first (ft - 1)) % ft and rep = K F / Cs. The host admits
  // Cs = K (source channel c) and Cs = 2K (source channel 2c + o / rep): a lane's 8 output
  // channels read 16 or 32 contiguous source bytes. Uniform per tile.
  const bool shortcut = MODE == kPhase && SC && p.sc != nullptr;
  Rsrc scs = make_rsrc(p.y, 0);
  int sc_step = 1, sc_e = 0;
  if (shortcut) {
    const int tt = t + p.sc_first * (p.sc_ft - 1);
    const int tsrc = tt / p.sc_ft, a = tt - tsrc * p.sc_ft;
    const int F = 4 * p.sc_ft;
    const int rep = K * F / p.sc_C;
    sc_step = p.sc_C / K;
    sc_e = ((a * 2 + pa) * 2 + pb) / rep;
    scs = make_rsrc(p.sc + ((int64_t)n * p.sc_T + tsrc) * HW * p.sc_C, (uint32_t)((int64_t)HW * p.sc_C * 2));
  }
  // Statistics for the next GroupNorm: this lane's stored values and their exact squares.
  const bool stats = MODE == kCausal && p.nws != nullptr;
  double ss = 0.0, sq = 0.0;
  // Residual of every row this lane stores, before any store.
  u32x4 rv[MODE == kCausal ? TM : 1][MODE == kCausal ? NI : 1];
  if (MODE == kCausal && p.res) {
    const Rsrc rs = make_rsrc(p.res + fidx * fpos * K, (uint32_t)(fpos * K * 2));
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        const int ml = pos0 + wm * WTM + 32 * j + it * RPI + lane / LPR;
        // past the frame: zeros; past K (a tail lane): the next row's channels, never used
        rv[MODE == kCausal ? j : 0][MODE == kCausal ? it : 0] =
            __builtin_amdgcn_raw_buffer_load_b128(rs, out_off(ml), 0, 0);
      }
  }
  stage_barrier();                                   // every wave is done with the operand stages
  // The biases of this lane's 8 channels, read once: the staging writes below could alias
  // the bias area as far as the compiler knows, so a bias read per staged fragment would
  // wait for its data before each write.
  float bsv[8];
  {
    const float4 b0 = *reinterpret_cast<const float4*>(lbias + 8 * g);
    const float4 b1 = *reinterpret_cast<const float4*>(lbias + 8 * g + 4);
    bsv[0] = b0.x, bsv[1] = b0.y, bsv[2] = b0.z, bsv[3] = b0.w;
    bsv[4] = b1.x, bsv[5] = b1.y, bsv[6] = b1.z, bsv[7] = b1.w;
  }
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    // Shortcut rows of this fragment row block, issued before its staging writes.
    u32x4 sv[MODE == kPhase ? NI : 1][2];
    if (shortcut) {
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        const int ml = pos0 + wm * WTM + 32 * j + it * RPI + lane / LPR;
        const uint32_t so = (uint32_t)(((int64_t)ml * p.sc_C + k0 * sc_step) * 2);
        sv[MODE == kPhase ? it : 0][0] = __builtin_amdgcn_raw_buffer_load_b128(scs, so, 0, 0);
        if (sc_step == 2) sv[MODE == kPhase ? it : 0][1] = __builtin_amdgcn_raw_buffer_load_b128(scs, so + 16, 0, 0);
      }
    }
    {
      const int r = lane & 31;
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kr = i * 32 + 8 * q + 4 * (lane >> 5);
          float4 v;
          v.x = acc[i][j][4 * q + 0];
          v.y = acc[i][j][4 * q + 1];
          v.z = acc[i][j][4 * q + 2];
          v.w = acc[i][j][4 * q + 3];
          *reinterpret_cast<float4*>(stage + r * ROW + (((kr >> 2) ^ (r & SWZ)) << 4)) = v;
        }
    }
    wait_lgkm0();                                    // this wave's rows are in its area
    // All of the block's staged rows are read before the first store: one LDS round trip
    // per block instead of one per row group.
    float4 lov[NI], hiv[NI];
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int r = it * RPI + lane / LPR;
      lov[it] = *reinterpret_cast<const float4*>(stage + r * ROW + (((2 * g) ^ (r & SWZ)) << 4));
      hiv[it] = *reinterpret_cast<const float4*>(stage + r * ROW + (((2 * g + 1) ^ (r & SWZ)) << 4));
    }
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int r = it * RPI + lane / LPR;
      const float4 lo = lov[it], hi = hiv[it];
      float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += bsv[e];    // acc + bias, as before the residual
      if (MODE == kCausal && p.res) {
        const u32x4 rr = rv[MODE == kCausal ? j : 0][MODE == kCausal ? it : 0];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] += bf16_lo(rr[e]);
          v[2 * e + 1] += bf16_hi(rr[e]);
        }
      }
      if (shortcut) {
        const u32x4 s0 = sv[MODE == kPhase ? it : 0][0];
        if (sc_step == 1) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] += bf16_lo(s0[e]);
            v[2 * e + 1] += bf16_hi(s0[e]);
          }
        } else {                                     // source channels 2c + sc_e
          const u32x4 s1 = sv[MODE == kPhase ? it : 0][1];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] += sc_e ? bf16_hi(s0[e]) : bf16_lo(s0[e]);
            v[4 + e] += sc_e ? bf16_hi(s1[e]) : bf16_lo(s1[e]);
          }
        }
      }
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
      const int ml = pos0 + wm * WTM + 32 * j + r;
      if (stats && ml < HW && k0 < K) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double lo2 = bf16_lo(o[e]), hi2 = bf16_hi(o[e]);
          ss += lo2;
          ss += hi2;
          sq = fma(lo2, lo2, sq);
          sq = fma(hi2, hi2, sq);
        }
      }
      if (kfull) {
        __builtin_amdgcn_raw_buffer_store_b128(o, ys, out_off(ml), 0, 0);   // past the frame: dropped
      } else if (k0 < K && ml < HW) {
        uint16_t* dst = p.y + ybase + out_off(ml) / 2;
        if (k0 + 8 <= K)
          *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
        else
          *reinterpret_cast<uint2*>(dst) = make_uint2(o[0], o[1]);
      }
    }
    wait_lgkm0();                                    // reads done before the next rows land
  }
  return Sums{ss, sq};
}

// Epilogue of the Winograd products: fp32 acc of 32 positions x WTN channels per wave staged
// in LDS as store_tile_staged does, read back as 4 channels (16 bytes) per lane and stored,
// unrounded, to yf: frame n * T + t of H x W positions (the tiles), K channels each, through a
// descriptor over that frame (rows past it are dropped). K % 4 == 0.
template <int TN, int TM, int WTM, int WTN>
__device__ __forceinline__ void store_tile_f32(const f32x16 (&acc)[TN][TM], const ConvParams& p, int n, int t,
                                               int pos0, int kbase, int wm, int lane, char* stage) {
  constexpr int ROW = WTN * 4;                       // staging row bytes
  constexpr int LPR = WTN / 4;                       // lanes per row on the way out
  constexpr int RPI = 64 / LPR;                      // rows per instruction
  constexpr int NI = 32 / RPI;                       // instructions per 32 rows
  static_assert(LPR * RPI == 64 && RPI * NI == 32, "staging shape");
  constexpr int SWZ = WTN / 4 < 16 ? WTN / 4 - 1 : 15;
  const int K = p.K, HW = p.H * p.W;
  const int g = lane % LPR;                          // 4-channel group of this lane
  const int k0 = kbase + 4 * g;
  const int64_t base = ((int64_t)n * p.T + t) * HW * K;
  const Rsrc ms = make_rsrc(p.yf + base, (uint32_t)((int64_t)HW * K * 4));
  const bool kfull = kbase + WTN <= K;
  stage_barrier();                                   // every wave is done with the operand stages
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    {
      const int r = lane & 31;
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kr = i * 32 + 8 * q + 4 * (lane >> 5);
          float4 v;
          v.x = acc[i][j][4 * q + 0];
          v.y = acc[i][j][4 * q + 1];
          v.z = acc[i][j][4 * q + 2];
          v.w = acc[i][j][4 * q + 3];
          *reinterpret_cast<float4*>(stage + r * ROW + (((kr >> 2) ^ (r & SWZ)) << 4)) = v;
        }
    }
    wait_lgkm0();                                    // this wave's rows are in its area
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int r = it * RPI + lane / LPR;
      const float4 v = *reinterpret_cast<const float4*>(stage + r * ROW + ((g ^ (r & SWZ)) << 4));
      const int ml = pos0 + wm * WTM + 32 * j + r;
      if (kfull) {
        const u32x4 o = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
        __builtin_amdgcn_raw_buffer_store_b128(o, ms, (uint32_t)(((int64_t)ml * K + k0) * 4), 0, 0);
      } else if (k0 < K && ml < HW) {
        *reinterpret_cast<float4*>(p.yf + base + (int64_t)ml * K + k0) = v;
      }
    }
    wait_lgkm0();                                    // reads done before the next rows land
  }
}

// Causal epilogue that also applies the next RMS norm + SiLU (the decoder's norm is per
// position, so a workgroup whose N tile holds all K channels has every value it needs). Per
// 32-row block: stage fp32 (acc + bias) as store_tile_staged does, form the rounded outputs
// (+ residual) and each lane's fp64 sum of their exact squares; add the sums of a row's LPR
// lanes by DPP moves, publish the wave's row sums in LDS (two buffers by block
// parity, one barrier per block), add the WGN waves' sums in wave order, and activate with
// gain * rstd in fp64 through activate_packet (the code rms_silu runs). Channels past K
// add nothing; rows past the frame and channels past K store nothing. Every wave takes
// the same barriers.
// v of the lane LPR lanes away in DPP terms: a 32-bit cross-lane move per half of the double.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  union {
    double d;
    int i[2];
  } u, r;
  u.d = v;
  r.i[0] = __builtin_amdgcn_update_dpp(0, u.i[0], CTRL, 0xF, 0xF, false);
  r.i[1] = __builtin_amdgcn_update_dpp(0, u.i[1], CTRL, 0xF, 0xF, false);
  return r.d;
}

// Sum of v over each aligned group of LPR (8 or 16) lanes, in lane 0 of the group: a row
// mirror (16), a half-row mirror (8), then two quad permutes -- register-to-register moves,
// a fixed order of additions.
template <int LPR>
__device__ __forceinline__ double group_sum_dpp(double v) {
  static_assert(LPR == 8 || LPR == 16, "lane groups of 8 or 16");
  if constexpr (LPR == 16) v += dpp_f64<0x140>(v);   // row_mirror: lane i + lane 15 - i
  v += dpp_f64<0x141>(v);                           // row_half_mirror: lane i + lane 7 - i
  v += dpp_f64<0x4E>(v);                            // quad_perm [2, 3, 0, 1]
  v += dpp_f64<0xB1>(v);                            // quad_perm [1, 0, 3, 2]
  return v;
}

template <int TN, int TM, int WTM, int WTN, int WGM, int WGN>
__device__ __forceinline__ void store_tile_rms(const f32x16 (&acc)[TN][TM], const ConvParams& p, int n, int t,
                                               int pos0, int kbase, int wm, int wn, int lane, const float* lbias,
                                               char* stage, double* rred, char* opark, float* lgain) {
  constexpr int ROW = WTN * 4;
  constexpr int LPR = WTN / 8;
  constexpr int RPI = 64 / LPR;
  constexpr int NI = 32 / RPI;
  static_assert(LPR * RPI == 64 && RPI * NI == 32, "staging shape");
  constexpr int SWZ = WTN / 4 < 16 ? WTN / 4 - 1 : 15;
  const int K = p.K, HW = p.H * p.W;
  const int g = lane % LPR;
  const int k0 = kbase + 8 * g;
  const bool kin = k0 < K;
  const int64_t base = ((int64_t)n * p.T + t) * HW * K;
  const uint32_t fbytes = (uint32_t)((int64_t)HW * K * 2);
  const Rsrc as = make_rsrc(p.act + base, fbytes);
  const Rsrc ys = make_rsrc(p.y ? p.y + base : p.act, p.y ? fbytes : 0u);
  const bool kfull = kbase + WTN <= K;
  const Rsrc rs = make_rsrc(p.res ? p.res + base : p.act, p.res ? fbytes : 0u);
  // The wave's WTN gains, read before any store (a load issued after stores would wait for
  // them: vmcnt counts both) and kept in LDS.
  float gload[(WTN + 63) / 64];
#pragma unroll
  for (int q = 0; q < (WTN + 63) / 64; ++q) {
    const int kk = kbase + q * 64 + lane;
    gload[q] = (q * 64 + lane < WTN && kk < K) ? p.rms_gain[kk] : 0.0f;
  }
  stage_barrier();                                   // every wave is done with the operand stages
#pragma unroll
  for (int q = 0; q < (WTN + 63) / 64; ++q)
    if (q * 64 + lane < WTN) lgain[q * 64 + lane] = gload[q];
  // this lane's 8 biases, read once (as in store_tile_staged)
  float bsv[8];
  {
    const float4 b0 = *reinterpret_cast<const float4*>(lbias + 8 * g);
    const float4 b1 = *reinterpret_cast<const float4*>(lbias + 8 * g + 4);
    bsv[0] = b0.x, bsv[1] = b0.y, bsv[2] = b0.z, bsv[3] = b0.w;
    bsv[4] = b1.x, bsv[5] = b1.y, bsv[6] = b1.z, bsv[7] = b1.w;
  }
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    {
      const int r = lane & 31;
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kr = i * 32 + 8 * q + 4 * (lane >> 5);
          float4 v;
          v.x = acc[i][j][4 * q + 0];
          v.y = acc[i][j][4 * q + 1];
          v.z = acc[i][j][4 * q + 2];
          v.w = acc[i][j][4 * q + 3];
          *reinterpret_cast<float4*>(stage + r * ROW + (((kr >> 2) ^ (r & SWZ)) << 4)) = v;
        }
    }
    // this block's residual (one block at a time, after the staging writes: registers are
    // short here)
    u32x4 rv[NI];
    if (p.res) {
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        const int ml = pos0 + wm * WTM + 32 * j + it * RPI + lane / LPR;
        rv[it] = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(((int64_t)ml * K + k0) * 2), 0, 0);
      }
    }
    wait_lgkm0();
    double* rb = rred + (j & 1) * (WGN * WGM * 32);
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int r = it * RPI + lane / LPR;
      const float4 lo = *reinterpret_cast<const float4*>(stage + r * ROW + (((2 * g) ^ (r & SWZ)) << 4));
      const float4 hi = *reinterpret_cast<const float4*>(stage + r * ROW + (((2 * g + 1) ^ (r & SWZ)) << 4));
      float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += bsv[e];    // acc + bias, as before the residual
      if (p.res) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] += bf16_lo(rv[it][e]);
          v[2 * e + 1] += bf16_hi(rv[it][e]);
        }
      }
      double ss = 0.0;
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
        const double a = bf16_lo(o[e]), b = bf16_hi(o[e]);
        ss = fma(a, a, ss);
        ss = fma(b, b, ss);
      }
      // the rounded outputs wait in this wave's LDS area across the barrier below
      *reinterpret_cast<u32x4*>(opark + (it * 64 + lane) * 16) = o;
      // this wave's sum for the row: its LPR lanes, by DPP moves (in lane g == 0)
      if (!kin) ss = 0.0;
      ss = group_sum_dpp<LPR>(ss);
      if (g == 0) rb[(wn * WGM + wm) * 32 + it * RPI + lane / LPR] = ss;
    }
    wait_lgkm0();                                    // staging reads and row sums done
    stage_barrier();                                 // every wave's row sums of this block
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int r = it * RPI + lane / LPR;
      double tot = rb[wm * 32 + r];
#pragma unroll
      for (int q = 1; q < WGN; ++q) tot += rb[(q * WGM + wm) * 32 + r];
      const double rstd = 1.0 / sqrt(tot / (double)K + p.rms_eps);
      // the lane's 8 gains from LDS (not held across the block: registers are short)
      const float4 g0 = *reinterpret_cast<const float4*>(lgain + 8 * g);
      const float4 g1 = *reinterpret_cast<const float4*>(lgain + 8 * g + 4);
      const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      Affine a[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        a[i].s = (double)gv[i] * rstd;
        a[i].b = 0.0;
      }
      const u32x4 ovv = *reinterpret_cast<const u32x4*>(opark + (it * 64 + lane) * 16);
      const uint4 o4 = make_uint4(ovv[0], ovv[1], ovv[2], ovv[3]);
      const uint4 act = activate_packet(o4, a);
      const int ml = pos0 + wm * WTM + 32 * j + r;
      const uint32_t off = (uint32_t)(((int64_t)ml * K + k0) * 2);
      if (kfull) {                                   // past the frame: dropped
        u32x4 av;
        av[0] = act.x;
        av[1] = act.y;
        av[2] = act.z;
        av[3] = act.w;
        __builtin_amdgcn_raw_buffer_store_b128(av, as, off, 0, 0);
        if (p.y) __builtin_amdgcn_raw_buffer_store_b128(ovv, ys, off, 0, 0);
      } else if (kin && ml < HW) {
        const int64_t e0 = base + (int64_t)ml * K + k0;
        if (k0 + 8 <= K) {
          *reinterpret_cast<uint4*>(p.act + e0) = act;
          if (p.y) *reinterpret_cast<uint4*>(p.y + e0) = o4;
        } else {
          *reinterpret_cast<uint2*>(p.act + e0) = make_uint2(act.x, act.y);
          if (p.y) *reinterpret_cast<uint2*>(p.y + e0) = make_uint2(o4.x, o4.y);
        }
      }
    }
  }
}

// Statistics for the next GroupNorm, per workgroup: every lane's (S, Q) of the rounded
// values it stored (8 channels of one group, its rows) goes to LDS; then one thread per
// group of the tile adds the lanes holding that group in a fixed order (waves by channel
// block, then row block; lanes by channel, then row) and writes the tile's partial where
// gn_stats_finalize reads it: ws[((n * G + g) * 2 + {0, 1}) * nblk + blk], nblk = T x tiles
// per frame, blk = t x tiles per frame + mt. A group lies inside one N tile (BN % cg == 0).
template <int NW, int WGM, int WTN, int BN>
__device__ __forceinline__ void next_stats_partials(const ConvParams& p, int n, int t, int mt, int ntile,
                                                    int wave, int lane, Sums sums, double* red) {
  constexpr int LPR = WTN / 8, RPI = 64 / LPR;
  red[(wave * 64 + lane) * 2 + 0] = sums.s;
  red[(wave * 64 + lane) * 2 + 1] = sums.q;
  __syncthreads();
  const int tid = threadIdx.x, cg = p.ncg;
  const int k_lo = ntile * BN;
  const int kt = p.K - k_lo < BN ? p.K - k_lo : BN;   // channels of this N tile
  if (tid < kt / cg) {
    const int c_begin = tid * cg;                   // the group's first channel in the tile
    double S = 0.0, Q = 0.0;
    for (int wn = 0; wn < NW / WGM; ++wn)
      for (int wm = 0; wm < WGM; ++wm)
        for (int c8 = 0; c8 < LPR; ++c8) {
          const int ch = wn * WTN + 8 * c8;
          if (ch < c_begin || ch >= c_begin + cg) continue;
          for (int rr = 0; rr < RPI; ++rr) {
            const int e = ((wn * WGM + wm) * 64 + rr * LPR + c8) * 2;
            S += red[e];
            Q += red[e + 1];
          }
        }
    const int nblk = p.T * p.tiles_f, blk = t * p.tiles_f + mt;
    double* o = p.nws + (((int64_t)n * p.ngroups + k_lo / cg + tid) * 2) * nblk;
    o[blk] = S;
    o[nblk + blk] = Q;
  }
}

// The bias of the workgroup's BN output channels (zeros past K or without a bias) into
// LDS: each of the first BN / 4 threads loads 16 bytes at issue_bias() and stores them at
// commit_bias(), which must come after a wait that covers the load (the load is issued
// before any other move, and counted waits complete moves in issue order).
template <int BN>
struct BiasStage {
  float4 v;
  __device__ __forceinline__ void issue(const ConvParams& p, int ntile, int tid) {
    v = make_float4(0.f, 0.f, 0.f, 0.f);
    const int k = ntile * BN + 4 * tid;
    if (tid < BN / 4 && p.bias && k < p.K) v = *reinterpret_cast<const float4*>(p.bias + k);
  }
  __device__ __forceinline__ void commit(float* lbias, int tid) {
    if (tid < BN / 4) *reinterpret_cast<float4*>(lbias + 4 * tid) = v;
  }
};

// cache_out = the last 2 frames of P = cat(cache_in, a), a = frames x0 .. x0 + T - 1 of the
// Tx frames per sample of x; frames of x are activated when fused (same per-thread column
// layout and activate_packet as gn_silu_apply; with rstd, rms_silu's per-position affine).
// Grid: (blocks over the H x W positions of a frame, sample n, cache frame f): the source
// frame of a block -- a frame of x, of cache_in, or zeros -- is uniform, and no thread
// divides by the frame size. A row of cp packets is covered by tpr = min(cp, 256) threads,
// each taking every tpr-th packet; rstep rows per block pass. A thread moves kCacheRows rows
// per iteration with all loads issued before the first store. ACT = false is the plain copy
// (no activation, few registers: more rows in flight per thread).
template <bool ACT>
__global__ __launch_bounds__(256) void cache_out_kernel(
    const uint4* __restrict__ x, const uint4* __restrict__ cache_in, uint4* __restrict__ cache_out, int T,
    int Tx, int x0, int64_t hw, int cp, int rstep, int64_t rows_per_block, const double* __restrict__ stats,
    const float* __restrict__ gamma, const float* __restrict__ beta, double eps, int groups,
    const double* __restrict__ rstd) {
  const int tid = threadIdx.x, n = blockIdx.y, f = blockIdx.z;
  const int tpr = cp < 256 ? cp : 256;
  if (tid >= rstep * tpr) return;
  constexpr int kCacheRows = ACT ? 4 : 8;
  const int c0 = tid % tpr;
  const int64_t start = (int64_t)blockIdx.x * rows_per_block;
  int64_t end = start + rows_per_block;
  if (end > hw) end = hw;
  const int pf = T + f;                              // frame of P = cat(cache_in, x)
  const uint4* src = nullptr;
  const double* rs = nullptr;
  if (pf >= 2) {
    const int64_t fx = (int64_t)n * Tx + x0 + pf - 2;
    src = x + fx * hw * cp;
    if (!stats && rstd) rs = rstd + fx * hw;
  } else if (cache_in) {
    src = cache_in + ((int64_t)n * 2 + pf) * hw * cp;
  }
  const bool act = ACT && pf >= 2 && (stats || rs);
  uint4* dst = cache_out + ((int64_t)n * 2 + f) * hw * cp;
  for (int col = c0; col < cp; col += tpr) {
    Affine a[8];
    if (ACT && stats && pf >= 2) {
      const int cg = cp * 8 / groups;
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] = channel_affine(stats, gamma, beta, eps, groups, cg, n, col * 8 + i);
    }
    for (int64_t q0 = start + tid / tpr; q0 < end; q0 += kCacheRows * rstep) {
      uint4 v[kCacheRows];
      double r[kCacheRows];
#pragma unroll
      for (int u = 0; u < kCacheRows; ++u) {
        const int64_t q = q0 + (int64_t)u * rstep;
        v[u] = make_uint4(0, 0, 0, 0);
        r[u] = 0.0;
        if (q < end && src) {
          v[u] = src[q * cp + col];
          if (ACT && rs) r[u] = rs[q];
        }
      }
#pragma unroll
      for (int u = 0; u < kCacheRows; ++u) {
        const int64_t q = q0 + (int64_t)u * rstep;
        if (q >= end) continue;
        uint4 o = v[u];
        if (act) {
          if (stats) {
            o = activate_packet(o, a);
          } else {                                   // the RMS norm: gain (in gamma) * rstd
            Affine ar[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              ar[i].s = (double)gamma[col * 8 + i] * r[u];
              ar[i].b = 0.0;
            }
            o = activate_packet(o, ar);
          }
        }
        dst[q * cp + col] = o;
      }
    }
  }
}

// y[n, 0] = x[n, 0] for every sample n (packets of 8 channels per frame; xs, ys: packets
// per sample of x and y): the frame the temporal x2 passes through on the first pass.
__global__ __launch_bounds__(256) void copy_first_frame_kernel(const uint4* __restrict__ x, uint4* __restrict__ y,
                                                              int64_t packets, int64_t xs, int64_t ys) {
  const int64_t n = blockIdx.y;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < packets; i += (int64_t)gridDim.x * 256)
    y[n * ys + i] = x[n * xs + i];
}

// ---------------------------------------------------------------- the convolution kernel
//
// Tiles never straddle a frame: a tile is BM consecutive positions of one frame t (the last
// tile of a frame is ragged), so every tap reads one source frame -- frame t + dt - 2 of x,
// a cache frame, or none -- chosen once per tap in scalar registers.
// Operands move with raw buffer instructions over 128-bit descriptors. A descriptor spans
// exactly the source frame, so a row above or below the frame falls outside it and reads
// zeros; a row left or right of the frame gets an offset past every descriptor and reads
// zeros too. Padding costs two VALU instructions per row and tap and no branch.
// A stage is one tap x 32 channels: its BN weight rows and BM position rows (64 bytes each)
// go to one of NS LDS stage buffers. Stage order, causal: (frame tap dt, row tap dh), then
// the 32-channel chunk, then the column tap dw -- the order of conv_slab_kernel, so that
// both accumulate every output in the same sequence; phases: tap, then chunk.
// - Weights (and, unfused, position rows) move global -> LDS with buffer_load_dwordx4 ...
//   lds, NS-1 stages ahead, waited for with counted vmcnt.
// - Fused GroupNorm: the position rows are loaded into VGPRs one stage ahead, activated by
//   activate_packet() (the code gn_silu_apply runs, so the result is bitwise that of
//   apply-then-convolve) and stored to the same swizzled LDS slots.
// - Each stage runs two MFMA phases of 16 channels; the next phase's fragments are read
//   from LDS between the current phase's MFMAs, so LDS latency never stalls the matrix pipe.
// - One barrier per stage, between its two phases: it publishes stage s+1 (each wave has
//   waited for its own moves of it) and retires stage s-1's buffer, which the moves of stage
//   s+NS-1 then overwrite.
// The 16-byte chunks of each 64-byte row sit at physical chunk = logical ^ g(row), g(row) =
// ((row >> 1) & 3) ^ ((row >> 3) & 1): fragment reads (32 consecutive rows, one logical
// chunk) are conflict free for 8 and for 16 lanes per LDS cycle.
// Per output the accumulation order is fixed -- the stage order above, then 16 channels at
// a time -- and independent of T, the tile and the launch: results are deterministic, and
// a pass split along T gives the same bits.

constexpr int kPK = 32;                  // channels per stage
constexpr int kStages = 4;               // LDS stage buffers (a fifth measured no faster)


// 16 bytes per lane from r at voff + soff into LDS at lds + 16 * lane (lds wave-uniform).
__device__ __forceinline__ void dma16(Rsrc r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ uint4 load16(Rsrc r, uint32_t voff, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}


template <int BM, int BN, int WGM, int WGN, int NS, int MODE, int FUSE>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void conv_kernel(ConvParams p) {
  constexpr bool RMS = FUSE == kFuseRms;
  constexpr int NW = WGM * WGN;
  constexpr int TAPS = MODE == kPhase ? 4 : MODE == kTime ? 3 : 27;
  constexpr int INNER = MODE == kCausal || MODE == kHead ? 3 : 1;   // taps sharing a channel chunk in a row
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM * 32 * WGM == BM && TN * 32 * WGN == BN, "tile shape");
  static_assert(BM % 16 == 0 && BN % 16 == 0 && NS >= 4, "pipeline shape");
  static_assert(MODE != kTime || !FUSE, "the temporal x2 reads its input as it is");
  constexpr int ROWB = kPK * 2;                      // bytes per LDS row
  constexpr int STAGE = (BN + BM) * ROWB;
  constexpr int IA = BN / 16, IB = BM / 16;          // 1 KB moves (16 rows) per stage
  constexpr int IAW = (IA + NW - 1) / NW, IBW = (IB + NW - 1) / NW;

  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches

  // Workgroup -> tile. Workgroups are dealt to the 8 XCDs round-robin; renumber so that
  // each XCD works through a contiguous run of tiles (neighbouring tiles share input rows
  // and weights in that XCD's L2). Order inside a run: N tile, phase, tile of the frame,
  // frame, sample.
  int tile;
  {
    const int bid = blockIdx.x, nb = p.nblocks;
    const int xcd = bid & 7, idx = bid >> 3, q = nb >> 3, r = nb & 7;
    tile = xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
  }
  const int ntile = tile % p.tiles_n;
  tile /= p.tiles_n;
  int phase = 0;
  if (MODE == kPhase) {
    phase = tile & 3;
    tile >>= 2;
  }
  const int mt = tile % p.tiles_f;
  tile /= p.tiles_f;
  const int t = tile % p.T;
  const int n = tile / p.T;
  const int pa = phase >> 1, pb = phase & 1;

  const int C = p.C, K = p.K, H = p.H, W = p.W, T = p.T;
  const int HW = H * W;
  const uint32_t frame_bytes = (uint32_t)HW * C * 2;
  const int kpt = C / kPK;                           // stages per tap
  const int KS = TAPS * kpt;
  // This lane moves logical chunk lc of row (16 qi + (lane >> 2)); (row & 15) = lane >> 2.
  const int lc = (lane & 3) ^ ((lane >> 3) & 3) ^ ((lane >> 5) & 1);

  const Rsrc wr = make_rsrc(p.w + (MODE == kPhase ? (int64_t)phase * K * 4 * C : 0),
                            (uint32_t)K * TAPS * C * 2);
  uint32_t wvo[IAW];
#pragma unroll
  for (int j = 0; j < IAW; ++j) {
    int k = ntile * BN + (wave + NW * j) * 16 + (lane >> 2);
    if (k > K - 1) k = K - 1;                        // columns past K: computed, never stored
    wvo[j] = ((uint32_t)k * TAPS * C + lc * 8) * 2;
  }
  // Position rows this lane moves: byte offset in the frame, and which row / column
  // neighbours exist.
  uint32_t pvo[IBW];
  int ppos[RMS ? IBW : 1];                           // RMS: the row's position in the frame
  bool wl[IBW], wrt[IBW], hu[IBW], hd[IBW];
#pragma unroll
  for (int j = 0; j < IBW; ++j) {
    int pos = mt * BM + (wave + NW * j) * 16 + (lane >> 2);
    if (pos > HW - 1) pos = HW - 1;                  // rows past the frame: computed, never stored
    const int h_ = pos / W, w_ = pos - h_ * W;
    pvo[j] = ((uint32_t)pos * C + lc * 8) * 2;
    if constexpr (RMS) ppos[j] = pos;
    wl[j] = w_ > 0;
    wrt[j] = w_ < W - 1;
    hu[j] = h_ > 0;
    hd[j] = h_ < H - 1;
  }

  // Per-tap state of the position cursor (uniform): the source frame's descriptor, whether
  // it is a frame of x (fused: activate), the tap's byte offset within the frame and its
  // row and column offsets dh, dw (0 = one before).
  Rsrc prs = make_rsrc(p.x, 0);
  Rsrc rrs = make_rsrc(p.x, 0);                      // RMS: the source frame's rstd (x frames only)
  bool from_x = false;
  int pdelta = 0, rdelta = 0, tdh = 1, tdw = 1;
  auto set_tap = [&](int tap) {
    int dt, dh, dw;
    if (MODE == kPhase) {
      dt = 2;
      dh = (tap >> 1) + pa;                          // row offset u + a - 1, stored +1
      dw = (tap & 1) + pb;
    } else if (MODE == kTime) {
      dt = tap;                                      // 3 x 1 x 1: the same position
      dh = 1;
      dw = 1;
    } else {
      dt = tap / 9;
      dh = (tap / 3) % 3;
      dw = tap % 3;
    }
    const int tf = t + dt - 2;
    from_x = tf >= 0;
    if (tf >= 0)
      prs = make_rsrc(p.x + (MODE == kTime ? (int64_t)n * p.Tx + p.x0 + tf : (int64_t)n * T + tf) * HW * C,
                      frame_bytes);
    else if (p.cache)
      prs = make_rsrc(p.cache + ((int64_t)n * 2 + tf + 2) * HW * C, frame_bytes);
    else
      prs = make_rsrc(p.x, 0);                       // no cache: zero frames
    if constexpr (RMS)
      rrs = tf >= 0 ? make_rsrc(p.rstd + ((int64_t)n * T + tf) * HW, (uint32_t)HW * 8) : make_rsrc(p.rstd, 0);
    pdelta = ((dh - 1) * W + (dw - 1)) * C * 2;
    rdelta = (dh - 1) * W + (dw - 1);
    tdh = dh;
    tdw = dw;
  };

  uint4 held[FUSE ? IBW : 1];
  bool hact[FUSE ? IBW : 1];                         // fused: activate (a row of x in the frame)
  double hr[RMS ? IBW : 1];                          // RMS: the held row's rstd

  // Stage cursors (uniform): inner tap i, channel chunk ch, tap group o; stage (o, ch, i)
  // is tap o * INNER + i over channels ch * 32 .. ch * 32 + 31.
  auto next_stage = [&](int& i, int& ch, int& o) {
    if (++i == INNER) {
      i = 0;
      if (++ch == kpt) {
        ch = 0;
        ++o;
      }
    }
  };
  // Weight rows of stage s -> LDS (calls come in stage order): channels tap * C + ch * 32
  // of every row.
  int wi = 0, wch = 0, wo = 0;
  auto issue_w = [&](int s) {
    char* lw = smem + (s % NS) * STAGE;
    const uint32_t soff = ((uint32_t)(wo * INNER + wi) * C + wch * kPK) * 2;
#pragma unroll
    for (int j = 0; j < IAW; ++j) {
      const int qi = wave + NW * j;
      if (IA % NW == 0 || qi < IA) dma16(wr, wvo[j], soff, lw + qi * 1024);
    }
    next_stage(wi, wch, wo);
  };
  // Position rows of the cursor's stage -> LDS (unfused) or VGPRs (fused); then the cursor
  // moves to the next stage.
  int pstage = 0, pi = 0, pch = 0, po = 0;
  set_tap(0);
  auto issue_p = [&]() {
    char* lp = smem + (pstage % NS) * STAGE + BN * ROWB;
    const int d = pdelta + pch * kPK * 2;
#pragma unroll
    for (int j = 0; j < IBW; ++j) {
      const int qi = wave + NW * j;
      if (IB % NW == 0 || qi < IB) {
        const bool okw = (tdw != 0 || wl[j]) && (tdw != 2 || wrt[j]);
        const uint32_t voff = okw ? pvo[j] + (uint32_t)d : kOOB;
        if (FUSE) {
          held[j] = load16(prs, voff, 0);
          hact[j] = from_x && okw && (tdh != 0 || hu[j]) && (tdh != 2 || hd[j]);
          if constexpr (RMS) {
            // the row's rstd (positions outside the frame, which are never activated, read 0)
            const uint32_t roff = okw ? (uint32_t)(ppos[j] + rdelta) * 8u : kOOB;
            const auto rv = __builtin_amdgcn_raw_buffer_load_b64(rrs, roff, 0, 0);
            hr[j] = __builtin_bit_cast(double, rv);
          }
        } else {
          dma16(prs, voff, 0, lp + qi * 1024);
        }
      }
    }
    ++pstage;
    next_stage(pi, pch, po);
    if ((INNER > 1 || pch == 0) && po < TAPS / INNER) set_tap(po * INNER + pi);
  };
  // Fused: per-channel fp64 affines of this sample (GroupNorm), or the fp64 gains (RMS, the
  // affine of a row being gain * its rstd), in LDS after the stage buffers; the held rows of
  // stage s are activated into its buffer (calls come in stage order). The bias of the
  // tile's BN output channels follows.
  double* tab = reinterpret_cast<double*>(smem + NS * STAGE);
  float* lbias = reinterpret_cast<float*>(smem + NS * STAGE + (FUSE ? C * 16 : 0));
  int ci = 0, cch = 0, co = 0;
  auto commit_p = [&](int s) {
    if (!FUSE) return;
    const int c0 = cch * kPK + lc * 8;
    next_stage(ci, cch, co);
    char* lp = smem + (s % NS) * STAGE + BN * ROWB;
    Affine a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i].s = tab[2 * (c0 + i)];
      a[i].b = tab[2 * (c0 + i) + 1];
    }
#pragma unroll
    for (int j = 0; j < IBW; ++j) {
      const int qi = wave + NW * j;
      if (IB % NW == 0 || qi < IB) {
        uint4 v = held[j];
        if (hact[j]) {
          if constexpr (RMS) {
            // rms_silu's affine: (double) gain * rstd, no shift
            Affine ar[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              ar[i].s = a[i].s * hr[j];
              ar[i].b = 0.0;
            }
            v = activate_packet(v, ar);
          } else {
            v = activate_packet(v, a);
          }
        }
        *reinterpret_cast<uint4*>(lp + qi * 1024 + lane * 16) = v;
      }
    }
  };

  // Fragment reads: operand rows are (multiple of 32) + (lane & 31), so g(row) comes from
  // lane bits 0-3; lanes 32-63 take the second logical chunk of a 16-channel phase.
  const int wm = wave % WGM, wn = wave / WGM;
  const int gl = ((lane >> 1) & 3) ^ ((lane >> 3) & 1);
  const int rd = (lane & 31) * ROWB;
  const int ck0 = ((lane >> 5) ^ gl) << 4;
  const int ck1 = ((2 + (lane >> 5)) ^ gl) << 4;
  auto load_frags = [&](bf16x8 (&a)[TN], bf16x8 (&b)[TM], int buf, int kk) {
    const char* base = smem + buf * STAGE + rd + (kk ? ck1 : ck0);
#pragma unroll
    for (int i = 0; i < TN; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(base + (wn * WTN + i * 32) * ROWB);
#pragma unroll
    for (int j = 0; j < TM; ++j)
      b[j] = *reinterpret_cast<const bf16x8*>(base + (BN + wm * WTM + j * 32) * ROWB);
  };

  f32x16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  auto mfmas = [&](const bf16x8 (&a)[TN], const bf16x8 (&b)[TM]) {
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  };
  // One phase: its MFMAs with the next phase's fragment reads between the first few, so
  // the reads complete long before the next phase needs them.
  constexpr int NRD = TN + TM, NMF = TN * TM;
  constexpr int PAIRS = NRD < NMF ? NRD : NMF;
  auto interleave = [&]() {
#pragma unroll
    for (int r = 0; r < PAIRS; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // one DS read
    }
    if (NRD > PAIRS) __builtin_amdgcn_sched_group_barrier(0x100, NRD - PAIRS, 0);
    if (NMF > PAIRS) __builtin_amdgcn_sched_group_barrier(0x008, NMF - PAIRS, 0);
  };
  // Fewest moves any wave issues per stage: weights only (DW), and with unfused position
  // rows (DMIN). A wave waiting until at most DMIN * j of its moves are in flight has
  // completed all but (at most) its last j stages.
  constexpr int DW = IA / NW;
  constexpr int DMIN = DW + IB / NW;

  // Prologue: stage 0 published; the weights (unfused: and positions) of the next NS-2
  // stages in flight; fused, the position rows of stage 1 in flight to VGPRs. KS >= NS
  // always (C >= 64).
  BiasStage<BN> bias;
  bias.issue(p, ntile, tid);                         // before any move: the waits below cover it
  if (FUSE) {
    if constexpr (RMS) {
      for (int c = tid; c < C; c += 64 * NW) {
        tab[2 * c] = (double)p.gamma[c];
        tab[2 * c + 1] = 0.0;
      }
    } else {
      const int cg = C / p.groups;
      for (int c = tid; c < C; c += 64 * NW) {
        const Affine a = channel_affine(p.stats, p.gamma, p.beta, p.eps, p.groups, cg, n, c);
        tab[2 * c] = a.s;
        tab[2 * c + 1] = a.b;
      }
    }
#pragma unroll
    for (int s = 0; s < NS - 2; ++s) issue_w(s);
    issue_p();                                       // stage 0
    wait_vm<0>();
    bias.commit(lbias, tid);
    __syncthreads();                                 // affine table and bias visible
    commit_p(0);
    issue_p();                                       // stage 1
    issue_w(NS - 2);
    wait_lgkm0();
  } else {
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) {
      issue_w(s);
      issue_p();
    }
    wait_vm<DMIN * (NS - 2)>();
    bias.commit(lbias, tid);
    wait_lgkm0();
  }
  stage_barrier();
  bf16x8 a0[TN], b0[TM], a1[TN], b1[TM];
  load_frags(a0, b0, 0, 0);
  int buf = 0;
  for (int s = 0; s < KS - 1; ++s) {
    load_frags(a1, b1, buf, 1);
    mfmas(a0, b0);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    if (FUSE) {
      // Everything before the last weight moves (of stage s+NS-2) has completed: the held
      // rows of stage s+1, and the weights of stage s+1.
      if (s + NS - 2 < KS)
        wait_vm<DW>();
      else
        wait_vm<0>();
      commit_p(s + 1);
      wait_lgkm0();
    } else {
      // Own moves of stage s+1 complete (those of the stages after it may stay in flight).
      if (s + NS - 1 <= KS)
        wait_vm<DMIN * (NS - 3)>();
      else
        wait_vm<0>();                                // the last few stages: wait for all
    }
    stage_barrier();                                 // stage s+1 published, s-1 retired
    if (FUSE) {
      if (s + 2 < KS) issue_p();                     // stage s+2
      if (s + NS - 1 < KS) issue_w(s + NS - 1);
    } else if (s + NS - 1 < KS) {
      issue_w(s + NS - 1);
      issue_p();                                     // stage s+NS-1
    }
    __builtin_amdgcn_sched_barrier(0);
    buf = buf == NS - 1 ? 0 : buf + 1;
    load_frags(a0, b0, buf, 0);
    mfmas(a1, b1);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
  }
  load_frags(a1, b1, buf, 1);
  mfmas(a0, b0);
  mfmas(a1, b1);

  if constexpr (MODE == kHead) {
    store_tile<MODE, TN, TM, WTM, WTN>(acc, p, n, (int64_t)t * HW + mt * BM, (int64_t)(t + 1) * HW,
                                       ntile * BN + wn * WTN, wm, lane, phase, lbias + wn * WTN);
  } else if (K % 8 == 0) {                           // rows of y 16-byte aligned
    static_assert(NW * 32 * WTN * 4 + NW * 64 * 16 <= NS * STAGE, "epilogue staging fits the stages");
    const Sums sums = store_tile_staged<MODE, TN, TM, WTM, WTN, true>(
        acc, p, n, t, mt * BM, ntile * BN + wn * WTN, wm, lane, phase, lbias + wn * WTN,
        smem + wave * (32 * WTN * 4));
    if (MODE == kCausal && p.nws)
      next_stats_partials<NW, WGM, WTN, BN>(p, n, t, mt, ntile, wave, lane, sums,
                                            reinterpret_cast<double*>(smem + NW * 32 * WTN * 4));
  } else if constexpr (MODE != kTime) {               // the temporal x2 needs K % 16 == 0
    store_tile<MODE, TN, TM, WTM, WTN>(acc, p, n, (int64_t)t * HW + mt * BM, (int64_t)(t + 1) * HW,
                                       ntile * BN + wn * WTN, wm, lane, phase, lbias + wn * WTN);
  }
}

// ---------------------------------------------------------------- slab form
//
// The unfused causal convolution and the upsample phases, for K > 128. Tiles and epilogue
// as in conv_kernel. Stage order: causal, (frame tap dt, row tap dh), then the 32-channel
// chunk, then the column tap dw (conv_kernel's order, so that both accumulate every output
// in the same sequence); phases, row tap u, then the chunk, then the column tap v. The
// INNER column taps of a group (3 causal, 2 per phase) read the same input rows shifted by
// one position each: the input rows of column tap i for output positions m0 .. m0 + BM - 1
// are positions m0 + (dh - 1) W + c0 + i + r of the source frame, c0 = -1 (causal) or
// b - 1 (phase (a, b)), so one slab of BM + INNER - 1 rows starting at m0 + (dh - 1) W + c0
// serves all of them, tap i reading the BM-row window that starts at slab row i. A third
// (causal) or half (phases) of the position rows of conv_kernel move.
// - Padding: slab rows above or below the frame read zeros through the frame's descriptor
//   (a negative offset wraps past it). The window row of an output in column 0 for a tap
//   with column offset -1, or in column W - 1 for offset +1, holds the neighbour across the
//   image-row edge; such lanes read a 64-byte zero row of LDS instead (one address select
//   per fragment, chosen per tile).
// - Pipeline: NS weight stage buffers, weights moved L = NS - 1 stages ahead. The slab of
//   group G moves in INNER parts, each right after the weights of one stage of group G - 1,
//   into one of NSL slab buffers (enough that a buffer is retired before it is refilled).
//   "Iteration" i issues the weights of stage i + L and then SPW slab blocks per wave (a
//   wave without a block of that part moves an out-of-range row: zeros into a dummy LDS
//   block, no memory access), so every wave has the same moves in flight. Iterations
//   -L .. -1 form the prologue. The wait before the barrier of iteration s lets exactly the
//   moves issued after the weights of stage s + 1 stay in flight (vmcnt counts in issue
//   order): a constant while every iteration moves its slab blocks, counted per iteration
//   in the last TAILG groups.
// - A steady-state iteration is one basic block (cursors advance by selects, the frame
//   descriptor is a select of precomputed ones), so the iteration's moves and the next
//   stage's fragment reads are scheduled between the second phase's MFMAs: with one wave
//   per SIMD nothing else would keep the matrix pipe busy while the wave issues them.
// - Slab row r of the swizzled LDS layout keeps g(r) of conv_kernel; the window rows of a
//   fragment are (multiple of 32) + (lane & 31) + i, and g only reads row bits 1-3, so each
//   (i, 16-channel phase) has one per-lane chunk offset. Any 8 consecutive rows hit 8
//   distinct 16-byte bank groups, whatever the window offset.
constexpr int kSlabStages = 4;           // weight stage buffers of the slab kernel

__host__ __device__ constexpr int slab_inner(int mode) { return mode == kPhase ? 2 : (mode == kTime || mode == kWino) ? 1 : 3; }

// Slab buffers: slab G starts moving L + INNER stages before stage INNER G and its buffer
// must have been retired (after stage INNER (G - NSL) + INNER - 1): INNER NSL >= L + 2 INNER.
__host__ __device__ constexpr int slab_bufs(int ns, int inner) {
  return (ns - 1 + 2 * inner + inner - 1) / inner;
}

template <int BM, int BN, int NS, int MODE>
constexpr int slab_lds_bytes() {
  return NS * BN * kPK * 2 +
         slab_bufs(NS, slab_inner(MODE)) * ((BM + slab_inner(MODE) - 1 + 15) / 16) * 1024 + 1024 + 64 +
         BN * 4;
}

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 31].
__device__ __forceinline__ void wait_vm_n(int n) {
  switch (n) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<1>(); break;
    case 2: wait_vm<2>(); break;
    case 3: wait_vm<3>(); break;
    case 4: wait_vm<4>(); break;
    case 5: wait_vm<5>(); break;
    case 6: wait_vm<6>(); break;
    case 7: wait_vm<7>(); break;
    case 8: wait_vm<8>(); break;
    case 9: wait_vm<9>(); break;
    case 10: wait_vm<10>(); break;
    case 11: wait_vm<11>(); break;
    case 12: wait_vm<12>(); break;
    case 13: wait_vm<13>(); break;
    case 14: wait_vm<14>(); break;
    case 15: wait_vm<15>(); break;
    case 16: wait_vm<16>(); break;
    case 17: wait_vm<17>(); break;
    case 18: wait_vm<18>(); break;
    case 19: wait_vm<19>(); break;
    case 20: wait_vm<20>(); break;
    case 21: wait_vm<21>(); break;
    case 22: wait_vm<22>(); break;
    case 23: wait_vm<23>(); break;
    case 24: wait_vm<24>(); break;
    case 25: wait_vm<25>(); break;
    case 26: wait_vm<26>(); break;
    case 27: wait_vm<27>(); break;
    case 28: wait_vm<28>(); break;
    case 29: wait_vm<29>(); break;
    case 30: wait_vm<30>(); break;
    default: wait_vm<31>(); break;
  }
}

// EPI: the instantiation with the epilogue's extra work -- the next RMS norm (causal) or the
// DupUp3D shortcut (phases). A separate one, so that the plain convolution keeps its
// spill-free register allocation and its stores need no wait for the extra loads.
template <int BM, int BN, int WGM, int WGN, int NS, int MODE, bool EPI = false>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void conv_slab_kernel(ConvParams p) {
  static_assert(MODE == kCausal || MODE == kPhase || MODE == kTime || MODE == kWino, "slab modes");
  constexpr bool TEMPORAL = MODE == kTime || MODE == kWino;   // 3 frame taps, one row, no column taps
  constexpr int INNER = slab_inner(MODE);            // column taps per group
  constexpr int TAPS = MODE == kPhase ? 4 : TEMPORAL ? 3 : 27;
  constexpr int NW = WGM * WGN, L = NS - 1, NSL = slab_bufs(NS, INNER);
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM * 32 * WGM == BM && TN * 32 * WGN == BN, "tile shape");
  static_assert(NS >= 4 && INNER * NSL >= L + 2 * INNER, "pipeline depth");
  constexpr int ROWB = kPK * 2;                      // bytes per LDS row
  constexpr int WSTAGE = BN * ROWB;                  // weight rows of one stage
  constexpr int SMOVES = (BM + INNER - 1 + 15) / 16; // 16-row moves per slab
  constexpr int SLAB = SMOVES * 1024;
  constexpr int SLABS = NS * WSTAGE;                 // slab buffers follow the weight stages
  constexpr int DUMMY = SLABS + NSL * SLAB;          // 1 KB written by the dummy moves
  constexpr int ZROW = DUMMY + 1024;                 // 64 zero bytes
  constexpr int LBIAS = ZROW + 64;                   // the workgroup's BN biases
  static_assert(LBIAS + BN * 4 == slab_lds_bytes<BM, BN, NS, MODE>(), "LDS layout");
  constexpr int IA = BN / 16, DW = IA / NW;          // weight moves per wave and stage
  constexpr int SP = (SMOVES + INNER - 1) / INNER;   // slab moves of each part but the last
  constexpr int SPL = SMOVES - (INNER - 1) * SP;     // ... and of the last
  constexpr int SPW = (SP + NW - 1) / NW;            // slab moves per wave and part
  static_assert(IA % NW == 0 && SPL >= 0, "moves per wave");
  constexpr int STEADY = SPW + (L - 2) * (DW + SPW); // moves after those of stage s + 1
  static_assert(STEADY + DW <= 31, "wait range");
  constexpr int TAILG = (L + 2 * INNER - 1) / INNER; // last groups, waited for exactly

  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches

  // Workgroup -> tile, XCD-aware as in conv_kernel. Order inside a run: N tile, phase,
  // frame, tile of the frame, sample: tiles at one position of consecutive frames share two
  // of their three source frames, and with frames fastest they run at the same time (the
  // upsample block's conv 4.53 -> 4.40 ms; with a 4 MB L2 per XCD the gain is small).
  int tile;
  {
    const int bid = blockIdx.x, nb = p.nblocks;
    const int xcd = bid & 7, idx = bid >> 3, q = nb >> 3, r = nb & 7;
    tile = xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
  }
  const int ntile = tile % p.tiles_n;
  tile /= p.tiles_n;
  int phase = 0;
  if (MODE == kPhase) {
    phase = tile & 3;
    tile >>= 2;
  }
  const int t = tile % p.T;
  tile /= p.T;
  const int mt = tile % p.tiles_f;
  const int n = tile / p.tiles_f;
  const int pa = phase >> 1, pb = phase & 1;

  const int C = p.C, K = p.K, H = p.H, W = p.W, T = p.T;
  const int HW = H * W;
  const uint32_t frame_bytes = (uint32_t)HW * C * 2;
  const int kpt = C / kPK;
  const int NG = (TAPS / INNER) * kpt;               // groups, INNER stages each
  const int KS = INNER * NG;
  const int pos0 = mt * BM;
  const int c0 = MODE == kPhase ? pb - 1 : TEMPORAL ? 0 : -1;   // column offset of slab row 0
  // This lane moves logical chunk lc of row (16 qi + (lane >> 2)); (row & 15) = lane >> 2.
  const int lc = (lane & 3) ^ ((lane >> 3) & 3) ^ ((lane >> 5) & 1);

  const int64_t wsel = MODE == kPhase ? (int64_t)phase * K * 4 * C
                       : MODE == kWino ? (int64_t)(n / p.wino_n) * K * 3 * C : 0;
  const Rsrc wr = make_rsrc(p.w + wsel, (uint32_t)K * TAPS * C * 2);
  uint32_t wvo[DW];
#pragma unroll
  for (int j = 0; j < DW; ++j) {
    int k = ntile * BN + (wave + NW * j) * 16 + (lane >> 2);
    if (k > K - 1) k = K - 1;                        // columns past K: computed, never stored
    wvo[j] = ((uint32_t)k * TAPS * C + lc * 8) * 2;
  }
  // Slab rows this lane moves in part k: slab row 16 q + lane / 4 with
  // q = k * SP + wave + NW * j, i.e. position pos0 + c0 + row (plus (dh - 1) W per group).
  uint32_t svo[INNER][SPW];
#pragma unroll
  for (int k = 0; k < INNER; ++k)
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int64_t pos = (int64_t)pos0 + c0 + 16 * (k * SP + wave + NW * j) + (lane >> 2);
      svo[k][j] = (uint32_t)((pos * C + lc * 8) * 2);
    }
  // Slab moves of iteration i (i >= -L) per wave: SPW (real or dummy) while group
  // (i + L) / INNER + 1 exists.
  auto slab_moves = [&](int i) __attribute__((always_inline)) -> int {
    return (i + L) / INNER + 1 < NG ? SPW : 0;
  };

  // Weight cursor (tap o * INNER + i, chunk ch) and slab cursor (group: tap row o, chunk).
  // Both advance by selects.
  int wi = 0, wch = 0, wo = 0, wbi = 0;
  auto issue_w = [&]() __attribute__((always_inline)) {
    char* lw = smem + wbi * WSTAGE;
    const uint32_t soff = __builtin_amdgcn_readfirstlane(((wo * INNER + wi) * C + wch * kPK) * 2);
#pragma unroll
    for (int j = 0; j < DW; ++j) dma16(wr, wvo[j], soff, lw + (wave + NW * j) * 1024);
    wbi = wbi == NS - 1 ? 0 : wbi + 1;
    const bool wrap_i = wi == INNER - 1, wrap_c = wrap_i && wch == kpt - 1;
    wi = wrap_i ? 0 : wi + 1;
    wch = wrap_c ? 0 : (wrap_i ? wch + 1 : wch);
    wo += wrap_c ? 1 : 0;
  };
  // Descriptors of the source frames of frame taps dt = 0, 1, 2: frame t + dt - 2 of x, a
  // cache frame, or (no cache) zeros. The phases read frame t only. The temporal x2 reads
  // x from frame x0 on, Tx frames per sample; the Winograd products read frames t .. t + 2
  // of the Tx = T + 2 transformed frames of P (x0 = 2), which always exist.
  const int64_t xf0 = TEMPORAL ? (int64_t)n * p.Tx + p.x0 : (int64_t)n * T;
  const Rsrc frs2 = make_rsrc(p.x + (xf0 + t) * HW * C, frame_bytes);
  Rsrc frs0 = frs2, frs1 = frs2;
  if (MODE == kCausal || TEMPORAL) {
    if (t >= 2 || MODE == kWino)
      frs0 = make_rsrc(p.x + (xf0 + t - 2) * HW * C, frame_bytes);
    else if (p.cache)
      frs0 = make_rsrc(p.cache + ((int64_t)n * 2 + t) * HW * C, frame_bytes);
    else
      frs0 = make_rsrc(p.x, 0);
    if (t >= 1 || MODE == kWino)
      frs1 = make_rsrc(p.x + (xf0 + t - 1) * HW * C, frame_bytes);
    else if (p.cache)
      frs1 = make_rsrc(p.cache + ((int64_t)n * 2 + t + 1) * HW * C, frame_bytes);
    else
      frs1 = make_rsrc(p.x, 0);
  }
  Rsrc srs = frs0;
  int sdelta = 0, gch = 0, go = 0, gbuf = 0;
  auto issue_s = [&](auto part_c) __attribute__((always_inline)) {
    constexpr int PART = decltype(part_c)::value;
    if (PART == 0) {
      // dh: the row tap, stored + 1 (causal dh; phase u + a; the temporal x2's one row).
      const int dt = MODE == kPhase ? 2 : TEMPORAL ? go : go / 3;
      const int dh = MODE == kPhase ? go + pa : TEMPORAL ? 1 : go - 3 * dt;
      const Rsrc r0 = frs0, r1 = frs1, r2 = frs2;     // values: a select of lvalues would
      srs = dt == 0 ? r0 : dt == 1 ? r1 : r2;        // select their addresses
      sdelta = ((dh - 1) * W * C + gch * kPK) * 2;
    }
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int q = wave + NW * j;
      const bool real = q < (PART < INNER - 1 ? SP : SPL);
      dma16(srs, real ? svo[PART][j] + (uint32_t)sdelta : kOOB, 0,
            real ? smem + SLABS + gbuf * SLAB + (PART * SP + q) * 1024 : smem + DUMMY);
    }
    if (PART == INNER - 1) {
      gbuf = gbuf == NSL - 1 ? 0 : gbuf + 1;
      const bool wrap = gch == kpt - 1;
      gch = wrap ? 0 : gch + 1;
      go += wrap ? 1 : 0;
    }
  };
  // Moves issued after the weights of stage s + 1 by the end of iteration last (>= s + 1 - L).
  auto in_flight_after = [&](int s, int last) __attribute__((always_inline)) -> int {
    int c = 0;
    for (int i = s + 1 - L; i <= last; ++i) {
      if (i > s + 1 - L && i + L < KS) c += DW;
      c += slab_moves(i);
    }
    return c;
  };

  // Fragment reads. A (weights): rows (multiple of 32) + (lane & 31) of the stage buffer, as
  // in conv_kernel. B (positions): window rows (multiple of 32) + (lane & 31) + i of the
  // slab, or the zero row for an output at the image-row edge the tap crosses.
  const int wm = wave % WGM, wn = wave / WGM;
  const int gl = ((lane >> 1) & 3) ^ ((lane >> 3) & 1);
  const int rd = (lane & 31) * ROWB;
  const int ck0 = ((lane >> 5) ^ gl) << 4;
  const int ck1 = ((2 + (lane >> 5)) ^ gl) << 4;
  int bo[INNER][2];
#pragma unroll
  for (int i = 0; i < INNER; ++i) {
    const int r = (lane & 31) + i;
    const int g = ((r >> 1) & 3) ^ ((r >> 3) & 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) bo[i][kk] = r * ROWB + (((2 * kk + (lane >> 5)) ^ g) << 4);
  }
  bool edge[INNER][TM];
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int pos = pos0 + wm * WTM + 32 * j + (lane & 31);
    const int w_ = pos % W;
#pragma unroll
    for (int i = 0; i < INNER; ++i) {
      const int coff = c0 + i;                       // the tap's column offset
      edge[i][j] = (coff == -1 && w_ == 0) || (coff == 1 && w_ == W - 1);
    }
  }
  auto load_frags = [&](auto i_c, bf16x8 (&a)[TN], bf16x8 (&b)[TM], int wbuf, int sbuf,
                        int kk) __attribute__((always_inline)) {
    constexpr int IV = decltype(i_c)::value;
    const char* abase = smem + wbuf * WSTAGE + rd + (kk ? ck1 : ck0);
#pragma unroll
    for (int i = 0; i < TN; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(abase + (wn * WTN + i * 32) * ROWB);
    const int boff = bo[IV][kk];
    const char* bbase = smem + SLABS + sbuf * SLAB + boff;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const char* ptr = bbase + (wm * WTM + j * 32) * ROWB;
      if (edge[IV][j]) ptr = smem + ZROW + (boff & 63);
      b[j] = *reinterpret_cast<const bf16x8*>(ptr);
    }
  };

  f32x16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  auto mfmas = [&](const bf16x8 (&a)[TN], const bf16x8 (&b)[TM]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  };
  constexpr int NRD = TN + TM, NMF = TN * TM;
  constexpr int PAIRS = NRD < NMF ? NRD : NMF;
  auto interleave = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < PAIRS; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // one DS read
    }
    if (NRD > PAIRS) __builtin_amdgcn_sched_group_barrier(0x100, NRD - PAIRS, 0);
    if (NMF > PAIRS) __builtin_amdgcn_sched_group_barrier(0x008, NMF - PAIRS, 0);
  };
  // Steady-state second phase: the next stage's fragment reads first (the next phase's
  // first MFMA needs them), then the iteration's moves (needed L stages later), each placed
  // after one MFMA. The reads come first in program order too: a move writes LDS, so the
  // scheduler would not lift a read above it.
  constexpr int NV = DW + SPW;
  constexpr int PD = NRD < NMF ? NRD : NMF;
  constexpr int RM = NMF - PD;
  constexpr int PV = NV < RM ? NV : RM;
  auto interleave_moves = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < PD; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // one DS read
    }
    if (NRD > PD) __builtin_amdgcn_sched_group_barrier(0x100, NRD - PD, 0);
#pragma unroll
    for (int r = 0; r < PV; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);     // one global -> LDS move
    }
    if (NV > PV) __builtin_amdgcn_sched_group_barrier(0x010, NV - PV, 0);
    if (RM > PV) __builtin_amdgcn_sched_group_barrier(0x008, RM - PV, 0);
  };

  // Prologue: the bias load, slab 0, then iterations -L .. -1 (weights of stage u = i + L,
  // part u % INNER of slab u / INNER + 1); once the weights of stage 0 (and so everything
  // issued before them) have landed, the bias and the zero row are written to LDS and
  // published with stage 0.
  BiasStage<BN> bias;
  bias.issue(p, ntile, tid);
  if (tid < 4) *reinterpret_cast<uint4*>(smem + ZROW + 16 * tid) = make_uint4(0, 0, 0, 0);
  issue_s(IC<0>{});
  if constexpr (INNER > 1) issue_s(IC<1>{});
  if constexpr (INNER > 2) issue_s(IC<2>{});
  static_assert(L >= 3 && L <= 5 && INNER <= 3, "prologue");
  issue_w();
  issue_s(IC<0 % INNER>{});
  issue_w();
  issue_s(IC<1 % INNER>{});
  issue_w();
  issue_s(IC<2 % INNER>{});
  if constexpr (L > 3) {
    issue_w();
    issue_s(IC<3 % INNER>{});
  }
  if constexpr (L > 4) {
    issue_w();
    issue_s(IC<4 % INNER>{});
  }
  wait_vm_n(in_flight_after(-1, -1));
  bias.commit(reinterpret_cast<float*>(smem + LBIAS), tid);
  wait_lgkm0();
  stage_barrier();
  bf16x8 a0[TN], b0[TM], a1[TN], b1[TM];
  load_frags(IC<0>{}, a0, b0, 0, 0, 0);
  int wbuf = 0, sbuf = 0;
  // Iteration s: second phase's fragments of stage s, first-phase MFMAs; wait for the own
  // moves of stage s + 1; barrier: stage s + 1 published, stage s - 1 retired; first
  // phase's fragments of stage s + 1 and the moves of iteration s during the second-phase
  // MFMAs.
  auto step = [&](auto i_c, auto steady_c, int s) __attribute__((always_inline)) {
    constexpr int IV = decltype(i_c)::value;
    constexpr int NXT = IV == INNER - 1 ? 0 : IV + 1;
    load_frags(i_c, a1, b1, wbuf, sbuf, 1);
    mfmas(a0, b0);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    if (decltype(steady_c)::value)
      wait_vm<STEADY>();
    else
      wait_vm_n(in_flight_after(s, s - 1));
    stage_barrier();
    wbuf = wbuf == NS - 1 ? 0 : wbuf + 1;
    if (IV == INNER - 1) sbuf = sbuf == NSL - 1 ? 0 : sbuf + 1;
    if constexpr (decltype(steady_c)::value) {
      load_frags(IC<NXT>{}, a0, b0, wbuf, sbuf, 0);
      // the weights of stage s + L and the slab blocks both exist
      issue_w();
      issue_s(IC<(IV + L) % INNER>{});
    } else {
      if (s + L < KS) issue_w();
      if ((s + L) / INNER + 1 < NG) issue_s(IC<(IV + L) % INNER>{});
      __builtin_amdgcn_sched_barrier(0);
      load_frags(IC<NXT>{}, a0, b0, wbuf, sbuf, 0);
    }
    mfmas(a1, b1);
    if constexpr (decltype(steady_c)::value)
      interleave_moves();
    else
      interleave();
    __builtin_amdgcn_sched_barrier(0);
  };
  // Groups before the last TAILG (s <= KS - INNER TAILG - 1 < KS - INNER - L): iteration s
  // moves the weights of stage s + L and a slab part, and so did every iteration before it.
  static_assert(INNER * TAILG >= L + INNER, "tail");
  for (int g = 0; g < NG - TAILG; ++g) {
    step(IC<0>{}, IC<1>{}, INNER * g);
    if constexpr (INNER > 1) step(IC<1>{}, IC<1>{}, INNER * g + 1);
    if constexpr (INNER > 2) step(IC<2>{}, IC<1>{}, INNER * g + 2);
  }
  for (int g = NG - TAILG; g < NG - 1; ++g) {
    step(IC<0>{}, IC<0>{}, INNER * g);
    if constexpr (INNER > 1) step(IC<1>{}, IC<0>{}, INNER * g + 1);
    if constexpr (INNER > 2) step(IC<2>{}, IC<0>{}, INNER * g + 2);
  }
  // the last group: all its stages but the last (that one follows, without moves)
  if constexpr (INNER > 1) step(IC<0>{}, IC<0>{}, KS - INNER);
  if constexpr (INNER > 2) step(IC<1>{}, IC<0>{}, KS - 2);
  load_frags(IC<INNER - 1>{}, a1, b1, wbuf, sbuf, 1);
  mfmas(a0, b0);
  mfmas(a1, b1);

  static_assert(NW * 32 * WTN * 4 <= SLABS, "epilogue staging fits the weight stages");
  const float* lb = reinterpret_cast<const float*>(smem + LBIAS) + wn * WTN;
  // The next RMS norm in the epilogue (LDS: the waves' staging areas, the row sums, then
  // each wave's parked outputs, NI x 64 lanes x 16 bytes).
  bool rms_done = false;
  if constexpr (MODE == kCausal && EPI) {
    if (p.act) {
      constexpr int RSUM = NW * 32 * WTN * 4, PARK = RSUM + 2 * NW * 32 * 8;
      constexpr int NIP = 32 / (64 / (WTN / 8));
      constexpr int GAIN = PARK + NW * NIP * 64 * 16;
      static_assert(GAIN + NW * WTN * 4 <= SLABS + NSL * SLAB, "epilogue LDS");
      store_tile_rms<TN, TM, WTM, WTN, WGM, WGN>(acc, p, n, t, pos0, ntile * BN + wn * WTN, wm, wn, lane, lb,
                                                 smem + wave * (32 * WTN * 4),
                                                 reinterpret_cast<double*>(smem + RSUM),
                                                 smem + PARK + wave * (NIP * 64 * 16),
                                                 reinterpret_cast<float*>(smem + GAIN) + wave * WTN);
      rms_done = true;
    }
  }
  if (rms_done) {
  } else if constexpr (MODE == kWino) {
    store_tile_f32<TN, TM, WTM, WTN>(acc, p, n, t, pos0, ntile * BN + wn * WTN, wm, lane,
                                     smem + wave * (32 * WTN * 4));
  } else {
    // K % 8 == 0 (the host takes this kernel only then): rows of y are 16-byte aligned. With
    // the staged epilogue as the only one, the accumulators reach LDS straight from the
    // accumulator registers; a second epilogue that adds to them in vector registers would
    // make the compiler copy all of them out of the accumulator file and spill.
    const Sums sums = store_tile_staged<MODE, TN, TM, WTM, WTN, MODE == kPhase && EPI>(
        acc, p, n, t, pos0, ntile * BN + wn * WTN, wm, lane, phase, lb, smem + wave * (32 * WTN * 4));
    static_assert(NW * 32 * WTN * 4 + NW * 64 * 16 <= SLABS + NSL * SLAB, "statistics area");
    if (MODE == kCausal && p.nws)
      next_stats_partials<NW, WGM, WTN, BN>(p, n, t, mt, ntile, wave, lane, sums,
                                            reinterpret_cast<double*>(smem + NW * 32 * WTN * 4));
  }
}

// ---------------------------------------------------------------- the output head
//
// The head convolution has K = 12 output channels: as an implicit GEMM every input row it
// stages feeds only 12 (padded 16) MACs per channel, so the generic tile above spends its
// time moving operands. This kernel keeps the operands where the reuse is instead:
// - Weights live in registers for the whole kernel. Wave w of NW owns the 32-channel chunk
//   w and holds its 27 weight fragments (the A operand of v_mfma_f32_16x16x32_bf16: 16
//   output channels x 32 input channels, rows 12-15 zero). The waves' partial sums are
//   added through LDS when an output frame is complete. Eight waves (two per SIMD) cover
//   C = 256, four cover C = 128.
// - A workgroup owns two output rows h0, h0 + 1 and 48 columns (3 segments of 16) for every
//   frame, and streams the input frames of P = cat(cache, x) once: frame p feeds output
//   frames p - dt, dt = 0..2, held in a ring of 3 accumulators per (output row, segment).
//   Output frame t is complete after input frame t + 2.
// - A unit of work is (input frame, input row h0 - 1 + r, r = 0..3, the wave's chunk): input
//   row h0 - 1 + r feeds output row h0 through row tap r and row h0 + 1 through row tap
//   r - 1. Its 50 input columns w0 - 1 .. w0 + 48 (64-byte rows) move global -> LDS with
//   buffer_load ... lds into the wave's own ring of 3 units, two units ahead; each wave waits
//   only for its own moves (counted vmcnt), so the ring needs no barrier.
// - The matrix work and the moves overlap (together they take only a little more cycles
//   than either alone), but together they draw enough power that the board lowers the
//   clock: energy per output is what bounds the kernel. Two output rows per workgroup stage
//   4 input rows per frame for 2 output rows, where one row per workgroup staged 3 for
//   each; the moves per output pixel drop by about a third. (The accumulators of 2 rows fit
//   the register file with 3 segments.)
// - The loop over a group of 3 frames (12 units) is unrolled so that a unit's ring slot, row
//   taps and accumulator slots are constants, every LDS read is a per-lane base (one per
//   column tap) plus an immediate, and the frame descriptors are built once per group.
// - The B operand of a column tap dw is the 16-row LDS window starting at row 16 s + dw:
//   one input row staged once serves all 3 column taps, both output rows and, through the
//   frame ring, all 3 frame taps. The 16-byte chunks of row r sit at chunk
//   logical ^ ((r >> 1) & 3): LDS serves a 16-byte read 8 lanes (128 bytes) at a time, and
//   any 8 consecutive rows then hit 8 distinct bank groups, whatever the window offset.
// - Raw-buffer loads over the input frame: rows above or below the frame and columns
//   outside [0, W) read zeros; without a cache the two zero frames are skipped.
// The epilogue adds the bias, clamps if asked, and writes the 2x2 depth-to-space video
// (channel k = 4c + 2dy + dx) as 4-byte pairs, 64 contiguous bytes per 16 columns.
typedef __attribute__((ext_vector_type(4))) float f32x4;
constexpr int kHeadSeg = 3;              // 16-column segments per workgroup (W = 624: 13 blocks)
constexpr int kHeadOut = 2;              // output rows per workgroup
constexpr int kHeadIn = kHeadOut + 2;    // input rows per frame (units)
constexpr int kHeadRows = 64;            // LDS rows per unit (50 used: 48 columns + 2 edges)
constexpr int kHeadMoves = kHeadRows / 16; // 1 KB moves per unit and wave
constexpr int kHeadRing = 3;             // units per wave in LDS (unit u in slot u % 3)

__host__ __device__ constexpr int head_lds_bytes(int nw) {
  return nw * kHeadRing * kHeadRows * 64 + nw * kHeadOut * kHeadSeg * 64 * 16 + 64;
}

template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void head_kernel(ConvParams p, int wblocks) {
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, g = lane >> 4;            // row in a 16-row window, channel group
  const int C = p.C, H = p.H, W = p.W, T = p.T;
  const int HW = H * W;
  const int HP = (H + kHeadOut - 1) / kHeadOut;      // row pairs
  const uint32_t frame_bytes = (uint32_t)HW * C * 2;
  constexpr int UNIT = kHeadRows * 64;               // bytes per unit in LDS
  char* ring = smem + wave * (kHeadRing * UNIT);
  f32x4* red = reinterpret_cast<f32x4*>(smem + NW * kHeadRing * UNIT);   // [NW][out row][seg][64]
  float* sbias = reinterpret_cast<float*>(red + NW * kHeadOut * kHeadSeg * 64);

  // Workgroup -> (n, column block, row pair), row pairs fastest and XCD-aware: each XCD
  // takes a contiguous run, so the workgroups it runs at once are consecutive row pairs of
  // one column block, and the input rows two neighbouring pairs share are read from L2.
  int blk;
  {
    const int bid = blockIdx.x, nb = p.nblocks;
    const int xcd = bid & 7, idx = bid >> 3, q = nb >> 3, r = nb & 7;
    blk = xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
  }
  const int h0 = (blk % HP) * kHeadOut;
  const int wb = (blk / HP) % wblocks;
  const int n = blk / (wblocks * HP);
  const int w0 = wb * (16 * kHeadSeg);

  // Weight fragments of this wave's chunk, one per tap.
  bf16x8 a[27];
#pragma unroll
  for (int tap = 0; tap < 27; ++tap) {
    const int ch = wave * 32 + 8 * g;
    if (j < 12)
      a[tap] = *reinterpret_cast<const bf16x8*>(p.w + ((int64_t)j * 27 + tap) * C + ch);
    else
      a[tap] = bf16x8{};
  }
  if (tid < 16) sbias[tid] = (p.bias && tid < 12) ? p.bias[tid] : 0.0f;

  // The moves of a unit: move i writes LDS rows 16 i .. 16 i + 15; lane l fills row
  // 16 i + l / 4 (column w0 - 1 + row) at physical chunk l & 3, i.e. it loads logical chunk
  // (l & 3) ^ ((row >> 1) & 3) = (l & 3) ^ ((l >> 3) & 3). Rows past 49 and columns outside
  // the frame get kOOB (zeros, no memory access); adding a row offset keeps them out of range.
  uint32_t pvo[kHeadMoves];
  {
    const int lc = (lane & 3) ^ ((lane >> 3) & 3);
#pragma unroll
    for (int i = 0; i < kHeadMoves; ++i) {
      const int r = 16 * i + (lane >> 2), col = w0 - 1 + r;
      pvo[i] = (r < 16 * kHeadSeg + 2 && col >= 0 && col < W)
                   ? ((uint32_t)col * C + wave * 32 + lc * 8) * 2 : kOOB;
    }
  }

  f32x4 acc[kHeadOut][3][kHeadSeg];
#pragma unroll
  for (int o = 0; o < kHeadOut; ++o)
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
      for (int s = 0; s < kHeadSeg; ++s) acc[o][r][s] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Source frame pf of P = cat(cache, x): a descriptor over it (no records: zeros).
  auto frame_rsrc = [&](int pf) {
    if (pf >= 2 && pf < T + 2) return make_rsrc(p.x + ((int64_t)n * T + pf - 2) * HW * C, frame_bytes);
    if (pf < 2 && p.cache) return make_rsrc(p.cache + ((int64_t)n * 2 + pf) * HW * C, frame_bytes);
    return make_rsrc(p.x, 0);
  };
  // Byte offset of input row h0 - 1 + r in a frame (row -1 wraps, rows past H - 1 run past
  // the frame: both out of range, zeros).
  uint32_t rowoff[kHeadIn];
#pragma unroll
  for (int r = 0; r < kHeadIn; ++r) rowoff[r] = (uint32_t)((h0 - 1 + r) * W * C * 2);
  // Unit (frame, input row R) into ring slot SL.
  auto issue = [&](const Rsrc& rs, auto R_, auto SL_) __attribute__((always_inline)) {
    constexpr int R = decltype(R_)::value, SL = decltype(SL_)::value;
    char* dst = ring + SL * UNIT;
#pragma unroll
    for (int i = 0; i < kHeadMoves; ++i) dma16(rs, pvo[i] + rowoff[R], 0, dst + i * 1024);
  };
  // Window of column tap dw in segment s: rows 16 s + dw + j at chunk g ^ ((row >> 1) & 3);
  // 16 s does not change row bits 1-2, so per lane one base per dw, plus s KB.
  uint32_t woff[3];
#pragma unroll
  for (int dw = 0; dw < 3; ++dw) {
    const int r = dw + j;
    woff[dw] = (uint32_t)(ring - smem) + r * 64 + ((g ^ ((r >> 1) & 3)) << 4);
  }
  // Unit of frame pf = 3 q + U, input row R (in ring slot SL): for each output row o with
  // row tap dh = R - o in 0..2, 3 column taps x 3 frame taps per segment into the
  // accumulator slots of output frames pf - dt (slot (U - dt) mod 3). The windows of segment
  // s + 1 are read while segment s's MFMAs run (two buffers of 3 fragments).
  auto compute_unit = [&](auto U_, auto R_, auto SL_) __attribute__((always_inline)) {
    constexpr int U = decltype(U_)::value;
    constexpr int R = decltype(R_)::value, SL = decltype(SL_)::value;
    bf16x8 bb[2][3];
#pragma unroll
    for (int dw = 0; dw < 3; ++dw) bb[0][dw] = *reinterpret_cast<const bf16x8*>(smem + woff[dw] + SL * UNIT);
#pragma unroll
    for (int sg = 0; sg < kHeadSeg; ++sg) {
      if (sg + 1 < kHeadSeg) {
#pragma unroll
        for (int dw = 0; dw < 3; ++dw)
          bb[(sg + 1) & 1][dw] = *reinterpret_cast<const bf16x8*>(smem + woff[dw] + SL * UNIT + (sg + 1) * 1024);
      }
#pragma unroll
      for (int dw = 0; dw < 3; ++dw)
#pragma unroll
        for (int o = 0; o < kHeadOut; ++o) {
          const int dh = R - o;
          if (dh < 0 || dh > 2) continue;            // constant after unrolling
#pragma unroll
          for (int dt = 0; dt < 3; ++dt) {
            const int slot = ((U - dt) % 3 + 3) % 3;
            acc[o][slot][sg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[dt * 9 + dh * 3 + dw], bb[sg & 1][dw],
                                                                       acc[o][slot][sg], 0, 0, 0);
          }
        }
    }
  };

  // Output frame t (accumulator slot S) is complete: add the waves' partial sums through LDS
  // (one buffer: a barrier before the writes as well as after them), then wave
  // o * kHeadSeg + s writes output row h0 + o, segment s; the slot is cleared for output
  // frame t + 3. Slots of frames before 0 only collect the taps that reach before the first
  // frame: they are cleared without a store.
  auto retire = [&](int t, auto S_) __attribute__((always_inline)) {
    constexpr int S = decltype(S_)::value;
    if (t < 0) {
#pragma unroll
      for (int o = 0; o < kHeadOut; ++o)
#pragma unroll
        for (int sg = 0; sg < kHeadSeg; ++sg) acc[o][S][sg] = f32x4{0.f, 0.f, 0.f, 0.f};
      return;
    }
    stage_barrier();                                 // every wave has read the previous frame's sums
#pragma unroll
    for (int o = 0; o < kHeadOut; ++o)
#pragma unroll
      for (int sg = 0; sg < kHeadSeg; ++sg) {
        red[((wave * kHeadOut + o) * kHeadSeg + sg) * 64 + lane] = acc[o][S][sg];
        acc[o][S][sg] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    // LDS writes complete, then the barrier: not __syncthreads, whose fence would also
    // wait for the moves in flight.
    wait_lgkm0();
    stage_barrier();
    // (output row, segment) part `part` is added and stored by wave part % NW (with 4 waves,
    // each takes two of the 6 parts).
    constexpr int PARTS = kHeadOut * kHeadSeg;
#pragma unroll
    for (int part0 = 0; part0 < PARTS; part0 += NW) {
      const int part = part0 + wave;
      if (t >= T || g >= 3 || part >= PARTS) continue;
      const int o = part / kHeadSeg, sg = part % kHeadSeg;
      const int h = h0 + o;
      const int col = w0 + 16 * sg + j;
      if (h < H && col < W) {
        f32x4 v = red[part * 64 + lane];
#pragma unroll
        for (int q = 1; q < NW; ++q) v += red[(q * PARTS + part) * 64 + lane];
        float ov[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ov[r] = v[r] + sbias[4 * g + r];
          if (p.clamp) ov[r] = fminf(fmaxf(ov[r], -1.0f), 1.0f);
        }
        const int64_t W2 = 2 * (int64_t)W;
        const int64_t base = (((int64_t)n * 3 + g) * T + t) * (2 * (int64_t)H) * W2 + 2 * (int64_t)col;
        *reinterpret_cast<uint32_t*>(p.y + base + (2 * h) * W2) = pack_bf16x2(ov[0], ov[1]);
        *reinterpret_cast<uint32_t*>(p.y + base + (2 * h + 1) * W2) = pack_bf16x2(ov[2], ov[3]);
      }
    }
  };

  // Frames in groups of three (12 units); without a cache the first group skips the compute
  // of the two zero frames (a separate copy of the group, so both keep static registers).
  // Frames past T + 1 read zeros and store nothing. Units go in order (frame, input row);
  // the moves of the next two units are in flight while one computes.
  const int groups3 = (T + 2 + 2) / 3;
  {
    const Rsrc f0 = frame_rsrc(0);
    issue(f0, IC<0>{}, IC<0>{});
    issue(f0, IC<1>{}, IC<1>{});
  }
  auto group = [&](int q, auto SKIP_) __attribute__((always_inline)) {
    constexpr bool SKIP = decltype(SKIP_)::value != 0;
    // frames 3q .. 3q + 3: the group's own and the first of the next (units run 2 ahead)
    const Rsrc fr0 = frame_rsrc(3 * q), fr1 = frame_rsrc(3 * q + 1), fr2 = frame_rsrc(3 * q + 2),
               fr3 = frame_rsrc(3 * q + 3);
    auto step = [&](auto K_) __attribute__((always_inline)) {
      constexpr int K = decltype(K_)::value;
      constexpr int U = K / kHeadIn, R = K % kHeadIn;
      constexpr int KN = K + 2, UN = KN / kHeadIn, RN = KN % kHeadIn;   // the unit issued after this one
      wait_vm<kHeadMoves>();                         // this wave's moves of this unit landed
      if (!SKIP || U == 2) compute_unit(IC<U>{}, IC<R>{}, IC<K % kHeadRing>{});
      const Rsrc& rn = UN == 0 ? fr0 : UN == 1 ? fr1 : UN == 2 ? fr2 : fr3;
      issue(rn, IC<RN>{}, IC<KN % kHeadRing>{});     // into the slot the unit before this one used
      if (R == kHeadIn - 1) retire(3 * q + U - 2, IC<(U + 1) % 3>{});
    };
    step(IC<0>{});
    step(IC<1>{});
    step(IC<2>{});
    step(IC<3>{});
    step(IC<4>{});
    step(IC<5>{});
    step(IC<6>{});
    step(IC<7>{});
    step(IC<8>{});
    step(IC<9>{});
    step(IC<10>{});
    step(IC<11>{});
  };
  if (p.cache)
    group(0, IC<0>{});
  else
    group(0, IC<1>{});
  for (int q = 1; q < groups3; ++q) group(q, IC<0>{});
  wait_vm<0>();
}

// ---------------------------------------------------------------- Winograd F(4x4, 3x3)
//
// The causal 3x3x3 convolution as 36 per-component causal 3-tap temporal products (binding.cpp
// page: prepare()'s F(4x4,3x3) weight transform, whose 36 components each keep the 3 frame
// taps; Decoder::conv: input transform, the per-component products, an epilogue forming the
// output with bias and residual). Three launches:
//  1. wino_input_kernel: V = B^T d B of every tile's 6 x 6 patch in every frame of
//     P = cat(cache, x), in fp32 from the bf16 input, rounded once to bf16, component-major:
//     V[36][N][T + 2][TH x TW tiles][C].
//  2. conv_slab_kernel<.., kWino>: per component, M[t][tile][k] = sum_{dt, c} U[k][dt][c] V[t +
//     dt][tile][c] -- the slab kernel's temporal mode over the 36 N "samples", fp32 out.
//  3. wino_output_kernel: Y = A^T M A per tile and channel in fp32, + bias + residual, one
//     rounding to bf16, the pixels inside the frame stored NDHWC.
// The transforms use the interpolation points 0, 1, -1, 2, -2 and infinity of the page's G.

// Input transform of 6 values (one row or column of a patch): B^T d.
__device__ __forceinline__ void wino_bt(const float d[6], float o[6]) {
  o[0] = 4.0f * d[0] - 5.0f * d[2] + d[4];
  o[1] = -4.0f * d[1] - 4.0f * d[2] + d[3] + d[4];
  o[2] = 4.0f * d[1] - 4.0f * d[2] - d[3] + d[4];
  o[3] = -2.0f * d[1] - d[2] + 2.0f * d[3] + d[4];
  o[4] = 2.0f * d[1] - d[2] - 2.0f * d[3] + d[4];
  o[5] = 4.0f * d[1] - 5.0f * d[3] + d[5];
}

// One thread: channels 2 c2, 2 c2 + 1 of one tile of frame f (blockIdx.y) of sample n
// (blockIdx.z); grid-stride over tiles x channel pairs, channel pairs fastest (coalesced).
__global__ __launch_bounds__(256) void wino_input_kernel(const uint32_t* __restrict__ x,
                                                         const uint32_t* __restrict__ cache,
                                                         uint32_t* __restrict__ v, int N, int T, int H,
                                                         int W, int cp, int TW, int64_t TP) {
  const int f = blockIdx.y, n = blockIdx.z;
  const int64_t fsz = (int64_t)H * W * cp;           // dwords per frame
  const uint32_t* src = f >= 2 ? x + ((int64_t)n * T + f - 2) * fsz
                               : (cache ? cache + ((int64_t)n * 2 + f) * fsz : nullptr);
  const int64_t cstride = (int64_t)N * (T + 2) * TP * cp;   // dwords between components
  uint32_t* dst = v + ((int64_t)n * (T + 2) + f) * TP * cp;
  const int64_t items = TP * cp;
  for (int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x; it < items; it += (int64_t)gridDim.x * 256) {
    const int c2 = (int)(it % cp);
    const int64_t tile = it / cp;
    const int ti = (int)(tile / TW), tj = (int)(tile - (int64_t)ti * TW);
    float d0[6][6], d1[6][6];
#pragma unroll
    for (int r = 0; r < 6; ++r) {
      const int yy = 4 * ti - 1 + r;
#pragma unroll
      for (int q = 0; q < 6; ++q) {
        const int xx = 4 * tj - 1 + q;
        uint32_t u = 0;
        if (src && yy >= 0 && yy < H && xx >= 0 && xx < W) u = src[((int64_t)yy * W + xx) * cp + c2];
        d0[r][q] = bf16_lo(u);
        d1[r][q] = bf16_hi(u);
      }
    }
    // rows: e[r][b] = (B^T d[r][:])[b]; then columns: V[a][b] = (B^T e[:][b])[a]
    float e0[6][6], e1[6][6];
#pragma unroll
    for (int r = 0; r < 6; ++r) {
      wino_bt(d0[r], e0[r]);
      wino_bt(d1[r], e1[r]);
    }
#pragma unroll
    for (int b = 0; b < 6; ++b) {
      float c0v[6], c1v[6], o0[6], o1[6];
#pragma unroll
      for (int r = 0; r < 6; ++r) {
        c0v[r] = e0[r][b];
        c1v[r] = e1[r][b];
      }
      wino_bt(c0v, o0);
      wino_bt(c1v, o1);
#pragma unroll
      for (int a = 0; a < 6; ++a) dst[(int64_t)(a * 6 + b) * cstride + tile * cp + c2] = pack_bf16x2(o0[a], o1[a]);
    }
  }
}

// One thread: channels 4 k4 .. 4 k4 + 3 of one tile of output frame t (blockIdx.y) of sample
// n (blockIdx.z). Rows of A^T M A first along the component's column index b, then along a.
__global__ __launch_bounds__(256) void wino_output_kernel(const float* __restrict__ m, const float* __restrict__ bias,
                                                          const uint16_t* __restrict__ res, uint16_t* __restrict__ y,
                                                          int N, int T, int H, int W, int K, int TW, int64_t TP) {
  const int t = blockIdx.y, n = blockIdx.z;
  const int kq = K / 4;
  const int64_t cstride = (int64_t)N * T * TP * K;   // floats between components
  const float* src = m + ((int64_t)n * T + t) * TP * K;
  const int64_t fbase = ((int64_t)n * T + t) * H * W;
  const int64_t items = TP * kq;
  for (int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x; it < items; it += (int64_t)gridDim.x * 256) {
    const int k4 = (int)(it % kq);
    const int64_t tile = it / kq;
    const int ti = (int)(tile / TW), tj = (int)(tile - (int64_t)ti * TW);
    float o[4][4][4];                                // [row][column][channel]
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[a][b][e] = 0.0f;
#pragma unroll
    for (int a = 0; a < 6; ++a) {
      float4 mm[6];
#pragma unroll
      for (int b = 0; b < 6; ++b)
        mm[b] = *reinterpret_cast<const float4*>(src + (int64_t)(a * 6 + b) * cstride + tile * K + 4 * k4);
      // s[x] = (A^T row x) . mm, per channel
      float sx[4][4];
      const float* q0 = &mm[0].x;
      const float* q1 = &mm[1].x;
      const float* q2 = &mm[2].x;
      const float* q3 = &mm[3].x;
      const float* q4 = &mm[4].x;
      const float* q5 = &mm[5].x;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sx[0][e] = q0[e] + q1[e] + q2[e] + q3[e] + q4[e];
        sx[1][e] = q1[e] - q2[e] + 2.0f * q3[e] - 2.0f * q4[e];
        sx[2][e] = q1[e] + q2[e] + 4.0f * q3[e] + 4.0f * q4[e];
        sx[3][e] = q1[e] - q2[e] + 8.0f * q3[e] - 8.0f * q4[e] + q5[e];
      }
      // o[row][x] += A^T[row][a] s[x]; A^T column a: (1,0,0,0), (1,1,1,1), (1,-1,1,-1),
      // (1,2,4,8), (1,-2,4,-8), (0,0,0,1)
      const float c1 = a == 0 ? 0.0f : a == 1 ? 1.0f : a == 2 ? -1.0f : a == 3 ? 2.0f : a == 4 ? -2.0f : 0.0f;
      const float c2 = a == 0 ? 0.0f : a == 1 ? 1.0f : a == 2 ? 1.0f : a == 3 ? 4.0f : a == 4 ? 4.0f : 0.0f;
      const float c3 = a == 0 ? 0.0f : a == 1 ? 1.0f : a == 2 ? -1.0f : a == 3 ? 8.0f : a == 4 ? -8.0f : 1.0f;
      const float c0 = a == 5 ? 0.0f : 1.0f;
#pragma unroll
      for (int xx = 0; xx < 4; ++xx)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[0][xx][e] += c0 * sx[xx][e];
          o[1][xx][e] += c1 * sx[xx][e];
          o[2][xx][e] += c2 * sx[xx][e];
          o[3][xx][e] += c3 * sx[xx][e];
        }
    }
    float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (bias) {
      const float4 b4 = *reinterpret_cast<const float4*>(bias + 4 * k4);
      bv[0] = b4.x;
      bv[1] = b4.y;
      bv[2] = b4.z;
      bv[3] = b4.w;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int yy = 4 * ti + r;
#pragma unroll
      for (int xx = 0; xx < 4; ++xx) {
        const int xc = 4 * tj + xx;
        if (yy < H && xc < W) {
          const int64_t off = (fbase + (int64_t)yy * W + xc) * K + 4 * k4;
          float vv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) vv[e] = o[r][xx][e] + bv[e];
          if (res) {
            const uint2 rr = *reinterpret_cast<const uint2*>(res + off);
            vv[0] += bf16_lo(rr.x);
            vv[1] += bf16_hi(rr.x);
            vv[2] += bf16_lo(rr.y);
            vv[3] += bf16_hi(rr.y);
          }
          *reinterpret_cast<uint2*>(y + off) = make_uint2(pack_bf16x2(vv[0], vv[1]), pack_bf16x2(vv[2], vv[3]));
        }
      }
    }
  }
}

// ---------------------------------------------------------------- host side

typedef void (*ConvFn)(ConvParams);

struct TileCfg {
  int bm, bn;
  ConvFn fn;
  int lds;
  int threads;
  bool rms_epilogue;   // the kernel applies the next RMS norm in its epilogue when p.act is set
  bool shortcut;       // a phase kernel adds the DupUp3D shortcut when p.sc is set
  bool slab;           // conv_slab_kernel (else conv_kernel)
};

template <int BM, int BN, int WGM, int WGN, int NS, int MODE, int FUSE>
static TileCfg make_cfg(int c) {
  TileCfg t;
  t.bm = BM;
  t.bn = BN;
  t.fn = conv_kernel<BM, BN, WGM, WGN, NS, MODE, FUSE>;
  t.lds = NS * (BM + BN) * kPK * 2 + (FUSE ? c * 16 : 0) + BN * 4;
  t.threads = 64 * WGM * WGN;
  t.rms_epilogue = false;
  t.shortcut = true;
  t.slab = false;
  return t;
}

template <int BM, int BN, int WGM, int WGN, int MODE, bool EPI = false>
static TileCfg make_slab_cfg() {
  TileCfg t;
  t.bm = BM;
  t.bn = BN;
  t.fn = conv_slab_kernel<BM, BN, WGM, WGN, kSlabStages, MODE, EPI>;
  t.lds = slab_lds_bytes<BM, BN, kSlabStages, MODE>();
  t.threads = 64 * WGM * WGN;
  t.rms_epilogue = MODE == kCausal && EPI;
  t.shortcut = MODE != kPhase || EPI;
  t.slab = true;
  return t;
}

// Candidate tiles for N-tile width bn (largest M tile first).
template <int MODE, int FUSE>
static int candidates(int bn, int c, TileCfg* out) {
  int n = 0;
  if constexpr (MODE == kWino) {                    // K > 128 only: the slab tiles
    out[n++] = make_slab_cfg<256, 256, 2, 2, MODE>();
    out[n++] = make_slab_cfg<224, 256, 1, 4, MODE>();
  } else {
    switch (bn) {
      case 256:
        // conv_kernel: 8 waves, two per SIMD: one wave's barrier and LDS waits hide under the
        // other's MFMAs (measured faster than 4-wave 224/192-row tiles, latent block 0.74 vs
        // 0.81 ms). The slab kernel: 4 waves of 128 x 128 (accumulators in AGPRs), a third
        // fewer fragment reads per MFMA; its moves are scheduled between MFMAs, so one wave
        // per SIMD keeps the matrix pipe fed (latent block 0.600 vs 0.632 ms with 8 waves).
        if constexpr ((MODE == kCausal || MODE == kPhase || MODE == kTime) && !FUSE) {
          out[n++] = make_slab_cfg<256, 256, 2, 2, MODE>();
          out[n++] = make_slab_cfg<224, 256, 1, 4, MODE>();
        } else {
          out[n++] = make_cfg<256, 256, 2, 4, kStages, MODE, FUSE>(c);
        }
        break;
      case 128:
        out[n++] = make_cfg<256, 128, 2, 2, kStages, MODE, FUSE>(c);
        break;
      case 64:
        out[n++] = make_cfg<256, 64, 4, 1, kStages, MODE, FUSE>(c);
        break;
      default:
        out[n++] = make_cfg<256, 32, 4, 1, kStages, MODE, FUSE>(c);
        break;
    }
  }
  return n;
}

// Pick the M tile that minimises (waves of workgroups over 256 CUs) x (work per tile).
// Tiles do not straddle frames: hw positions per frame, frames frames in all.
template <int MODE, int FUSE>
static TileCfg choose_tile(int64_t hw, int64_t frames, int k, int c, int64_t groups_of_tiles) {
  const int bn = k > 128 ? 256 : k > 64 ? 128 : k > 32 ? 64 : 32;
  TileCfg cand[4];
  int nc = candidates<MODE, FUSE>(bn, c, cand);
  if constexpr ((MODE == kCausal || MODE == kPhase) && !FUSE) {
    // the slab kernel has only the staged epilogue (16-byte rows of y): K % 8 != 0 takes
    // the generic tile
    if (bn == 256 && k % 8 != 0) {
      cand[0] = make_cfg<256, 256, 2, 4, kStages, MODE, FUSE>(c);
      nc = 1;
    }
  }
  TileCfg best = cand[0];
  double best_cost = 1e300;
  for (int i = 0; i < nc; ++i) {
    const int64_t tiles_m = (hw + cand[i].bm - 1) / cand[i].bm * frames;
    const int64_t tiles = tiles_m * ((k + bn - 1) / bn) * groups_of_tiles;
    const double cost = (double)((tiles + 255) / 256) * cand[i].bm;
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = cand[i];
    }
  }
  return best;
}

static bool launch_conv(const TileCfg& cfg, ConvParams& p, int64_t n_samples, int phases,
                        hipStream_t stream, const char* fn) {
  p.tiles_n = (p.K + cfg.bn - 1) / cfg.bn;
  const int64_t tiles_f = ((int64_t)p.H * p.W + cfg.bm - 1) / cfg.bm;
  const int64_t nb = tiles_f * p.T * p.tiles_n * phases * n_samples;
  // A launch holds fewer than 2^32 work-items.
  if (tiles_f > (1 << 30) || nb * cfg.threads >= (int64_t)1 << 32) {
    set_error("%s: problem too large for one launch", fn);
    return false;
  }
  p.tiles_f = (int)tiles_f;
  p.nblocks = (int)nb;
  hipError_t e = hipFuncSetAttribute((const void*)cfg.fn, hipFuncAttributeMaxDynamicSharedMemorySize, cfg.lds);
  if (e != hipSuccess) {
    set_error("%s: cannot reserve %d bytes of LDS: %s", fn, cfg.lds, hipGetErrorString(e));
    return false;
  }
  void* args[] = {&p};
  e = hipLaunchKernel((const void*)cfg.fn, dim3((unsigned)nb), dim3(cfg.threads), args, cfg.lds, stream);
  if (e != hipSuccess) {
    set_error("%s: launch failed: %s", fn, hipGetErrorString(e));
    return false;
  }
  return launch_ok(fn);
}

// cache_out of a causal convolution over frames x0 .. x0 + T - 1 (T = d.t - x0) of x.
static bool launch_cache_out(const uint16_t* x, sgn_dims d, const uint16_t* cache_in,
                             const sgn_gn* fuse, uint16_t* cache_out, hipStream_t stream, int x0 = 0,
                             const double* rms_rstd = nullptr, const float* rms_gain = nullptr) {
  const int cp = (int)(d.c / 8);
  int rstep = 256 / cp;
  if (rstep < 1) rstep = 1;
  const int64_t hw = d.h * d.w;
  int64_t blocks = (hw + rstep * 16 - 1) / (rstep * 16);  // 16 rows per thread
  if (blocks > 2048) blocks = 2048;
  int64_t rows = (hw + blocks - 1) / blocks;
  rows = (rows + rstep - 1) / rstep * rstep;
  blocks = (hw + rows - 1) / rows;
  const bool act = fuse || rms_rstd;
  auto kern = act ? cache_out_kernel<true> : cache_out_kernel<false>;
  kern<<<dim3((unsigned)blocks, (unsigned)d.n, 2), 256, 0, stream>>>(
      reinterpret_cast<const uint4*>(x), reinterpret_cast<const uint4*>(cache_in),
      reinterpret_cast<uint4*>(cache_out), (int)d.t - x0, (int)d.t, x0, hw, cp, rstep, rows,
      fuse ? fuse->stats : nullptr, fuse ? fuse->gamma : rms_gain, fuse ? fuse->beta : nullptr,
      fuse ? (double)fuse->eps : 0.0, fuse ? fuse->groups : 1, fuse ? nullptr : rms_rstd);
  return launch_ok("cache_out");
}

// The shapes the convolution kernels take (no pointers involved).
static bool conv_shape_ok(sgn_dims d, int k, const char* fn) {
  if (!dims_ok(d, fn)) return false;
  if (d.c % 64 != 0 || d.c > kCMax) {
    set_error("%s: C=%lld must be a multiple of 64 and at most %d", fn, (long long)d.c, kCMax);
    return false;
  }
  if (k < 4 || k > 4096 || k % 4 != 0) {
    set_error("%s: K=%d must be a multiple of 4 in [4, 4096]", fn, k);
    return false;
  }
  if (d.t * d.h * d.w >= ((int64_t)1 << 40)) {
    set_error("%s: too many positions per sample", fn);
    return false;
  }
  // Operands are read through 32-bit buffer offsets within one frame (plus a row above and
  // below it): a frame of C channels must stay well under 2 GiB.
  if ((d.h + 2) * d.w * d.c * 2 >= ((int64_t)1 << 31)) {
    set_error("%s: a frame of H=%lld x W=%lld x C=%lld exceeds the 2 GiB frame limit", fn,
              (long long)d.h, (long long)d.w, (long long)d.c);
    return false;
  }
  // The epilogue writes (and reads the residual) through one descriptor per output frame:
  // H x W x K, or 2H x 2W x K for the upsample, also under 2 GiB.
  if (4 * d.h * d.w * (int64_t)k * 2 >= ((int64_t)1 << 31)) {
    set_error("%s: an output frame of 4 x H=%lld x W=%lld x K=%d exceeds the 2 GiB frame limit", fn,
              (long long)d.h, (long long)d.w, k);
    return false;
  }
  return true;
}

static bool conv_common_checks(const uint16_t* x, sgn_dims d, const uint16_t* w, int k,
                               uint16_t* y, const char* fn) {
  if (!conv_shape_ok(d, k, fn)) return false;
  if (!x || !w || !y) {
    set_error("%s: x, w and the output are required", fn);
    return false;
  }
  return true;
}

static int check_fuse(const sgn_gn* f, sgn_dims d, const char* fn) {
  if (!f) return SGN_OK;
  if (!f->stats || !f->gamma || !f->beta) {
    set_error("%s: fuse needs stats, gamma and beta", fn);
    return SGN_EINVAL;
  }
  if (f->groups <= 0 || d.c % f->groups != 0) {
    set_error("%s: fuse groups=%d must divide C=%lld", fn, f->groups, (long long)d.c);
    return SGN_EINVAL;
  }
  if (!(f->eps > 0.0f) || !isfinite(f->eps)) {
    set_error("%s: fuse eps must be a positive finite number", fn);
    return SGN_EINVAL;
  }
  if (d.c > 2048) {
    set_error("%s: fused GroupNorm supports C <= 2048", fn);
    return SGN_EINVAL;
  }
  if (((uintptr_t)f->stats & 7) || ((uintptr_t)f->gamma & 3) || ((uintptr_t)f->beta & 3)) {
    set_error("%s: fuse stats must be 8-byte, gamma/beta 4-byte aligned", fn);
    return SGN_EALIGN;
  }
  return SGN_OK;
}

}  // namespace sgn

using namespace sgn;

namespace sgn {

// The GroupNorm statistics of y requested by causal_conv3d_next_stats.
struct NextStats {
  int groups;
  double* stats;
  void* ws;
  size_t ws_bytes;
};

// Workspace of causal_conv3d_next_stats: the larger of its two paths (partial sums of the
// epilogue, sized for the smallest M tile; or gn_silu_stats over y).
static size_t next_stats_bytes(sgn_dims d, int k, int groups) {
  const int64_t tiles_f = (d.h * d.w + 223) / 224;
  const size_t fused = (size_t)d.n * groups * 2 * (size_t)(d.t * tiles_f) * sizeof(double);
  sgn_dims yd = d;
  yd.c = k;
  const size_t plain = gn_silu_stats_workspace(yd, groups);
  return fused > plain ? fused : plain;
}

// The RMS norm + SiLU of y requested by causal_conv3d_rms.
struct RmsOut {
  const float* gain;
  float eps;
  uint16_t* act;
};

// The RMS norm + SiLU a convolution applies to x in its operand load
// (causal_conv3d_rms_input): rstd per position of x from rms_silu_rstd, the gain.
struct RmsIn {
  const double* rstd;
  const float* gain;
};

// causal_conv3d_rms computes act in the epilogue for an unfused convolution whose one N
// tile holds all K channels (128 < K <= 256, the 224-row slab tile); y may then be NULL.
static bool rms_in_epilogue(int k, const sgn_gn* fuse) { return !fuse && k > 128 && k <= 256 && k % 8 == 0; }

static int causal_conv_impl(const char* fn, const uint16_t* x, sgn_dims d, const uint16_t* cache_in,
                            const uint16_t* w, int k, const float* bias, const uint16_t* residual,
                            const sgn_gn* fuse, uint16_t* y, uint16_t* cache_out, const NextStats* ns,
                            hipStream_t stream, const RmsOut* ro = nullptr, const RmsIn* ri = nullptr) {
  if (ri && (fuse || ro)) {
    set_error("%s: internal: an RMS-normalised input takes no GroupNorm and no RMS epilogue", fn);
    return SGN_EINVAL;
  }
  const bool rms_epi = ro && rms_in_epilogue(k, fuse);
  uint16_t* yo = y ? y : (rms_epi ? ro->act : nullptr);   // the conv's primary output
  if (!conv_common_checks(x, d, w, k, yo, fn)) return SGN_EINVAL;
  int rc = check_fuse(fuse, d, fn);
  if (rc) return rc;
  if (ri) {
    if (!ri->rstd || !ri->gain) {
      set_error("%s: rstd and gain are required", fn);
      return SGN_EINVAL;
    }
    if (d.c > 2048) {
      set_error("%s: the RMS norm in the operand load supports C <= 2048", fn);
      return SGN_EINVAL;
    }
    if (((uintptr_t)ri->rstd & 7) || ((uintptr_t)ri->gain & 3)) {
      set_error("%s: rstd must be 8-byte and gain 4-byte aligned", fn);
      return SGN_EALIGN;
    }
  }
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (cache_in && !aligned16(cache_in)) ||
      (residual && !aligned16(residual)) || (cache_out && !aligned16(cache_out)) ||
      (bias && !aligned16(bias))) {
    set_error("%s: tensors (and bias) must be 16-byte aligned", fn);
    return SGN_EALIGN;
  }
  const size_t xb = (size_t)(d.n * d.t * d.h * d.w * d.c) * 2;
  const size_t yb = (size_t)(d.n * d.t * d.h * d.w) * k * 2;
  if (ri) {
    const size_t rb = (size_t)(d.n * d.t * d.h * d.w) * 8, gb = (size_t)d.c * 4;
    const size_t cob = (size_t)(d.n * 2 * d.h * d.w * d.c) * 2;
    if (overlap(y, yb, ri->rstd, rb) || overlap(y, yb, ri->gain, gb) ||
        (cache_out && (overlap(cache_out, cob, ri->rstd, rb) || overlap(cache_out, cob, ri->gain, gb)))) {
      set_error("%s: an output overlaps rstd or gain", fn);
      return SGN_EALIAS;
    }
  }
  const size_t cb = (size_t)(d.n * 2 * d.h * d.w * d.c) * 2;
  const size_t wb = (size_t)k * 27 * d.c * 2;
  if (overlap(yo, yb, x, xb) || overlap(yo, yb, w, wb) || (cache_in && overlap(yo, yb, cache_in, cb)) ||
      (residual && overlap(yo, yb, residual, yb)) ||
      (cache_out && (overlap(cache_out, cb, x, xb) || overlap(cache_out, cb, yo, yb) ||
                     overlap(cache_out, cb, w, wb) ||
                     (cache_in && overlap(cache_out, cb, cache_in, cb)) ||
                     (residual && overlap(cache_out, cb, residual, yb))))) {
    set_error("%s: an output overlaps an input or the other output", fn);
    return SGN_EALIAS;
  }
  if (ro && ro->act != yo &&
      (overlap(ro->act, yb, x, xb) || overlap(ro->act, yb, w, wb) || overlap(ro->act, yb, yo, yb) ||
       (cache_in && overlap(ro->act, yb, cache_in, cb)) || (residual && overlap(ro->act, yb, residual, yb)) ||
       (cache_out && overlap(ro->act, yb, cache_out, cb)))) {
    set_error("%s: act overlaps an input or another output", fn);
    return SGN_EALIAS;
  }
  ConvParams p = {};
  p.x = x;
  p.cache = cache_in;
  p.w = w;
  p.bias = bias;
  p.res = residual;
  p.y = y;
  if (fuse) {
    p.stats = fuse->stats;
    p.gamma = fuse->gamma;
    p.beta = fuse->beta;
    p.eps = (double)fuse->eps;
    p.groups = fuse->groups;
  }
  p.T = (int)d.t;
  p.H = (int)d.h;
  p.W = (int)d.w;
  p.C = (int)d.c;
  p.K = k;
  p.mper = d.t * d.h * d.w;
  if (ri) {
    p.rstd = ri->rstd;
    p.gamma = ri->gain;
  }
  TileCfg cfg = fuse ? choose_tile<kCausal, kFuseGn>(d.h * d.w, d.t, k, p.C, d.n)
                : ri ? choose_tile<kCausal, kFuseRms>(d.h * d.w, d.t, k, p.C, d.n)
                     : choose_tile<kCausal, kFuseNone>(d.h * d.w, d.t, k, p.C, d.n);
  if (rms_epi)      // the same tile, in its instantiation with the RMS epilogue
    cfg = cfg.bm == 256 ? make_slab_cfg<256, 256, 2, 2, kCausal, true>() : make_slab_cfg<224, 256, 1, 4, kCausal, true>();
  if (rms_epi) {
    // y may be NULL here: only a kernel with the RMS epilogue (which never stores a NULL y)
    // may take this call.
    if (!cfg.rms_epilogue || cfg.bn < k) {
      set_error("%s: internal: the chosen tile cannot apply the RMS norm in its epilogue", fn);
      return SGN_EINVAL;
    }
    p.act = ro->act;
    p.rms_gain = ro->gain;
    p.rms_eps = (double)ro->eps;
  }
  // Statistics of y from the epilogue when its lanes hold whole 8-channel slices of one group
  // inside one N tile; otherwise from gn_silu_stats over y after the convolution.
  const int ncg = ns ? k / ns->groups : 0;
  const bool in_epilogue = ns && k % 8 == 0 && ncg % 8 == 0 && cfg.bn % ncg == 0;
  if (in_epilogue) {
    p.nws = static_cast<double*>(ns->ws);
    p.ngroups = ns->groups;
    p.ncg = ncg;
  }
  if (!launch_conv(cfg, p, d.n, 1, stream, fn)) return SGN_ELAUNCH;
  if (cache_out && !launch_cache_out(x, d, cache_in, fuse, cache_out, stream, 0, ri ? ri->rstd : nullptr,
                                     ri ? ri->gain : nullptr))
    return SGN_ELAUNCH;
  if (ro && !rms_epi) {                              // act from y by the RMS norm kernel
    sgn_dims yd = d;
    yd.c = k;
    const int rc = rms_silu(y, yd, ro->gain, ro->eps, ro->act, stream);
    if (rc != SGN_OK) return rc;
  }
  if (in_epilogue) {
    const double length = (double)ncg * (double)(d.t * d.h * d.w);
    if (!launch_gn_finalize(p.nws, (int)(d.t * p.tiles_f), ns->groups, d.n, length, ns->stats, stream))
      return SGN_ELAUNCH;
  } else if (ns) {
    sgn_dims yd = d;
    yd.c = k;
    const int rc = gn_silu_stats(y, yd, ns->groups, ns->stats, ns->ws, ns->ws_bytes, stream);
    if (rc != SGN_OK) return rc;
  }
  return SGN_OK;
}

}  // namespace sgn

extern "C" int causal_conv3d_eligible(sgn_dims d, int k, int fuse_groups) {
  const char* fn = "causal_conv3d_eligible";
  clear_error();
  if (!conv_shape_ok(d, k, fn)) return 0;
  if (fuse_groups != 0) {
    if (fuse_groups < 0 || d.c % fuse_groups != 0) {
      set_error("%s: fuse groups=%d must divide C=%lld", fn, fuse_groups, (long long)d.c);
      return 0;
    }
    if (d.c > 2048) {
      set_error("%s: fused GroupNorm supports C <= 2048", fn);
      return 0;
    }
  }
  return 1;
}

extern "C" int sgn_conv_plan(int op, sgn_dims d, int k, int fused, sgn_plan* plan) {
  const char* fn = "sgn_conv_plan";
  clear_error();
  if (!plan) {
    set_error("%s: plan is required", fn);
    return SGN_EINVAL;
  }
  if (fused && op != SGN_OP_CAUSAL) {
    set_error("%s: only the causal convolution takes a fused GroupNorm", fn);
    return SGN_EINVAL;
  }
  TileCfg cfg;
  int64_t units = d.n;     // (sample, phase) pairs sharing the tile grid
  int kk = k;
  switch (op) {
    case SGN_OP_CAUSAL:
      if (!conv_shape_ok(d, k, fn)) return SGN_EINVAL;
      if (fused && d.c > 2048) {
        set_error("%s: fused GroupNorm supports C <= 2048", fn);
        return SGN_EINVAL;
      }
      cfg = fused ? choose_tile<kCausal, kFuseGn>(d.h * d.w, d.t, k, (int)d.c, d.n)
                  : choose_tile<kCausal, kFuseNone>(d.h * d.w, d.t, k, (int)d.c, d.n);
      break;
    case SGN_OP_PHASES:
      if (!conv_shape_ok(d, k, fn)) return SGN_EINVAL;
      units = d.n * 4;
      cfg = choose_tile<kPhase, kFuseNone>(d.h * d.w, d.t, k, (int)d.c, units);
      break;
    case SGN_OP_TIME:
      if (!dims_ok(d, fn)) return SGN_EINVAL;
      if (d.c > 2048) {
        set_error("%s: the temporal x2 takes C <= 2048", fn);
        return SGN_EINVAL;
      }
      kk = 2 * (int)d.c;
      if (!conv_shape_ok(d, kk, fn)) return SGN_EINVAL;
      cfg = choose_tile<kTime, kFuseNone>(d.h * d.w, d.t, kk, (int)d.c, d.n);
      break;
    default:
      set_error("%s: unknown op %d", fn, op);
      return SGN_EINVAL;
  }
  plan->kernel = cfg.slab ? SGN_KERNEL_SLAB : SGN_KERNEL_GENERIC;
  plan->tile_m = cfg.bm;
  plan->tile_n = cfg.bn;
  const int64_t tiles_f = (d.h * d.w + cfg.bm - 1) / cfg.bm;
  plan->workgroups = tiles_f * d.t * ((kk + cfg.bn - 1) / cfg.bn) * units;
  return SGN_OK;
}

extern "C" int causal_conv3d(const uint16_t* x, sgn_dims d, const uint16_t* cache_in,
                             const uint16_t* w, int k, const float* bias, const uint16_t* residual,
                             const sgn_gn* fuse, uint16_t* y, uint16_t* cache_out,
                             hipStream_t stream) {
  clear_error();
  return causal_conv_impl("causal_conv3d", x, d, cache_in, w, k, bias, residual, fuse, y, cache_out,
                          nullptr, stream);
}

extern "C" int causal_conv3d_rms(const uint16_t* x, sgn_dims d, const uint16_t* cache_in, const uint16_t* w,
                                 int k, const float* bias, const uint16_t* residual, const sgn_gn* fuse,
                                 const float* gain, float eps, uint16_t* y, uint16_t* act, uint16_t* cache_out,
                                 hipStream_t stream) {
  const char* fn = "causal_conv3d_rms";
  clear_error();
  if (!gain || !act) {
    set_error("%s: gain and act are required", fn);
    return SGN_EINVAL;
  }
  if (!(eps > 0.0f) || !isfinite(eps)) {
    set_error("%s: eps must be a positive finite number", fn);
    return SGN_EINVAL;
  }
  if (k % 64 != 0) {
    set_error("%s: K=%d must be a multiple of 64 (the RMS norm's channels)", fn, k);
    return SGN_EINVAL;
  }
  if (!y && !rms_in_epilogue(k, fuse)) {
    set_error("%s: y may be NULL only when the epilogue applies the norm (unfused, 128 < K <= 256)", fn);
    return SGN_EINVAL;
  }
  if (((uintptr_t)gain & 3) || !aligned16(act)) {
    set_error("%s: act must be 16-byte and gain 4-byte aligned", fn);
    return SGN_EALIGN;
  }
  const RmsOut ro = {gain, eps, act};
  return causal_conv_impl(fn, x, d, cache_in, w, k, bias, residual, fuse, y, cache_out, nullptr, stream, &ro);
}

extern "C" int causal_conv3d_rms_input(const uint16_t* x, sgn_dims d, const uint16_t* cache_in,
                                       const uint16_t* w, int k, const float* bias, const uint16_t* residual,
                                       const double* rstd, const float* gain, uint16_t* y,
                                       uint16_t* cache_out, hipStream_t stream) {
  clear_error();
  const RmsIn ri = {rstd, gain};
  return causal_conv_impl("causal_conv3d_rms_input", x, d, cache_in, w, k, bias, residual, nullptr, y,
                          cache_out, nullptr, stream, nullptr, &ri);
}

extern "C" size_t causal_conv3d_next_stats_workspace(sgn_dims d, int k, int next_groups) {
  if (d.n <= 0 || d.t <= 0 || d.h <= 0 || d.w <= 0 || k < 8 || next_groups <= 0 || k % next_groups)
    return 0;
  return next_stats_bytes(d, k, next_groups);
}

extern "C" int causal_conv3d_next_stats(const uint16_t* x, sgn_dims d, const uint16_t* cache_in,
                                        const uint16_t* w, int k, const float* bias,
                                        const uint16_t* residual, const sgn_gn* fuse, uint16_t* y,
                                        uint16_t* cache_out, int next_groups, double* next_stats,
                                        void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "causal_conv3d_next_stats";
  clear_error();
  if (next_groups <= 0 || k % next_groups != 0) {
    set_error("%s: next_groups=%d must divide K=%d", fn, next_groups, k);
    return SGN_EINVAL;
  }
  {
    sgn_dims yd = d;
    yd.c = k;
    if (gn_silu_stats_workspace(yd, next_groups) == 0) {
      set_error("%s: a GroupNorm of K=%d channels in %d groups is not supported (see gn_silu_stats)", fn, k,
                next_groups);
      return SGN_EINVAL;
    }
  }
  if (!next_stats || ((uintptr_t)next_stats & 7)) {
    set_error("%s: next_stats must be an 8-byte aligned device pointer", fn);
    return !next_stats ? SGN_EINVAL : SGN_EALIGN;
  }
  if (!dims_ok(d, fn)) return SGN_EINVAL;
  const size_t need = next_stats_bytes(d, k, next_groups);
  if (!ws || ws_bytes < need) {
    set_error("%s: workspace of %zu bytes required, got %zu", fn, need, ws ? ws_bytes : 0);
    return SGN_EWORKSPACE;
  }
  if (!aligned16(ws)) {
    set_error("%s: workspace must be 16-byte aligned", fn);
    return SGN_EALIGN;
  }
  const size_t yb = (size_t)(d.n * d.t * d.h * d.w) * k * 2;
  const size_t sb = (size_t)d.n * next_groups * 2 * sizeof(double);
  const size_t xb = (size_t)(d.n * d.t * d.h * d.w * d.c) * 2;
  const size_t cb = (size_t)(d.n * 2 * d.h * d.w * d.c) * 2;
  const size_t wb = (size_t)k * 27 * d.c * 2;
  // The workspace and next_stats are written: they may overlap no input and no other output.
  const struct {
    const void* p;
    size_t n;
  } others[] = {{y, yb}, {x, xb}, {w, wb}, {cache_in, cb}, {cache_out, cb}, {residual, yb},
                {bias, (size_t)k * 4}, {fuse ? fuse->stats : nullptr, fuse && fuse->groups > 0 ? (size_t)d.n * fuse->groups * 16 : 0},
                {fuse ? fuse->gamma : nullptr, (size_t)d.c * 4}, {fuse ? fuse->beta : nullptr, (size_t)d.c * 4}};
  bool alias = overlap(ws, ws_bytes, next_stats, sb);
  for (const auto& o : others)
    if (o.p) alias = alias || overlap(ws, ws_bytes, o.p, o.n) || overlap(next_stats, sb, o.p, o.n);
  if (alias) {
    set_error("%s: the workspace and next_stats must not overlap each other, an input or y", fn);
    return SGN_EALIAS;
  }
  const NextStats ns = {next_groups, next_stats, ws, ws_bytes};
  return causal_conv_impl(fn, x, d, cache_in, w, k, bias, residual, fuse, y, cache_out, &ns, stream);
}

namespace sgn {

// The DupUp3D shortcut of upsample2x_conv_phases_shortcut: the up block's input.
struct Shortcut {
  const uint16_t* src;
  sgn_dims d;
  int ft, first;
};

static int upsample_impl(const char* fn, const uint16_t* x, sgn_dims d, const uint16_t* w_phase, int k,
                         const float* bias, const Shortcut* sc, uint16_t* y, hipStream_t stream) {
  if (!conv_common_checks(x, d, w_phase, k, y, fn)) return SGN_EINVAL;
  if (!aligned16(x) || !aligned16(w_phase) || !aligned16(y) || (bias && !aligned16(bias))) {
    set_error("%s: tensors (and bias) must be 16-byte aligned", fn);
    return SGN_EALIGN;
  }
  const size_t xb = (size_t)(d.n * d.t * d.h * d.w * d.c) * 2;
  const size_t yb = (size_t)(d.n * d.t * 4 * d.h * d.w) * k * 2;
  const size_t wb = (size_t)16 * k * d.c * 2;
  if (overlap(y, yb, x, xb) || overlap(y, yb, w_phase, wb)) {
    set_error("%s: y overlaps x or w_phase", fn);
    return SGN_EALIAS;
  }
  ConvParams p = {};
  if (sc) {
    const sgn_dims& s = sc->d;
    if (!sc->src || !dims_ok(s, fn)) {
      if (!sc->src) set_error("%s: the shortcut source is required", fn);
      return SGN_EINVAL;
    }
    if ((sc->ft != 1 && sc->ft != 2) || (sc->first != 0 && sc->first != 1)) {
      set_error("%s: ft must be 1 or 2 and first 0 or 1", fn);
      return SGN_EINVAL;
    }
    if (s.n != d.n || s.h != d.h || s.w != d.w || d.t != sc->ft * s.t - sc->first * (sc->ft - 1)) {
      set_error("%s: the shortcut source (N=%lld, T=%lld, H=%lld, W=%lld) does not match x under ft=%d, first=%d",
                fn, (long long)s.n, (long long)s.t, (long long)s.h, (long long)s.w, sc->ft, sc->first);
      return SGN_EINVAL;
    }
    if (k % 8 != 0 || (s.c != k && s.c != 2 * (int64_t)k)) {
      set_error("%s: the shortcut needs K %% 8 == 0 and C_in = K or 2K (K=%d, C_in=%lld)", fn, k, (long long)s.c);
      return SGN_EINVAL;
    }
    if ((s.h * s.w + 256) * s.c * 2 >= ((int64_t)1 << 31)) {
      set_error("%s: a shortcut frame exceeds the 2 GiB frame limit", fn);
      return SGN_EINVAL;
    }
    if (!aligned16(sc->src)) {
      set_error("%s: the shortcut source must be 16-byte aligned", fn);
      return SGN_EALIGN;
    }
    if (overlap(y, yb, sc->src, (size_t)(s.n * s.t * s.h * s.w * s.c) * 2)) {
      set_error("%s: y overlaps the shortcut source", fn);
      return SGN_EALIAS;
    }
    p.sc = sc->src;
    p.sc_T = (int)s.t;
    p.sc_C = (int)s.c;
    p.sc_ft = sc->ft;
    p.sc_first = sc->first;
  }
  p.x = x;
  p.w = w_phase;
  p.bias = bias;
  p.y = y;
  p.T = (int)d.t;
  p.H = (int)d.h;
  p.W = (int)d.w;
  p.C = (int)d.c;
  p.K = k;
  p.mper = d.t * d.h * d.w;
  TileCfg cfg = choose_tile<kPhase, kFuseNone>(d.h * d.w, d.t, k, p.C, d.n * 4);
  if (sc && cfg.slab)   // the same tile, in its instantiation with the shortcut epilogue
    cfg = cfg.bm == 256 ? make_slab_cfg<256, 256, 2, 2, kPhase, true>() : make_slab_cfg<224, 256, 1, 4, kPhase, true>();
  if (sc && !cfg.shortcut) {
    set_error("%s: internal: the chosen tile cannot add the shortcut", fn);
    return SGN_EINVAL;
  }
  if (!launch_conv(cfg, p, d.n, 4, stream, fn)) return SGN_ELAUNCH;
  return SGN_OK;
}

}  // namespace sgn

extern "C" int upsample2x_conv_phases(const uint16_t* x, sgn_dims d, const uint16_t* w_phase, int k,
                                      const float* bias, uint16_t* y, hipStream_t stream) {
  clear_error();
  return upsample_impl("upsample2x_conv_phases", x, d, w_phase, k, bias, nullptr, y, stream);
}

extern "C" int upsample2x_conv_phases_shortcut(const uint16_t* x, sgn_dims d, const uint16_t* w_phase, int k,
                                               const float* bias, const uint16_t* shortcut, sgn_dims sd, int ft,
                                               int first, uint16_t* y, hipStream_t stream) {
  clear_error();
  const Shortcut sc = {shortcut, sd, ft, first};
  return upsample_impl("upsample2x_conv_phases_shortcut", x, d, w_phase, k, bias, &sc, y, stream);
}

extern "C" int time_upsample_conv(const uint16_t* x, sgn_dims d, const uint16_t* cache_in, const uint16_t* w,
                                  const float* bias, int first, uint16_t* y, uint16_t* cache_out,
                                  hipStream_t stream) {
  const char* fn = "time_upsample_conv";
  clear_error();
  if (first != 0 && first != 1) {
    set_error("%s: first must be 0 or 1", fn);
    return SGN_EINVAL;
  }
  if (!dims_ok(d, fn)) return SGN_EINVAL;
  if (d.c > 2048) {
    set_error("%s: C=%lld must be at most 2048 (2C output channels)", fn, (long long)d.c);
    return SGN_EINVAL;
  }
  const int k = 2 * (int)d.c;
  if (!conv_common_checks(x, d, w, k, y, fn)) return SGN_EINVAL;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (cache_in && !aligned16(cache_in)) ||
      (cache_out && !aligned16(cache_out)) || (bias && !aligned16(bias))) {
    set_error("%s: tensors (and bias) must be 16-byte aligned", fn);
    return SGN_EALIGN;
  }
  const int64_t hw = d.h * d.w;
  const int64_t nf = d.t - first;
  const int64_t to = first + 2 * nf;
  const size_t xb = (size_t)(d.n * d.t * hw * d.c) * 2;
  const size_t yb = (size_t)(d.n * to * hw * d.c) * 2;
  const size_t cb = (size_t)(d.n * 2 * hw * d.c) * 2;
  const size_t wb = (size_t)k * 3 * d.c * 2;
  if (overlap(y, yb, x, xb) || overlap(y, yb, w, wb) || (cache_in && overlap(y, yb, cache_in, cb)) ||
      (cache_out && (overlap(cache_out, cb, x, xb) || overlap(cache_out, cb, y, yb) ||
                     overlap(cache_out, cb, w, wb) || (cache_in && overlap(cache_out, cb, cache_in, cb))))) {
    set_error("%s: an output overlaps an input or the other output", fn);
    return SGN_EALIAS;
  }
  if (nf > 0) {
    ConvParams p = {};
    p.x = x;
    p.cache = cache_in;
    p.w = w;
    p.bias = bias;
    p.y = y;
    p.T = (int)nf;
    p.H = (int)d.h;
    p.W = (int)d.w;
    p.C = (int)d.c;
    p.K = k;
    p.mper = nf * hw;
    p.Tx = (int)d.t;
    p.x0 = first;
    p.To = (int)to;
    p.first = first;
    const TileCfg cfg = choose_tile<kTime, kFuseNone>(hw, nf, k, p.C, d.n);
    if (!launch_conv(cfg, p, d.n, 1, stream, fn)) return SGN_ELAUNCH;
  }
  if (first) {
    const int64_t packets = hw * d.c / 8;
    int64_t blocks = (packets + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    copy_first_frame_kernel<<<dim3((unsigned)blocks, (unsigned)d.n), 256, 0, stream>>>(
        reinterpret_cast<const uint4*>(x), reinterpret_cast<uint4*>(y), packets, d.t * packets, to * packets);
    if (!launch_ok(fn)) return SGN_ELAUNCH;
  }
  if (cache_out && !launch_cache_out(x, d, cache_in, nullptr, cache_out, stream, first)) return SGN_ELAUNCH;
  return SGN_OK;
}

extern "C" int head_conv_d2s(const uint16_t* x, sgn_dims d, const uint16_t* cache_in, const uint16_t* w,
                             const float* bias, const sgn_gn* fuse, int clamp, uint16_t* video,
                             uint16_t* cache_out, hipStream_t stream) {
  const char* fn = "head_conv_d2s";
  clear_error();
  const int k = 12;
  if (!conv_common_checks(x, d, w, k, video, fn)) return SGN_EINVAL;
  int rc = check_fuse(fuse, d, fn);
  if (rc) return rc;
  if (!aligned16(x) || !aligned16(w) || !aligned16(video) || (cache_in && !aligned16(cache_in)) ||
      (cache_out && !aligned16(cache_out)) || (bias && !aligned16(bias))) {
    set_error("%s: tensors (and bias) must be 16-byte aligned", fn);
    return SGN_EALIGN;
  }
  const size_t xb = (size_t)(d.n * d.t * d.h * d.w * d.c) * 2;
  const size_t vb = (size_t)(d.n * 3 * d.t * 4 * d.h * d.w) * 2;
  const size_t cb = (size_t)(d.n * 2 * d.h * d.w * d.c) * 2;
  const size_t wb = (size_t)k * 27 * d.c * 2;
  if (overlap(video, vb, x, xb) || overlap(video, vb, w, wb) || (cache_in && overlap(video, vb, cache_in, cb)) ||
      (cache_out && (overlap(cache_out, cb, x, xb) || overlap(cache_out, cb, video, vb) ||
                     overlap(cache_out, cb, w, wb) || (cache_in && overlap(cache_out, cb, cache_in, cb))))) {
    set_error("%s: an output overlaps an input or the other output", fn);
    return SGN_EALIAS;
  }
  ConvParams p = {};
  p.x = x;
  p.cache = cache_in;
  p.w = w;
  p.bias = bias;
  p.y = video;
  if (fuse) {
    p.stats = fuse->stats;
    p.gamma = fuse->gamma;
    p.beta = fuse->beta;
    p.eps = (double)fuse->eps;
    p.groups = fuse->groups;
  }
  p.T = (int)d.t;
  p.H = (int)d.h;
  p.W = (int)d.w;
  p.C = (int)d.c;
  p.K = k;
  p.mper = d.t * d.h * d.w;
  p.clamp = clamp ? 1 : 0;
  if (!fuse && (p.C == 128 || p.C == 256)) {
    // The dedicated head kernel: one workgroup per (sample, row pair, 48 columns).
    const int wblocks = (p.W + 16 * kHeadSeg - 1) / (16 * kHeadSeg);
    const int64_t nb = (int64_t)d.n * ((p.H + kHeadOut - 1) / kHeadOut) * wblocks;
    const int nw = p.C / 32;
    if (nb * nw * 64 >= ((int64_t)1 << 32)) {        // a launch holds fewer than 2^32 work-items
      set_error("%s: problem too large for one launch", fn);
      return SGN_ELAUNCH;
    }
    p.nblocks = (int)nb;
    const int lds = head_lds_bytes(nw);
    const void* fn_ptr = nw == 4 ? (const void*)head_kernel<4> : (const void*)head_kernel<8>;
    hipError_t e = hipFuncSetAttribute(fn_ptr, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) {
      set_error("%s: cannot reserve %d bytes of LDS: %s", fn, lds, hipGetErrorString(e));
      return SGN_ELAUNCH;
    }
    if (nw == 4)
      head_kernel<4><<<dim3((unsigned)nb), 256, lds, stream>>>(p, wblocks);
    else
      head_kernel<8><<<dim3((unsigned)nb), 512, lds, stream>>>(p, wblocks);
    if (!launch_ok(fn)) return SGN_ELAUNCH;
  } else {
    const TileCfg cfg = fuse ? make_cfg<256, 32, 4, 1, kStages, kHead, kFuseGn>(p.C)
                             : make_cfg<256, 32, 4, 1, kStages, kHead, kFuseNone>(p.C);
    if (!launch_conv(cfg, p, d.n, 1, stream, fn)) return SGN_ELAUNCH;
  }
  if (cache_out && !launch_cache_out(x, d, cache_in, fuse, cache_out, stream)) return SGN_ELAUNCH;
  return SGN_OK;
}

namespace sgn {

// Workspace of causal_conv3d_winograd: the transformed input V (bf16 [36][N][T + 2][TP][C])
// at offset 0, the products M (fp32 [36][N][T][TP][K]) at offset *m_off (256-byte aligned).
static size_t wino_workspace(sgn_dims d, int k, size_t* m_off) {
  const int64_t tp = ((d.h + 3) / 4) * ((d.w + 3) / 4);
  const size_t vb = (size_t)36 * d.n * (d.t + 2) * tp * d.c * 2;
  const size_t off = (vb + 255) / 256 * 256;
  if (m_off) *m_off = off;
  return off + (size_t)36 * d.n * d.t * tp * k * 4;
}

static bool wino_shape_ok(sgn_dims d, int k, const char* fn) {
  if (!conv_shape_ok(d, k, fn)) return false;
  if (k <= 128 || k % 8 != 0) {
    set_error("%s: K=%d must be a multiple of 8 above 128 (the slab kernel's tiles)", fn, k);
    return false;
  }
  if (d.t + 2 > 65535) {                             // the transforms' grids take a frame per y index
    set_error("%s: T=%lld exceeds the transforms' limit of 65533 frames", fn, (long long)d.t);
    return false;
  }
  const int64_t tp = ((d.h + 3) / 4) * ((d.w + 3) / 4);
  if ((tp + 256) * (int64_t)k * 4 >= ((int64_t)1 << 31) || (tp + 256) * d.c * 2 >= ((int64_t)1 << 31)) {
    set_error("%s: a frame of %lld tiles exceeds the 2 GiB frame limit of the products", fn, (long long)tp);
    return false;
  }
  return true;
}

}  // namespace sgn

extern "C" size_t causal_conv3d_winograd_workspace(sgn_dims d, int k) {
  clear_error();
  if (!wino_shape_ok(d, k, "causal_conv3d_winograd_workspace")) return 0;
  return wino_workspace(d, k, nullptr);
}

extern "C" int causal_conv3d_winograd(const uint16_t* x, sgn_dims d, const uint16_t* cache_in, const uint16_t* u,
                                      int k, const float* bias, const uint16_t* residual, uint16_t* y,
                                      uint16_t* cache_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "causal_conv3d_winograd";
  clear_error();
  if (!wino_shape_ok(d, k, fn)) return SGN_EINVAL;
  if (!x || !u || !y) {
    set_error("%s: x, u and y are required", fn);
    return SGN_EINVAL;
  }
  if (!aligned16(x) || !aligned16(u) || !aligned16(y) || (cache_in && !aligned16(cache_in)) ||
      (residual && !aligned16(residual)) || (cache_out && !aligned16(cache_out)) || (bias && !aligned16(bias))) {
    set_error("%s: tensors (and bias) must be 16-byte aligned", fn);
    return SGN_EALIGN;
  }
  size_t m_off = 0;
  const size_t need = wino_workspace(d, k, &m_off);
  if (!ws || ws_bytes < need) {
    set_error("%s: workspace of %zu bytes required, got %zu", fn, need, ws ? ws_bytes : 0);
    return SGN_EWORKSPACE;
  }
  if (!aligned16(ws)) {
    set_error("%s: workspace must be 16-byte aligned", fn);
    return SGN_EALIGN;
  }
  const size_t xb = (size_t)(d.n * d.t * d.h * d.w * d.c) * 2;
  const size_t yb = (size_t)(d.n * d.t * d.h * d.w) * k * 2;
  const size_t cb = (size_t)(d.n * 2 * d.h * d.w * d.c) * 2;
  const size_t ub = (size_t)36 * k * 3 * d.c * 2;
  if (overlap(y, yb, x, xb) || overlap(y, yb, u, ub) || (cache_in && overlap(y, yb, cache_in, cb)) ||
      (residual && overlap(y, yb, residual, yb)) ||
      (cache_out && (overlap(cache_out, cb, x, xb) || overlap(cache_out, cb, y, yb) ||
                     overlap(cache_out, cb, u, ub) || (cache_in && overlap(cache_out, cb, cache_in, cb)) ||
                     (residual && overlap(cache_out, cb, residual, yb))))) {
    set_error("%s: an output overlaps an input or the other output", fn);
    return SGN_EALIAS;
  }
  const struct {
    const void* p;
    size_t n;
  } others[] = {{x, xb}, {u, ub}, {y, yb}, {cache_in, cb}, {cache_out, cb}, {residual, yb}, {bias, (size_t)k * 4}};
  for (const auto& o : others)
    if (o.p && overlap(ws, need, o.p, o.n)) {
      set_error("%s: the workspace overlaps an input or an output", fn);
      return SGN_EALIAS;
    }
  const int th = (int)((d.h + 3) / 4), tw = (int)((d.w + 3) / 4);
  const int64_t tp = (int64_t)th * tw;
  uint16_t* v = static_cast<uint16_t*>(ws);
  float* m = reinterpret_cast<float*>(static_cast<char*>(ws) + m_off);
  {
    const int cp = (int)(d.c / 2);
    int64_t blocks = (tp * cp + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    wino_input_kernel<<<dim3((unsigned)blocks, (unsigned)(d.t + 2), (unsigned)d.n), 256, 0, stream>>>(
        reinterpret_cast<const uint32_t*>(x), reinterpret_cast<const uint32_t*>(cache_in),
        reinterpret_cast<uint32_t*>(v), (int)d.n, (int)d.t, (int)d.h, (int)d.w, cp, tw, tp);
    if (!launch_ok("causal_conv3d_winograd (input transform)")) return SGN_ELAUNCH;
  }
  {
    ConvParams p = {};
    p.x = v;
    p.w = u;
    p.yf = m;
    p.T = (int)d.t;
    p.H = th;
    p.W = tw;
    p.C = (int)d.c;
    p.K = k;
    p.mper = d.t * tp;
    p.Tx = (int)d.t + 2;
    p.x0 = 2;
    p.wino_n = (int)d.n;
    const TileCfg cfg = choose_tile<kWino, kFuseNone>(tp, d.t, k, p.C, 36 * d.n);
    if (!launch_conv(cfg, p, 36 * d.n, 1, stream, fn)) return SGN_ELAUNCH;
  }
  {
    int64_t blocks = (tp * (k / 4) + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    wino_output_kernel<<<dim3((unsigned)blocks, (unsigned)d.t, (unsigned)d.n), 256, 0, stream>>>(
        m, bias, residual, y, (int)d.n, (int)d.t, (int)d.h, (int)d.w, k, tw, tp);
    if (!launch_ok("causal_conv3d_winograd (output transform)")) return SGN_ELAUNCH;
  }
  if (cache_out && !launch_cache_out(x, d, cache_in, nullptr, cache_out, stream)) return SGN_ELAUNCH;
  return SGN_OK;
}
