/*
 * silugn.h -- C ABI of libsilugn.so: GroupNorm + SiLU (and the RMS norm + SiLU),
 * the causal / upsample / head convolutions and the rest of an up block (temporal
 * x2, DupUp3D shortcut) of a Wan2.2-style video VAE decoder, as gfx950 (MI355X)
 * HIP kernels; shape predicates for the GroupNorm and the convolution.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Activations are bf16 (passed as uint16_t bit patterns), channels-last
 *   (N, T, H, W, C), dense, with C the contiguous dimension. C % 8 == 0 so that
 *   a position's channels split into 16-byte packets of 8 channels; every
 *   tensor pointer must be 16-byte aligned.
 * - All tensor pointers are DEVICE pointers owned by the caller; inputs are
 *   read only. Except for upsample2x_prepare_weights (host memory, host
 *   compute), the library allocates nothing, keeps no state between calls and
 *   never synchronises the host: work is enqueued on the caller's stream and
 *   ordered by it.
 * - Return value: 0 on success, a negative SGN_E* code otherwise. Arguments are
 *   validated on the host before anything is enqueued, so an error leaves every
 *   output untouched. sgn_last_error() gives the calling thread's last message.
 * - Results are deterministic: partial sums are combined in a fixed order and
 *   no floating-point atomics are used.
 */
#ifndef SILUGN_H
#define SILUGN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SGN_OK = 0,
  SGN_EINVAL = -1,      /* bad size, null required pointer, unsupported shape */
  SGN_EALIGN = -2,      /* a tensor pointer is not 16-byte aligned */
  SGN_EALIAS = -3,      /* an output overlaps an input it may not overlap */
  SGN_ELAUNCH = -4,     /* a launch failed (message has the HIP error), or the problem exceeds one launch's grid */
  SGN_EWORKSPACE = -5   /* workspace missing or smaller than *_workspace() asks for */
};

/* Dimensions of a channels-last activation tensor. */
typedef struct {
  int64_t n, t, h, w, c;
} sgn_dims;

/*
 * GroupNorm parameters for a convolution that applies silu(group_norm(x)) to
 * its input while loading it (see causal_conv3d). stats is the output of
 * gn_silu_stats for the same x; gamma/beta are fp32 [C]; eps as in gn_silu_apply.
 */
typedef struct {
  const double* stats;
  const float* gamma;
  const float* beta;
  float eps;
  int groups;
} sgn_gn;

/* Message of the calling thread's last failed call ("" if none). Never NULL. */
const char* sgn_last_error(void);

/*
 * gn_silu_eligible -- 1 if gn_silu_stats / gn_silu_apply take dims d with `groups`
 * groups, else 0 (the reason in sgn_last_error()). A predicate apart from the
 * compute calls, as the group_norm_silu.py page's eligibility check (its
 * `eligible`: the kernels run only for inputs they support). No device work.
 */
int gn_silu_eligible(sgn_dims d, int groups);

/*
 * Bytes of device workspace gn_silu_stats needs for dims d and `groups`
 * (per-block fp64 partial sums). 0 if the arguments are invalid.
 */
size_t gn_silu_stats_workspace(sgn_dims d, int groups);

/*
 * gn_silu_stats -- GroupNorm statistics of x.
 * Defined by: WanGP group_norm_silu.py page, module docstring (per-group sums
 * of a span in compensated fp32, reduced in fp64 in a fixed order) and its
 * apply kernel (variance = mean of squared deviations, divided by the length).
 *
 * For every sample n and group g (channels [g*C/G, (g+1)*C/G), all T*H*W
 * positions of this call's x -- statistics never include a causal cache):
 *   stats[(n*G + g)*2 + 0] = mean,  stats[(n*G + g)*2 + 1] = biased variance,
 * both fp64. x: bf16 (N,T,H,W,C). ws: device workspace of at least
 * gn_silu_stats_workspace(d, groups) bytes, overwritten. C % groups == 0 and
 * C/groups must be 1, 2, 4 or a multiple of 8; C <= 2048. x, stats and ws must not
 * overlap (SGN_EALIAS).
 */
int gn_silu_stats(const uint16_t* x, sgn_dims d, int groups, double* stats,
                  void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * gn_silu_stats_noalloc -- gn_silu_stats without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). It allocates nothing: the per-block partial sums go
 * to a static 4 MiB device array inside the library, one per GPU, held until the process
 * ends. Same x, d, groups, stats and result as gn_silu_stats (bitwise the same for up to
 * 128 groups; with more, fewer partial blocks are used, so the sums are taken in another
 * fixed order). Requires N x groups <= 262144 (else SGN_EINVAL); stats must not overlap
 * x (SGN_EALIAS). All calls on one GPU share the array: calls that overlap in time on one
 * GPU (different streams, or host threads without ordering) race and must not be made.
 */
int gn_silu_stats_noalloc(const uint16_t* x, sgn_dims d, int groups, double* stats,
                          hipStream_t stream);

/*
 * gn_silu_apply -- y = silu(group_norm(x)), one rounding to bf16.
 * Defined by: WanGP group_norm_silu.py page, module docstring ("GroupNorm and
 * SiLU in FP32, one rounding to the output dtype") and its third pass.
 *
 *   z = (x - mean_g) * gamma_c / sqrt(var_g + eps) + beta_c   (computed in fp64)
 *   y = RNE_bf16( z * sigmoid(z) )
 * stats from gn_silu_stats; gamma, beta fp32 [C] (device); eps > 0 is used as
 * the exact fp64 value of the given float. y may equal x (in place); any other
 * overlap is SGN_EALIAS. Accuracy: within 1 bf16 ulp of the fp64 result rounded
 * once (finite inputs).
 */
int gn_silu_apply(const uint16_t* x, sgn_dims d, int groups, const double* stats,
                  const float* gamma, const float* beta, float eps, uint16_t* y,
                  hipStream_t stream);

/*
 * rms_silu -- RMS norm + SiLU per position.
 * Defined by: binding.cpp page, the comment above Decoder::output_head (the decoder
 * normalizes with an RMS norm followed by SiLU, with a per-channel gain: norm_pad(x,
 * gain, ...)). The pages do not print the formula; the usual RMS norm is read:
 *
 *   z[p, c] = x[p, c] * gain[c] / sqrt(mean_c(x[p, :]^2) + eps)
 *   y[p, c] = RNE_bf16( z * sigmoid(z) )
 *
 * for every position p = (n, t, h, w) on its own (no statistics across positions).
 * The mean of squares and z are formed in fp64, the SiLU in fp32 as in
 * gn_silu_apply. x, y: bf16 (N,T,H,W,C), 16-byte aligned, y == x allowed (in
 * place), any other overlap is SGN_EALIAS; gain: device fp32 [C]; eps > 0.
 * Requires C % 64 == 0 with C <= 4096, else SGN_EINVAL.
 */
int rms_silu(const uint16_t* x, sgn_dims d, const float* gain, float eps, uint16_t* y,
             hipStream_t stream);

/*
 * rms_silu_rstd -- the per-position factor of rms_silu: rstd[p] = 1 / sqrt(mean_c x[p,:]^2
 * + eps) in fp64, bitwise the value rms_silu applies (the same kernel and launch, which
 * writes rstd instead of y). It is what a convolution needs to apply the RMS norm in its
 * operand load (causal_conv3d_rms_input): the norm has no statistics across positions, so
 * this one fp64 per position is all that has to be formed before the convolution.
 * Defined by: binding.cpp page, the comment above Decoder::output_head (the decoder's RMS
 * norm + SiLU, norm_pad); the formula is rms_silu's.
 *   x     bf16 (N,T,H,W,C), 16-byte aligned; C % 64 == 0, C <= 4096 (else SGN_EINVAL)
 *   rstd  device fp64 [N][T][H][W], 8-byte aligned, written; must not overlap x (SGN_EALIAS)
 *   eps   > 0, used as its exact fp64 value
 */
int rms_silu_rstd(const uint16_t* x, sgn_dims d, float eps, double* rstd, hipStream_t stream);

/*
 * causal_conv3d -- causal 3x3x3 convolution with a 2-frame temporal cache.
 * Defined by: FastVideo wan22_vae_decode binding.cpp page, Decoder::conv (front
 * temporal padding of kt-1 = 2 frames taken from the per-conv cache, spatial
 * zero padding kh/2 = kw/2 = 1, the cache keeps the last 2 frames of the padded
 * input) and Decoder::resnet (bias and residual added to the conv output).
 *
 *   P = cat_T(cache_in, a),  a = x, or silu(group_norm(x)) when fuse != NULL
 *   y[n,t,h,w,k] = RNE_bf16( bias[k] + residual[n,t,h,w,k]
 *        + sum_{dt,dh,dw in 0..2} sum_c w[k,dt,dh,dw,c] * P[n, t+dt, h+dh-1, w+dw-1, c] )
 * with P zero outside the frame, bf16 products accumulated in fp32.
 *   x         bf16 (N,T,H,W,C), T >= 1
 *   cache_in  bf16 (N,2,H,W,C) already-activated frames preceding x, or NULL (zeros)
 *   w         bf16 (K,3,3,3,C): tap (dt,dh,dw) with dt = 0 the oldest frame
 *   bias      fp32 [K] or NULL; residual bf16 (N,T,H,W,K) or NULL
 *   fuse      NULL, or the GroupNorm of x to apply in the operand load; the
 *             result is bitwise equal to gn_silu_apply followed by this call
 *             with fuse == NULL
 *   y         bf16 (N,T,H,W,K); must not overlap x, cache_in, residual or w
 *   cache_out bf16 (N,2,H,W,C) = P[:, T:T+2] (activated when fused), or NULL;
 *             must not overlap cache_in, x or y
 * Requires C % 64 == 0 with C <= 4096 (C <= 2048 when fused), K % 4 == 0 with
 * 4 <= K <= 4096; any other shape is SGN_EINVAL.
 */
int causal_conv3d(const uint16_t* x, sgn_dims d, const uint16_t* cache_in,
                  const uint16_t* w, int k, const float* bias, const uint16_t* residual,
                  const sgn_gn* fuse, uint16_t* y, uint16_t* cache_out, hipStream_t stream);

/*
 * causal_conv3d_rms -- causal_conv3d, plus act = the decoder's RMS norm + SiLU of its
 * output (the next convolution's input), written by the convolution's epilogue when it
 * can be.
 * Defined by: binding.cpp page, Decoder's `prepared` edge (a convolution whose epilogue
 * already normalised and activated the next convolution's input, with the y store
 * suppressed when nothing else reads it: Decoder::conv's y_dead) and the decoder's RMS
 * norm (the comment above Decoder::output_head); the formula is rms_silu's.
 *
 *   y   = causal_conv3d(x, cache_in, w, k, bias, residual, fuse)   (bf16)
 *   act = rms_silu(y, gain, eps)                                   (bf16, N,T,H,W,K)
 * Unfused with 128 < K <= 256 (one N tile holds every channel of a position) the
 * epilogue forms each position's mean of squares from the rounded y in fp64 and stores
 * act beside y; y may then be NULL (not stored). Otherwise y is required and act comes
 * from rms_silu over y after the convolution. gain fp32 [K] (4-byte aligned); eps > 0;
 * K % 64 == 0. act must not overlap any input or other output (SGN_EALIAS). Accuracy:
 * y as causal_conv3d (bitwise the same); act within 1 bf16 ulp of rms_silu(y).
 */
int causal_conv3d_rms(const uint16_t* x, sgn_dims d, const uint16_t* cache_in,
                      const uint16_t* w, int k, const float* bias, const uint16_t* residual,
                      const sgn_gn* fuse, const float* gain, float eps, uint16_t* y,
                      uint16_t* act, uint16_t* cache_out, hipStream_t stream);

/*
 * causal_conv3d_rms_input -- causal_conv3d of the decoder's RMS norm + SiLU of x, the norm
 * applied in the convolution's operand load (the consumer side; causal_conv3d_rms is the
 * producer side).
 * Defined by: binding.cpp page, the comment above Decoder::output_head and Decoder::conv's
 * norm_pad(x, gain, cache, ...) (normalise, activate and pad the convolution's input); the
 * norm is rms_silu's.
 *
 *   a = rms_silu(x, gain, eps)   with rstd = rms_silu_rstd(x, eps) passed in
 *   y = causal_conv3d(a, cache_in, w, k, bias, residual)
 * Bitwise equal to rms_silu followed by causal_conv3d (fuse == NULL): the rows of x are
 * activated with rms_silu's arithmetic as they are loaded, and the accumulation order is
 * the unfused convolution's. cache_out (if not NULL) = the last 2 frames of cat(cache_in,
 * a), i.e. activated; cache_in holds activated frames.
 *   rstd  device fp64 [N][T][H][W] from rms_silu_rstd on the same x and eps (8-byte aligned)
 *   gain  device fp32 [C] (4-byte aligned)
 * Other arguments and errors as causal_conv3d; C <= 2048 (else SGN_EINVAL); y and
 * cache_out must not overlap rstd or gain (SGN_EALIAS). It runs the per-tap kernel
 * (sgn_conv_plan with fused != 0 names its tile), which activates each row once per tap.
 */
int causal_conv3d_rms_input(const uint16_t* x, sgn_dims d, const uint16_t* cache_in,
                            const uint16_t* w, int k, const float* bias, const uint16_t* residual,
                            const double* rstd, const float* gain, uint16_t* y,
                            uint16_t* cache_out, hipStream_t stream);

/*
 * causal_conv3d_eligible -- 1 if causal_conv3d takes input dims d and K = k output
 * channels (fuse_groups > 0: with a fused GroupNorm of that many groups; 0: unfused),
 * else 0 with the reason in sgn_last_error(). The shape part of causal_conv3d's
 * checks, as a predicate apart from compute (the group_norm_silu.py page's
 * `eligible` check). No device work.
 */
int causal_conv3d_eligible(sgn_dims d, int k, int fuse_groups);

/*
 * sgn_conv_plan -- which kernel and tile a convolution call would run, without running
 * it (a predicate-style query beside causal_conv3d_eligible, as the group_norm_silu.py
 * page separates its eligibility check from compute). No device work.
 *   op     SGN_OP_CAUSAL (causal_conv3d / causal_conv3d_next_stats / causal_conv3d_rms;
 *          fused != 0 for a fused GroupNorm), SGN_OP_PHASES (upsample2x_conv_phases[_shortcut]:
 *          d = the low-resolution input), SGN_OP_TIME (time_upsample_conv: d.t = the frames
 *          convolved, T - first; k is ignored, K = 2C)
 *   plan   receives the kernel (SGN_KERNEL_SLAB: the slab kernel whose three column taps
 *          share one staged slab; SGN_KERNEL_GENERIC: the per-tap kernel), the tile
 *          (output positions x output channels per workgroup) and the workgroup count.
 * Returns SGN_OK, or SGN_EINVAL for a shape the call would reject. The dedicated output
 * head kernel is not covered (head_conv_d2s picks it for unfused C = 128 or 256).
 */
enum { SGN_OP_CAUSAL = 0, SGN_OP_PHASES = 1, SGN_OP_TIME = 2 };
enum { SGN_KERNEL_SLAB = 1, SGN_KERNEL_GENERIC = 2 };
typedef struct {
  int kernel;
  int tile_m, tile_n;
  int64_t workgroups;
} sgn_plan;
int sgn_conv_plan(int op, sgn_dims d, int k, int fused, sgn_plan* plan);

/*
 * Bytes of device workspace causal_conv3d_next_stats needs for input dims d, K
 * output channels and next_groups groups (0 if the arguments are invalid).
 */
size_t causal_conv3d_next_stats_workspace(sgn_dims d, int k, int next_groups);

/*
 * causal_conv3d_next_stats -- causal_conv3d, and the GroupNorm statistics of its
 * output y for the GroupNorm that follows it.
 * Defined by: binding.cpp page, Decoder::conv (the producer convolution's fused
 * epilogue prepares the next convolution's normalized input: the next norm is
 * folded into the producer) and Decoder::resnet (conv1 -> norm2 -> conv2). A
 * GroupNorm needs statistics over the whole tensor before it can be applied, so
 * what the epilogue can take over is the statistics pass over y.
 *
 * All arguments before next_groups as in causal_conv3d (same checks, same y and
 * cache_out). Then:
 *   next_stats  device fp64 [N][next_groups][2]: mean and biased variance of each
 *               (n, g) over y's channels g*K/G .. (g+1)*K/G - 1 and all T*H*W
 *               positions -- what gn_silu_stats(y, next_groups) returns, the sums
 *               taken in a different fixed order (equal up to fp64 rounding).
 *   ws          device workspace of causal_conv3d_next_stats_workspace(d, k,
 *               next_groups) bytes, 16-byte aligned, overwritten.
 * The statistics come from the convolution's epilogue when K % 8 == 0 and K/G is a
 * multiple of 8 dividing the kernel's N tile; otherwise gn_silu_stats runs over y.
 * Errors: next_groups must divide K and y's GroupNorm must be one gn_silu_stats
 * accepts (K % 8 == 0; K/G = 1, 2, 4 or a multiple of 8), else SGN_EINVAL; a
 * missing or short workspace is SGN_EWORKSPACE; ws and next_stats must not overlap
 * each other, y or any input (SGN_EALIAS).
 */
int causal_conv3d_next_stats(const uint16_t* x, sgn_dims d, const uint16_t* cache_in,
                             const uint16_t* w, int k, const float* bias,
                             const uint16_t* residual, const sgn_gn* fuse, uint16_t* y,
                             uint16_t* cache_out, int next_groups, double* next_stats,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * winograd_prepare_weights -- HOST function: the F(4x4,3x3) Winograd weights of a causal
 * 3x3x3 convolution for causal_conv3d_winograd.
 * Defined by: binding.cpp page, prepare() ("F(4x4,3x3) Winograd weights": the 6x3 matrix G
 * below; each of the 36 components keeps the 3-tap temporal convolution; the sums are formed
 * in fp32 and stored in bf16).
 *
 *   G = [1/4 0 0; -1/6 -1/6 -1/6; -1/6 1/6 -1/6; 1/24 1/12 1/6; 1/24 -1/12 1/6; 0 0 1]
 *   u[a*6 + b][k][dt][c] = RNE_bf16( sum over (r, s) with G[a][r] G[b][s] != 0 of
 *                                    w[k][dt][r][s][c] * (G[a][r] G[b][s]) ), summed in fp32
 * w: host bf16 (K,3,3,3,C); u: host bf16 (36,K,3,C), i.e. 108*K*C values; u must not
 * overlap w (SGN_EALIAS).
 */
int winograd_prepare_weights(const uint16_t* w, int k, int c, uint16_t* u);

/*
 * Bytes of device workspace causal_conv3d_winograd needs for input dims d and K output
 * channels (0, with the reason in sgn_last_error(), for a shape it rejects).
 */
size_t causal_conv3d_winograd_workspace(sgn_dims d, int k);

/*
 * causal_conv3d_winograd -- causal_conv3d (unfused) through Winograd F(4x4,3x3): the spatial
 * 3x3 taps in 6x6-point transforms, each of the 36 components a causal 3-tap temporal
 * product.
 * Defined by: binding.cpp page, Decoder::conv (only the expensive spatial 3x3 convolutions
 * go through Winograd: the padded input is transformed, one 3-tap temporal convolution runs
 * per component, and an epilogue forms the output with the bias and the residual) and
 * prepare() (the weights: winograd_prepare_weights). The input and output transforms are
 * those of G's interpolation points 0, 1, -1, 2, -2 and infinity:
 *   V = B^T d B of each 4x4 output tile's 6x6 input patch (rows and columns 4i-1 .. 4i+4,
 *       zero outside the frame) in every frame of P = cat(cache_in, x), fp32 from the bf16
 *       input, rounded once to bf16;
 *   M[ab][n,t,tile,k] = sum_{dt,c} u[ab][k][dt][c] V[ab][n, t+dt, tile, c]   (fp32)
 *   y = RNE_bf16( A^T M A + bias + residual )   (fp32), the pixels inside the frame.
 * Arguments as causal_conv3d with u (device, from winograd_prepare_weights) for w, no fused
 * GroupNorm, and a device workspace ws of causal_conv3d_winograd_workspace(d, k) bytes,
 * 16-byte aligned, overwritten: V, bf16 [36][N][T+2][ceil(H/4)][ceil(W/4)][C], at offset 0,
 * then M, fp32 [36][N][T][ceil(H/4)][ceil(W/4)][K], at the next 256-byte boundary.
 * Accuracy: the same result as causal_conv3d up to the bf16 rounding of u and V, which the
 * output transform amplifies (by up to about 10x at a tile's far corner): about 2.5e-2
 * relative L2 error on unit-scale data against 1.7e-3 for causal_conv3d.
 * Requires C % 64 == 0 with C <= 4096 and 128 < K <= 4096 with K % 8 == 0; the outputs and
 * the workspace must not overlap any input or each other (SGN_EALIAS).
 */
int causal_conv3d_winograd(const uint16_t* x, sgn_dims d, const uint16_t* cache_in,
                           const uint16_t* u, int k, const float* bias, const uint16_t* residual,
                           uint16_t* y, uint16_t* cache_out, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/*
 * upsample2x_prepare_weights -- HOST function: the four 2x2 phase kernels of a
 * nearest-x2 + 3x3 convolution.
 * Defined by: binding.cpp page, prepare() ("Nearest-x2 + 3x3 convolution equals
 * four 2x2 low-resolution phases"; sums formed in fp32, stored in bf16).
 *
 * For output phase (a,b) in {0,1}^2 and phase tap (u,v) in {0,1}^2:
 *   w_phase[a][b][k][u][v][c] = RNE_bf16( sum of w3x3[k][r][s][c] over the taps
 *       with floor((a+r-1)/2) == u+a-1 and floor((b+s-1)/2) == v+b-1 ),
 * the sum taken in fp32. w3x3: host bf16 (K,3,3,C); w_phase: host bf16
 * (2,2,K,2,2,C), i.e. 16*K*C values.
 */
int upsample2x_prepare_weights(const uint16_t* w3x3, int k, int c, uint16_t* w_phase);

/*
 * upsample2x_conv_phases -- nearest-x2 upsample + 3x3 convolution, computed as
 * four 2x2 convolutions at the low resolution.
 * Defined by: binding.cpp page, prepare() (phase weights) and Decoder::up (the
 * four phase convolutions, then the interleave with the bias).
 *
 *   y[n,t,2i+a,2j+b,k] = RNE_bf16( bias[k] + sum_{u,v,c}
 *        w_phase[a][b][k][u][v][c] * x[n, t, i+u+a-1, j+v+b-1, c] ),  zero outside.
 * Per frame (no temporal taps, no cache). x bf16 (N,T,H,W,C); w_phase device bf16
 * from upsample2x_prepare_weights; bias fp32 [K] or NULL; y bf16 (N,T,2H,2W,K),
 * written interleaved, must not overlap x or w_phase. Requires C % 64 == 0 with
 * C <= 4096, K % 4 == 0 with 4 <= K <= 4096.
 */
int upsample2x_conv_phases(const uint16_t* x, sgn_dims d, const uint16_t* w_phase, int k,
                           const float* bias, uint16_t* y, hipStream_t stream);

/*
 * upsample2x_conv_phases_shortcut -- upsample2x_conv_phases plus the DupUp3D
 * shortcut of the up block's input, added before the one rounding.
 * Defined by: binding.cpp page, Decoder::up_block (the resampler's last pass
 * interleaves the four phases and adds the bias and the DupUp3D shortcut of the
 * block's input). The pages do not print DupUp3D; the reading used:
 *
 *   y[n,f,Y,X,k] = RNE_bf16( phases + bias[k]
 *        + sc[n, tt / ft, Y / 2, X / 2, (k F + o) / rep] ),
 *   tt = f + first (ft - 1), o = ((tt % ft) 2 + Y % 2) 2 + X % 2,
 *   F = 4 ft, rep = K F / C_in,
 * i.e. every input channel repeated rep times, read as (k, time, row, column)
 * sub-positions and unfolded ft x 2 x 2; on the video's first pass the first
 * ft - 1 output frames are dropped.
 *   shortcut  bf16 (N, T_in, H, W, C_in) with the phases' N, H, W, and
 *             T = ft T_in - first (ft - 1) (x's T); C_in = K or 2K
 *   ft        1 or 2 (the block upsamples time too); first 0 or 1
 * Requires K % 8 == 0 as well as upsample2x_conv_phases' shapes; y must not overlap
 * the shortcut (SGN_EALIAS). Other shapes are SGN_EINVAL.
 */
int upsample2x_conv_phases_shortcut(const uint16_t* x, sgn_dims d, const uint16_t* w_phase, int k,
                                    const float* bias, const uint16_t* shortcut, sgn_dims sd,
                                    int ft, int first, uint16_t* y, hipStream_t stream);

/*
 * time_upsample_conv -- temporal x2 of an up block: a causal 3x1x1 convolution to
 * 2C channels whose two halves become two consecutive output frames.
 * Defined by: binding.cpp page, Decoder::up_block, the seam after the resnets of
 * blocks 0 and 1 (time_upsample: the causal time convolution with its own 2-frame
 * cache and no normalisation writes the frame-interleaved tensor directly; on the
 * video's first pass the first frame is not convolved and goes straight to the
 * output). The layout of the halves is a reading:
 *
 *   nf = T - first,  P = cat_T(cache_in, x[:, first:])   (cache_in NULL: zeros)
 *   z[n,i,h,w,k] = bias[k] + sum_{dt in 0..2} sum_c w[k,dt,c] * P[n, i+dt, h, w, c]
 *   y[n, first + 2i + s, h, w, c] = RNE_bf16( z[n,i,h,w, s C + c] ),  s = 0, 1
 *   y[n, 0] = x[n, 0] when first (bit copy)
 * bf16 products accumulated in fp32.
 *   x         bf16 (N,T,H,W,C), T >= 1 (T = 1 with first: only the copied frame)
 *   cache_in  bf16 (N,2,H,W,C) or NULL; w bf16 (2C,3,C), dt = 0 the oldest frame
 *   bias      fp32 [2C] or NULL
 *   y         bf16 (N, first + 2 nf, H, W, C)
 *   cache_out bf16 (N,2,H,W,C) = P[:, nf:nf+2], or NULL
 * Requires C % 64 == 0 with C <= 2048. Outputs must not overlap the inputs or
 * each other (SGN_EALIAS); other shapes are SGN_EINVAL.
 */
int time_upsample_conv(const uint16_t* x, sgn_dims d, const uint16_t* cache_in,
                       const uint16_t* w, const float* bias, int first, uint16_t* y,
                       uint16_t* cache_out, hipStream_t stream);

/*
 * head_conv_d2s -- the decoder's output head: causal 3x3x3 convolution to 12
 * channels followed by a 2x2 depth-to-space into an RGB video.
 * Defined by: binding.cpp page, Decoder::output_head (norm + SiLU + causal pad,
 * the convolution to 12 = 3 x 2 x 2 channels, bias and clamp) and the video
 * write of decode_video.
 *
 *   o = causal_conv3d(x, cache_in, w, K=12, bias, fuse) in fp32 (before rounding)
 *   video[n, c, t, 2h+dy, 2w+dx] = RNE_bf16( clamp?( o[n,t,h,w, 4c+2dy+dx] ) )
 * with clamp to [-1, 1] when clamp != 0. video: bf16 (N,3,T,2H,2W) dense
 * (channels-first). cache_out as in causal_conv3d. Requires C % 64 == 0 with
 * C <= 4096 (C <= 2048 when fused).
 */
int head_conv_d2s(const uint16_t* x, sgn_dims d, const uint16_t* cache_in, const uint16_t* w,
                  const float* bias, const sgn_gn* fuse, int clamp, uint16_t* video,
                  uint16_t* cache_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SILUGN_H */
