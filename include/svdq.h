/*
 * svdq.h -- C ABI of the SVDQuant W4A4 linear layer for AMD Instinct MI355X
 * (gfx950).
 *
 * The layer computes
 *
 *     Y = X^ L1 L2 + dequant( Q4(X^) Q4(R)^T ) + b,
 *     X^ = X diag(lambda)^-1,   W^ = diag(lambda) W = L1 L2 + R
 *
 * (model card "svdq-int4-flux.1-dev", "Overview of SVDQuant" caption:
 * stage 2 migrates activation outliers into the weights, stage 3 splits the
 * weights by SVD into a 16-bit low-rank branch and a 4-bit residual; the
 * SVDQuant abstract: W4A4 with a high-precision low-rank branch).
 *
 * It runs as two fused kernels (same card, Nunchaku engine caption (b)):
 *   svdq_quantize_act_lora_down  smoothing + 4-bit activation quantization +
 *                                down projection X^ L1, reading X once;
 *   svdq_gemm_w4a4_lora_up       4-bit GEMM + per-group dequant + up
 *                                projection + bias, writing Y once.
 * The weights are packed offline on the CPU by svdq_pack_weights.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All buffers are allocated and owned by the caller.  The library keeps
 *    no per-call state and allocates nothing on the two hot calls.  Host
 *    pointers are marked (host), device pointers (dev).
 *  - Matrices are dense, row-major, contiguous.  bf16 and fp16 values are
 *    passed as their 16-bit patterns.
 *  - W is given in nn.Linear layout [N][K] (out x in); the blog "Nunchaku
 *    4-bit inference in Diffusers" ("Introducing Nunchaku Lite") replaces
 *    nn.Linear modules with the quantized layer.  The low-rank factors are
 *    stored the same way: lora_down = L1^T as [rank][K] and lora_up = L2^T
 *    as [N][rank], i.e. the weights of the two small linears K->rank and
 *    rank->N.
 *  - INT4 codes, q in [-7, 7]: 4 bits each, rows of K/2 bytes, in units of
 *    16 consecutive k stored as two little-endian 32-bit words I0, I1.
 *    Code q has the 6-bit image 32 [q < 0] + |q| (sign in bit 5, |q| in
 *    bits 0-2, bits 3-4 zero: the FP6 E2M3 pattern of q/8); image j of a
 *    unit sits at bits 6j..6j+5 of the 96-bit string D0 | D1<<32 | D2<<64,
 *    and I0 = D0 | (D2 & 0x18618618), I1 = D1 | (D2 & 0x86186186) (the
 *    masks are the zero bits 3-4 of the images in D0 and D1, which together
 *    are the data bits of D2).  Zero carries no sign.
 *    INT4 scales: fp16, one per 64 consecutive k of a row, group-major
 *    [K/64][rows].  MXFP4 codes: E2M1 nibbles (sign in bit 3), code k in
 *    the low nibble of byte k/2 when k is even;
 *    MXFP4 scales: E8M0 bytes, one per 32 k, group-major [K/32][rows].
 *  - Shapes: M, N >= 1 (any value); K >= 64 and K % 64 == 0 for INT4,
 *    K % 128 == 0 for MXFP4; rank == 0 (no low-rank branch) or a multiple of
 *    16, at most 256 and at most min(K, N).  The GEMM calls address each
 *    4-bit operand and its scale array with 32-bit byte offsets: rows * K/2
 *    code bytes and the scale bytes of X (rows = M) and of W (rows = N)
 *    must each stay below 2^31, else SVDQ_ERR_SHAPE (M or N up to ~349,000
 *    at K = 12288).
 *  - Device pointers must be 16-byte aligned.
 *  - Errors: arguments and the device are checked before anything is
 *    launched and reported as a status code; nothing is thrown across the
 *    ABI.  A launch failure returns SVDQ_ERR_HIP.  A device that is not
 *    gfx950 (or no device) gives SVDQ_ERR_UNSUPPORTED_DEVICE, never a wrong
 *    result: the blog's "Hardware support" section has the loader check the
 *    GPU generation and raise a clear error instead of producing wrong
 *    outputs.
 *  - The hot calls enqueue on `stream` (a hipStream_t; NULL = the default
 *    stream of the current device) and never synchronize.
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define SVDQ_API __attribute__((visibility("default")))
#else
#define SVDQ_API
#endif

#define SVDQ_OK                       0
#define SVDQ_ERR_INVALID_ARG         -1   /* NULL or misaligned pointer, bad enum */
#define SVDQ_ERR_SHAPE               -2   /* M, N, K or rank outside the rules above */
#define SVDQ_ERR_UNSUPPORTED_DEVICE  -3   /* no gfx950 device */
#define SVDQ_ERR_HIP                 -4   /* a HIP runtime call or launch failed */

#define SVDQ_INT4   0   /* int4 codes, groups of 64 along K, fp16 scales */
#define SVDQ_MXFP4  1   /* FP4 E2M1 codes, blocks of 32 along K, E8M0 scales */

/* Library version, major*10000 + minor*100 + patch. */
SVDQ_API int svdq_version(void);

/* Static text for a status code (never NULL). */
SVDQ_API const char* svdq_status_string(int status);

/* SVDQ_OK if HIP device `device` exists and is a gfx950, else
 * SVDQ_ERR_UNSUPPORTED_DEVICE.  The answer is cached per device. */
SVDQ_API int svdq_device_check(int device);

/* Byte sizes of the packed weight buffers for (K, N, rank, precision):
 * out_bytes[0] smooth_inv, [1] lora_down, [2] lora_up, [3] wq, [4] ws.
 * (host) out_bytes must hold 5 entries. */
SVDQ_API int svdq_packed_sizes(int K, int N, int rank, int precision, size_t* out_bytes);

/* Byte sizes of the activation buffers for (M, K, rank, precision):
 * out_bytes[0] xq, [1] xs, [2] lora_act.  (host) out_bytes holds 3 entries. */
SVDQ_API int svdq_act_sizes(int M, int K, int rank, int precision, size_t* out_bytes);

/* Offline pack, on the CPU (all pointers host).
 *
 * Stage 2 (smoothing): lambda_j = sqrt(max(act_absmax_j, 1e-5)) /
 * sqrt(max(max_n |W[n][j]|, 1e-5)) in fp64 (migration strength 0.5; the
 * pages give no formula) and smooth_inv_j = fp32(1/lambda_j).
 * W^ = W / smooth_inv in fp64.  Stage 3: top-`rank` SVD of W^ =
 * U S V^T by subspace iteration on the Gram matrix of the smaller side;
 * L1 = bf16(fp32(U_r S_r)), L2 = bf16(fp32(V_r^T)); residual
 * R = fp32(W^ - L1 L2) with the rounded factors; R quantized per output
 * channel with the layer's 4-bit rule.
 *
 *   w_bf16      [N][K] bf16 bits        nn.Linear weight
 *   act_absmax  [K] fp32                max |X[:, j]| of calibration data
 *   smooth_inv  [K] fp32                out
 *   lora_down   [rank][K] bf16          out (L1^T); may be NULL if rank == 0
 *   lora_up     [N][rank] bf16          out (L2^T); may be NULL if rank == 0
 *   wq          [N][K/2] uint8          out, packed codes of R
 *   ws          [K/64][N] fp16 (INT4) or [K/32][N] uint8 E8M0 (MXFP4), out
 *   r_out       [K][N] fp32             out, the unquantized residual; may be NULL
 * Threads: SVDQ_NUM_THREADS, else OMP_NUM_THREADS, else the host's cores
 * (at most 64). */
SVDQ_API int svdq_pack_weights(const uint16_t* w_bf16, const float* act_absmax,
                      int K, int N, int rank, int precision,
                      float* smooth_inv, uint16_t* lora_down, uint16_t* lora_up,
                      uint8_t* wq, void* ws, float* r_out);

/* Merge an off-the-shelf LoRA (Y += X A B) into the packed 16-bit branch,
 * on the CPU, without touching the 4-bit residual (SVDQuant abstract: the
 * engine supports low-rank adapters without re-quantization).  The branch
 * reads X^ = X diag(smooth_inv), so A is folded with 1/smooth_inv:
 * L1' = [L1 | A diag(1/smooth_inv)], L2' = [L2 ; B]; each folded element is
 * a[k][j] / smooth_inv[k] in fp64, rounded to fp32, then to bf16 (RNE).
 *
 *   lora_down      [rank][K] bf16        from svdq_pack_weights; NULL if rank == 0
 *   lora_up        [N][rank] bf16        from svdq_pack_weights; NULL if rank == 0
 *   smooth_inv     [K] fp32              from svdq_pack_weights
 *   a              [K][lora_rank] bf16   adapter down factor
 *   b              [lora_rank][N] bf16   adapter up factor
 *   lora_down_out  [rank+lora_rank][K] bf16, out (caller-allocated)
 *   lora_up_out    [N][rank+lora_rank] bf16, out (caller-allocated)
 * rank + lora_rank must meet the hot calls' rank rule (a multiple of 16, at
 * most 256 and at most min(K, N)), else SVDQ_ERR_SHAPE.  All pointers host;
 * the outputs must not overlap the inputs. */
SVDQ_API int svdq_merge_lora(const uint16_t* lora_down, const uint16_t* lora_up, int rank,
                             const float* smooth_inv, const uint16_t* a, const uint16_t* b,
                             int lora_rank, int K, int N,
                             uint16_t* lora_down_out, uint16_t* lora_up_out);

/* Fused kernel 1 (Nunchaku engine caption (b): the down projection and the
 * quantizer share their input, so X is read once).
 *
 *   x          (dev) [M][K] bf16        activations
 *   smooth_inv (dev) [K] fp32           from svdq_pack_weights
 *   lora_down  (dev) [rank][K] bf16     L1^T; ignored if rank == 0
 *   xq         (dev) [M][K/2] uint8     out, 4-bit codes of X^
 *   xs         (dev) [K/64][M] fp16 (INT4) | [K/32][M] E8M0 (MXFP4), out
 *   lora_act   (dev) [M][rank] fp32     out, X^ L1 (fp32 accumulation);
 *                                       ignored if rank == 0
 * X^ = bf16(fp32(x * smooth_inv)) is rounded once and feeds both branches.
 * INT4 rule per 64-group of a row: s = fp16(fp32(amax/7)) (round to
 * nearest even, saturating at 65504), s == 0 -> codes 0, else
 * q = clamp(rint(fp32(x^ * fp32(1/s))), -7, 7), ties to even.
 * MXFP4 rule per 32-block (OCP Microscaling v1.0): amax == 0 -> byte 0 and
 * codes 0; else e = clamp(floor(log2 amax) - 2, -127, 127) from the fp32
 * exponent field, byte e + 127, code = E2M1(x^ / 2^e) rounded to nearest
 * (ties to the even code, saturating at 6); zero magnitudes carry no sign.
 * lora_act partials of several workgroups may be summed with fp32 atomics,
 * so its last bits can differ between calls. */
SVDQ_API int svdq_quantize_act_lora_down(const void* x, int M, int K,
                                const float* smooth_inv, const void* lora_down,
                                int rank, int precision,
                                uint8_t* xq, void* xs, float* lora_act,
                                void* stream);

/* Fused kernel 2 (Nunchaku engine caption (b): the up projection and the
 * 4-bit compute share their output, so Y is written once).
 *
 *   xq, xs     (dev) from svdq_quantize_act_lora_down
 *   wq, ws     (dev) from svdq_pack_weights
 *   lora_act   (dev) [M][rank] fp32; ignored if rank == 0
 *   lora_up    (dev) [N][rank] bf16 (L2^T); ignored if rank == 0
 *   bias       (dev) [N] bf16, or NULL for no bias
 *   y          (dev) [M][N] bf16        out
 * INT4: for every 64-group g the exact integer partial
 * P = sum_k qx qw is scaled by s_x[m,g] s_w[n,g] into fp32 accumulators;
 * the up projection bf16(lora_act) L2 and the bias are added in fp32 and Y
 * is rounded to bf16 once.  MXFP4: the E2M1 codes with their E8M0 block
 * scales go to the matrix core as they are (fp32 accumulation); up
 * projection, bias and rounding as for INT4. */
SVDQ_API int svdq_gemm_w4a4_lora_up(const uint8_t* xq, const void* xs,
                           const uint8_t* wq, const void* ws,
                           const float* lora_act, const void* lora_up,
                           const void* bias, void* y,
                           int M, int N, int K, int rank, int precision,
                           void* stream);

/* svdq_gemm_w4a4_lora_up with a caller workspace, for grids that leave the
 * device mostly idle (the token rows one of several GPUs holds when a batch
 * is split by rows).  Same operation and arguments as above (the Nunchaku
 * engine caption (b) of the "svdq-int4-flux.1-dev" card), plus:
 *   workspace (dev) workspace_bytes bytes, 16-byte aligned, owned by the
 *             caller; its contents on entry do not matter; it must not be
 *             used by another call that may run at the same time.
 * svdq_gemm_workspace_size gives the bytes this call can use for the
 * shape on the current device: 0 when the single-pass schedule runs
 * anyway.  With a workspace of that size an INT4 grid whose tiles fill
 * under half the workgroup slots (two per CU) and whose K loop has at
 * least 16 stages of 128 k is cut along K: each part writes fp32 tile
 * partials into the workspace, and a second kernel adds them in a fixed
 * order and applies the up projection, the bias and the single rounding to
 * bf16.  The result is deterministic, and within the same bounds as the
 * single-pass schedule: its fp32 sums run in a different order.  A NULL
 * or smaller workspace runs the single-pass schedule.  MXFP4 always runs
 * the single-pass schedule. */
SVDQ_API int svdq_gemm_workspace_size(int M, int N, int K, int precision, size_t* out_bytes);
SVDQ_API int svdq_gemm_w4a4_lora_up_ws(const uint8_t* xq, const void* xs,
                              const uint8_t* wq, const void* ws,
                              const float* lora_act, const void* lora_up,
                              const void* bias, void* y,
                              int M, int N, int K, int rank, int precision,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/* First layer of an MLP pair with its activation fused: the original
 * engine's model-specific paths include a fused GELU/MLP kernel (blog
 * "Nunchaku 4-bit inference in Diffusers", "Introducing Nunchaku Lite").
 * The activation is the tanh-form GELU of FLUX's MLP (a reading; the pages
 * do not name the form).  INT4 only.
 *
 * svdq_gemm_w4a4_lora_up_gelu: as svdq_gemm_w4a4_lora_up, but y receives
 * bf16(GELU(Y)) with Y the layer's bf16 output (rounded first, as the next
 * layer would read it) and GELU(y) = 0.5 y (1 + tanh(sqrt(2/pi) (y +
 * 0.044715 y^3))) evaluated in fp32.
 *
 * svdq_mlp_gemm_gelu_quant: writes no Y at all.  The tile of X2 =
 * bf16(GELU(Y)) goes straight into the second layer's first kernel
 * (svdq_quantize_act_lora_down's rule with smooth_inv2 and lora_down2):
 *   smooth_inv2 (dev) [N] fp32            second layer's smoothing
 *   lora_down2  (dev) [rank2][N] bf16     second layer's L1^T; ignored if rank2 == 0
 *   xq2         (dev) [M][N/2] uint8      out, 4-bit codes of X2^
 *   xs2         (dev) [N/64][M] fp16      out
 *   lora_act2   (dev) [M][rank2] fp32     out (cleared, then summed over the
 *                                         output tiles with fp32 atomics)
 * N % 128 == 0 (a 64-column group lies inside one 128-column tile), else
 * SVDQ_ERR_SHAPE; rank2 follows the rank rule with K = N.  Other arguments
 * as for svdq_gemm_w4a4_lora_up. */
SVDQ_API int svdq_gemm_w4a4_lora_up_gelu(const uint8_t* xq, const void* xs,
                           const uint8_t* wq, const void* ws,
                           const float* lora_act, const void* lora_up,
                           const void* bias, void* y,
                           int M, int N, int K, int rank, int precision,
                           void* stream);
SVDQ_API int svdq_mlp_gemm_gelu_quant(const uint8_t* xq, const void* xs,
                           const uint8_t* wq, const void* ws,
                           const float* lora_act, const void* lora_up,
                           const void* bias, int M, int N, int K, int rank,
                           const float* smooth_inv2, const void* lora_down2, int rank2,
                           int precision, uint8_t* xq2, void* xs2, float* lora_act2,
                           void* stream);

/* W4A16 comparison layer: 4-bit weights, bf16 activations (the 4-bit
 * weight-only baseline that the SVDQuant abstract measures W4A4 against:
 * 3.0x with INT4, 3.1x with NVFP4, whole model).  The weights carry the
 * layer's INT4 rule per output channel in groups of 64 along K, with no
 * smoothing and no low-rank branch.
 *
 * svdq_pack_w4a16 (host): w_bf16 [N][K] -> wq [N][K/2] (same code layout as
 *   the W4A4 codes), ws [K/64][N] fp16.  K % 64 == 0.
 * svdq_gemm_w4a16 (device): y [M][N] bf16 = bf16(x . (q s)^T + bias); x
 *   bf16 [M][K], bias bf16 [N] or NULL.  Each weight q*s is rounded to bf16
 *   once, the products accumulate in fp32. */
SVDQ_API int svdq_pack_w4a16(const uint16_t* w_bf16, int K, int N, uint8_t* wq, void* ws);
SVDQ_API int svdq_gemm_w4a16(const void* x, const uint8_t* wq, const void* ws,
                             const void* bias, void* y, int M, int N, int K, void* stream);

/* Unfused baseline of the same layer, for measuring what the two fusions
 * save (model card "svdq-int4-flux.1-dev", Nunchaku engine caption (a): a
 * naive low-rank branch as separate kernels costs an extra 16-bit read of
 * X in the down projection and an extra 16-bit write of Y in the up
 * projection).  Four kernels on `stream`: quantize (writes xq, xs),
 * down projection (reads X again, writes lora_act), 4-bit GEMM (writes Y
 * in bf16) and up projection (reads Y, adds bf16(lora_act) L2 and the
 * bias, writes Y).  Arguments, layouts and errors as for the two fused
 * calls; xq, xs and lora_act are caller-owned intermediates.  Results equal
 * the fused path's up to the second bf16 rounding of Y.  INT4 only. */
SVDQ_API int svdq_unfused_linear(const void* x, int M, int K,
                        const float* smooth_inv, const void* lora_down, int rank,
                        const uint8_t* wq, const void* ws,
                        const void* lora_up, const void* bias, int N, int precision,
                        uint8_t* xq, void* xs, float* lora_act, void* y,
                        void* stream);

/* svdq_unfused_linear for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same four kernels and the same result, without the xq, xs and lora_act
 * workspace arguments.  Those intermediates live in one device array of
 * 32 MiB (SVDQ_NOALLOC_SCRATCH_BYTES) that the library holds on every GPU
 * it runs on until the process ends; the call itself allocates nothing.
 * The array needs M*K/2 + (K/64)*M*2 + M*rank*4 bytes, each part rounded up
 * to 256 bytes (FLUX.1's 12288 -> 3072 MLP layer at M = 4608, rank 32:
 * ~30.7 MB); a larger call returns SVDQ_ERR_SHAPE.  Every call on a GPU
 * shares that GPU's array and leaves its contents behind, so calls that
 * overlap on one GPU (two streams, two threads) race and must be
 * serialized by the caller.  INT4 only; other arguments and errors as for
 * svdq_unfused_linear. */
#define SVDQ_NOALLOC_SCRATCH_BYTES (32u << 20)
SVDQ_API int svdq_unfused_linear_noalloc(const void* x, int M, int K,
                        const float* smooth_inv, const void* lora_down, int rank,
                        const uint8_t* wq, const void* ws,
                        const void* lora_up, const void* bias, int N, int precision,
                        void* y, void* stream);

/* Measurement hook: the dense matrix-core rate this GPU sustains.  Each of
 * `blocks` workgroups (4 waves; launch two per CU) issues 8 * iters
 * independent v_mfma_scale_f32_32x32x64_f8f6f4 per wave, with FP8 operands
 * (precision SVDQ_INT4: 16 passes per instruction, the matrix time the INT4
 * GEMM spends per K-group and 32x32 tile as one 8-pass FP6 product plus one
 * 8-pass rank-1 scale product) or FP4 operands (SVDQ_MXFP4).
 * Ops per launch = blocks * 4 * 8 * iters * 131072;
 * the caller times it.  out (dev) [blocks] fp32 receives one checksum per
 * workgroup.  blocks, iters >= 1. */
SVDQ_API int svdq_bench_mfma_ceiling(int precision, int blocks, int iters, float* out, void* stream);

/* Test hook: the exact per-group integer partials of the INT4 GEMM for the
 * output window rows [m0, m0+mt) x columns [n0, n0+nt).  It runs the INT4
 * GEMM kernel of svdq_gemm_w4a4_lora_up in a test mode that shares its code
 * loader, the conversion of the codes for the matrix core, the LDS layout
 * and the matrix instruction that forms each group's partial; the scale
 * handling (the per-group dequant into the accumulators), the up
 * projection and the epilogue are replaced by a store of the partials.
 *   out (dev) [mt][nt][K/64] int32.  mt, nt >= 1; the window must lie
 *   inside [0, M) x [0, N). */
SVDQ_API int svdq_debug_group_partials(const uint8_t* xq, const uint8_t* wq,
                              int M, int N, int K,
                              int m0, int n0, int mt, int nt,
                              int32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H */
