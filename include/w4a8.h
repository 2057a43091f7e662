/*
 * w4a8.h -- C ABI of libw4a8.so: the MXFP4 W4A8 linear layer on MI355X (gfx950).
 *
 * Two halves, as on the pages:
 *   load time  NVFP4 -> MXFP4 requantization of a (possibly merged) linear
 *              ("radiance_nvfp4.py", dequant_nvfp4 / quant_mxfp4 / requant_rows /
 *              RadianceNvfp4ToMxfp4.process_weights_after_loading), and the
 *              int4 group-128 load-time check and transpose
 *              ("radiance_autoround.py", process_weights_after_loading);
 *   run time   per-token fp8 (e4m3) activation quantization and the block-scaled
 *              GEMM of fp8 activations against e2m1 weights with e8m0 scales
 *              ("vllm-radiance (MXFP4)", How the MXFP4 path works: The W4A8
 *              fp8-WMMA kernel), and the int4 g128 symmetric variant
 *              ("radiance_autoround.py", autoround_linear, _exact_ref).
 *
 * Conventions (all entry points):
 *   - Pointers named d_* / documented "device" are device (HBM) pointers owned by
 *     the caller; the library never allocates or frees device memory.  Host
 *     arrays are named h_*.  Every compute call is asynchronous on `stream`
 *     (a hipStream_t; NULL = the null stream) and returns after enqueueing,
 *     except w4a8_int4g128_prepare, which synchronizes `stream` (load time).
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     non-OK status nothing has been enqueued (W4A8_ERR_HIP aside: a launch
 *     or runtime call failed, and earlier work of the same call may have run).
 *   - Nothing is printed, nothing throws, no environment variable is read.
 *   - Numbers: e2m1 codes are 4 bits, bit 3 = sign, bits 0-2 index
 *     {0, .5, 1, 1.5, 2, 3, 4, 6}; two per byte, even k in the low nibble.
 *     e8m0 byte b means 2^(b-127).  e4m3 is OCP E4M3FN (max 448, 0x7F/0xFF
 *     NaN).  bf16 and fp16 travel as their raw 16-bit patterns (uint16_t).
 *   - Row-major throughout; leading dimensions are the logical widths unless a
 *     stride argument says otherwise.
 *   - Inputs must be finite (no NaN/Inf e4m3 scale bytes or activations); the
 *     result for non-finite inputs is unspecified.
 *   - Calls that share a workspace must not overlap in time (same stream or
 *     explicitly ordered).
 */
#ifndef W4A8_H
#define W4A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4A8_OK = 0,
    W4A8_ERR_INVALID_ARG = 1,       /* null pointer, size < 0 or == 0 where >= 1 is needed,
                                       unknown enum value, non-positive or non-finite divisor */
    W4A8_ERR_UNSUPPORTED_SHAPE = 2, /* K % 32 != 0; int4: K % 128 != 0 or N % 8 != 0;
                                       partition rows that do not add up; ldx < K */
    W4A8_ERR_WORKSPACE = 3,         /* workspace missing, too small or not 256-byte aligned */
    W4A8_ERR_ASYMMETRIC = 4,        /* int4: a qzeros word differs from 0x77777777 */
    W4A8_ERR_HIP = 5                /* a HIP runtime call or kernel launch failed */
} w4a8_status;

/* Block-exponent rule of the requant ("radiance_nvfp4.py", _block_exponent,
 * quant_mxfp4 and the module docstring):
 *   OCP     e = floor(log2 amax) - 2: amax/2^e in [4, 8), the top of the block clips;
 *   NOCLIP  e = ceil(log2(amax/6)):    amax/2^e in (3, 6], nothing clips;
 *   MSE     of NOCLIP and NOCLIP-1, the one with the strictly smaller squared
 *           error of the block (ties keep NOCLIP) -- the pages' default.
 * Exponents are exact integer functions of amax (not a float log2), amax == 0
 * gives e = 0, e is clamped to [-127, 127]; under MSE a NOCLIP exponent of -127
 * is kept (NOCLIP-1 has no e8m0 byte). */
typedef enum { W4A8_EXP_OCP = 0, W4A8_EXP_NOCLIP = 1, W4A8_EXP_MSE = 2 } w4a8_exp_mode;

/* Weight formats accepted by the GEMMs (for workspace sizing). */
typedef enum {
    W4A8_WEIGHT_MXFP4 = 0,           /* [N, K/2] codes + [N, K/32] e8m0 */
    W4A8_WEIGHT_INT4G128 = 1,        /* [N, K/8] int32 (w4a8_int4g128_prepare) + fp16 scales */
    W4A8_WEIGHT_MXFP4_PREPARED = 2,  /* fragment order (w4a8_mxfp4_prepare) */
    W4A8_WEIGHT_INT4G128_PREPARED = 3, /* fragment order (w4a8_int4g128_prepare_fragments) */
    W4A8_W4A4_PREPARED = 4,           /* MXFP4 fragment order with MXFP4 activations
                                         (w4a8_w4a4_gemm_prepared) */
    W4A8_WEIGHT_INT4G128_ZP_PREPARED = 5, /* int4 g128 with zero points, fragment order
                                            (w4a8_int4g128_zp_prepare_fragments) */
    W4A8_WEIGHT_INT5G128_PREPARED = 6    /* int5 g128, fragment order (w4a8_int5g128_prepare_fragments) */
} w4a8_weight_kind;

/* ---------------------------------------------------------------------------
 * NVFP4 -> MXFP4 requantization of one linear layer.
 * Source: "radiance_nvfp4.py": dequant_nvfp4, e2m1_index, _block_exponent,
 * _encode_blocks, quant_mxfp4, requant_rows, and
 * RadianceNvfp4ToMxfp4.process_weights_after_loading (one global divisor per
 * partition of a merged linear, outputs concatenated in row order).
 *
 * Per element: w = RN32(e2m1(code) * RN32(e4m3(scale) / divisor_p)) (IEEE fp32
 * division, then the product); per 32-block along K: exponent by `mode`, codes
 * rounded to nearest e2m1 after dividing by 2^e (clamped to 6, ties to the even
 * code), sign bit only on nonzero codes, e8m0 byte = e + 127.  The mse squared
 * error of a block is summed in fp32 in element order, each square rounded
 * first.  Codes and e8m0 bytes are bit-exact functions of the inputs.
 *
 *   d_nv_packed   device uint8 [rows, K/2]   NVFP4 codes, even k in the low nibble
 *   d_nv_scale    device uint8 [rows, K/16]  e4m3 scale per 16 elements
 *   h_part_rows   host int64 [n_parts]       rows of each partition, in order;
 *                                            rows = sum(h_part_rows)
 *   h_part_divisor host float [n_parts]      each partition's global scale as
 *                                            stored (6*448/amax): a divisor, > 0
 *   n_parts       >= 1
 *   K             elements per row, K % 32 == 0, K >= 32
 *   mode          w4a8_exp_mode
 *   row_chunk     rows per pass of the page's requant_rows (its ROW_CHUNK is
 *                 4096; 0 = one pass per partition).  Each block is encoded on
 *                 its own, so results do not depend on it, and every pass of
 *                 every partition runs in one kernel launch (one per group of
 *                 16 partitions).
 *   d_mx_packed   device uint8 [rows, K/2]   out: e2m1 codes, even k low nibble
 *   d_mx_e8m0     device uint8 [rows, K/32]  out: block exponents + 127
 *   d_err_stats   device double [2*n_parts] or NULL: out, per partition
 *                 {sum of chosen block squared errors, sum of w^2}, from which
 *                 relRMS = sqrt(sum err / sum w^2) as the page logs it.  Filled
 *                 with atomics: the low bits depend on summation order.
 * Inputs and outputs must not overlap.  Errors: INVALID_ARG (null pointers,
 * n_parts < 1, a divisor <= 0 or not finite, bad mode, row_chunk < 0, a
 * negative partition), UNSUPPORTED_SHAPE (K % 32), HIP. */
w4a8_status w4a8_requant_nvfp4_to_mxfp4(
    const uint8_t *d_nv_packed, const uint8_t *d_nv_scale,
    const int64_t *h_part_rows, const float *h_part_divisor, int n_parts,
    int64_t K, w4a8_exp_mode mode, int64_t row_chunk,
    uint8_t *d_mx_packed, uint8_t *d_mx_e8m0, double *d_err_stats, void *stream);

/* ---------------------------------------------------------------------------
 * bf16 and fp8-per-channel weights -> MXFP4 at load time, with the encoder of
 * w4a8_requant_nvfp4_to_mxfp4 (same exponent rules, code rounding, signs and
 * statistics).  Source: "radiance_nvfp4.py", RadianceBf16ToMxfp4 (the bf16
 * weight itself, widened exactly) and RadianceFp8ChannelToMxfp4 (each e4m3
 * weight times its row's fp32 scale, one rounded fp32 product) with
 * quant_mxfp4 / requant_rows (the page's row chunks change no output, so one
 * pass covers the weight).
 *   d_w_bf16      device uint16 [rows, K] bf16 bits, 16-byte aligned
 *   d_w_e4m3      device uint8 [rows, K] OCP e4m3 codes, 16-byte aligned
 *   d_row_scale   device float [rows], 4-byte aligned
 *   rows          >= 0;  K % 32 == 0 and rows * K/32 < 2^32 (else
 *                 UNSUPPORTED_SHAPE)
 *   mode          w4a8_exp_mode; the page's schemes use mse
 *   d_mx_packed   device uint8 [rows, K/2] out (16-byte aligned), d_mx_e8m0
 *                 device uint8 [rows, K/32] out
 *   d_err_stats   device double [2] or NULL: out {sum of chosen block squared
 *                 errors, sum of w^2} (atomics: low bits depend on order)
 * Non-finite inputs are excluded (unspecified results).  Inputs and outputs
 * must not overlap.  Errors: INVALID_ARG, UNSUPPORTED_SHAPE, HIP. */
w4a8_status w4a8_quant_bf16_to_mxfp4(const uint16_t *d_w_bf16, int64_t rows, int64_t K, w4a8_exp_mode mode,
                                     uint8_t *d_mx_packed, uint8_t *d_mx_e8m0, double *d_err_stats,
                                     void *stream);
w4a8_status w4a8_quant_fp8ch_to_mxfp4(const uint8_t *d_w_e4m3, const float *d_row_scale, int64_t rows,
                                      int64_t K, w4a8_exp_mode mode, uint8_t *d_mx_packed,
                                      uint8_t *d_mx_e8m0, double *d_err_stats, void *stream);

/* ---------------------------------------------------------------------------
 * The three load-time encoders above writing the GEMM's prepared layout
 * directly (the matrix-core fragment order of w4a8_mxfp4_prepare), so that a
 * checkpoint goes to the fast layout in one pass, with no row-major MXFP4 in
 * between.  Source: "radiance_nvfp4.py", module docstring (the weight is
 * requantized once at load, then handed to the fp8-WMMA GEMM, which reads
 * fragment-order weights) and the three schemes'
 * process_weights_after_loading.  Codes and e8m0 bytes are bit for bit those
 * of w4a8_mxfp4_prepare applied to the row-major encoder's output (the same
 * per-block rule), padding included (rows to 16, steps to a multiple of 4:
 * code 0, e8m0 127).
 *   arguments as the row-major encoders, K % 128 == 0 (else
 *   UNSUPPORTED_SHAPE), n_parts <= 16; rows = the partitions' rows summed
 *   d_w_prepared, d_s_prepared  out, sized by w4a8_mxfp4_prepared_bytes(rows,
 *                 K), 16- and 4-byte aligned
 * No statistics (the row-major entry points report them); no row chunking
 * (it changes no output).  Inputs and outputs must not overlap.  Errors:
 * INVALID_ARG, UNSUPPORTED_SHAPE, HIP. */
w4a8_status w4a8_requant_nvfp4_to_mxfp4_prepared(const uint8_t *d_nv_packed, const uint8_t *d_nv_scale,
                                                 const int64_t *h_part_rows, const float *h_part_divisor,
                                                 int n_parts, int64_t K, w4a8_exp_mode mode,
                                                 uint8_t *d_w_prepared, uint8_t *d_s_prepared, void *stream);
w4a8_status w4a8_quant_bf16_to_mxfp4_prepared(const uint16_t *d_w_bf16, int64_t rows, int64_t K,
                                              w4a8_exp_mode mode, uint8_t *d_w_prepared, uint8_t *d_s_prepared,
                                              void *stream);
w4a8_status w4a8_quant_fp8ch_to_mxfp4_prepared(const uint8_t *d_w_e4m3, const float *d_row_scale, int64_t rows,
                                               int64_t K, w4a8_exp_mode mode, uint8_t *d_w_prepared,
                                               uint8_t *d_s_prepared, void *stream);

/* ---------------------------------------------------------------------------
 * Dynamic per-token fp8 activation quantization.
 * Source: "radiance_autoround.py", autoround_linear (per-token dynamic e4m3
 * with one fp32 scale per row, consumed by the W4A8 GEMM).  The pages leave the
 * arithmetic to a library op; this is the plain reading:
 *   s_m = RN32(amax_k |x[m,k]| / 448)   (s_m = 1 for an all-zero row)
 *   x8[m,k] = e4m3 RNE of RN32(x[m,k] / s_m), saturating at +-448, sign kept.
 * Codes and scales are bit-exact functions of the inputs.
 *   d_x_bf16   device uint16 [M, ldx]  bf16 bits; only columns < K are read
 *   M >= 1, K >= 1, ldx >= K
 *   d_x_fp8    device uint8 [M, K]     out: e4m3 codes
 *   d_x_scale  device float [M]        out: per-token scales
 * Errors: INVALID_ARG, UNSUPPORTED_SHAPE (ldx < K), HIP. */
w4a8_status w4a8_quant_act_fp8_per_token(
    const uint16_t *d_x_bf16, int64_t M, int64_t K, int64_t ldx,
    uint8_t *d_x_fp8, float *d_x_scale, void *stream);

/* ---------------------------------------------------------------------------
 * GEMM workspace.  The decode band may split K across workgroups; the fp32
 * partial sums live in a caller-owned workspace ("radiance_autoround.py": the
 * split-K scratch is registered once, before any launch, because allocating
 * inside a captured graph is illegal).  In the decode kernels the last split
 * of an output block to arrive adds them in split order ("vllm-radiance
 * (MXFP4)", The W4A8 fp8-WMMA kernel), counting arrivals in one word per
 * block at the start of the workspace; the tile kernels' splits are added by
 * a second kernel on the same stream.  Zero the workspace once before its
 * first use (w4a8_workspace_init, or any zero fill): every call leaves the
 * counters at zero again, so it needs no clearing between calls.  Calls that
 * overlap on one workspace race.
 *
 * w4a8_gemm_workspace_bytes: bytes needed by every GEMM call with the given
 * N, K and kind and any M <= M_max (K splits; for W4A8_WEIGHT_MXFP4 and
 * W4A8_WEIGHT_INT4G128 with M_max > 64 also the weight repacked into fragment
 * order; for W4A8_WEIGHT_MXFP4_PREPARED on a wide layer with M_max > 16 the
 * linear's step-major copy of the codes; 0 if no call needs any).  Pure
 * host function, never fails (returns 0 for invalid sizes).
 * w4a8_workspace_init: zero a workspace of `bytes` bytes (device, 256-byte
 * aligned) on `stream`.  Errors: INVALID_ARG, WORKSPACE, HIP. */
size_t      w4a8_gemm_workspace_bytes(int64_t M_max, int64_t N, int64_t K, w4a8_weight_kind kind);
w4a8_status w4a8_workspace_init(void *d_ws, size_t bytes, void *stream);

/* ---------------------------------------------------------------------------
 * MXFP4 W4A8 GEMM:  out[m,n] = bf16_RNE( s_m * sum_k e4m3(x8[m,k]) * e2m1(w[n,k])
 *                                              * 2^(E[n, k/32] - 127) )
 * Source: "vllm-radiance (MXFP4)", How the MXFP4 path works: The W4A8 fp8-WMMA
 * kernel (fp8 activations, e8m0 folded into the product, separate decode and
 * prefill tilings, split-K decode whose last-arriving workgroup reduces in
 * place); layouts from "radiance_nvfp4.py" module docstring.  Accumulation is
 * fp32 (MFMA), then one scaling by s_m and one rounding to bf16.  No bias (the
 * caller adds it, as "radiance_autoround.py" apply does).  Results are
 * deterministic: identical bits on every call with the same inputs.
 *   d_x_fp8    device uint8 [M, K]      e4m3 activations (w4a8_quant_act_fp8_per_token)
 *   d_x_scale  device float [M]         per-token scales
 *   d_w_packed device uint8 [N, K/2]    e2m1 codes, even k in the low nibble
 *   d_w_e8m0   device uint8 [N, K/32]   block exponents + 127
 *   d_out      device uint16 [M, N]     out: bf16 bits
 *   M >= 1, N >= 1, K >= 32, K % 32 == 0
 *   d_ws, ws_bytes   workspace of at least w4a8_gemm_workspace_bytes(M, N, K,
 *                    W4A8_WEIGHT_MXFP4) bytes, initialized once; may be NULL/0
 *                    when that is 0.
 * Band: M <= 64 on wide layers (at least 1536 16-row tiles, at most 16 per
 * CU) with K a multiple of 1024 and d_w_e8m0 16-byte aligned runs the spread
 * tiles of w4a8_mxfp4_gemm_prepared on this layout directly (no workspace;
 * value identical to the prepared path); other M <= 64 the decode kernels
 * (weights streamed from HBM, split K).  M > 64 with K % 128 == 0 and
 * K < 2^24: each call repacks the weight into fragment order inside the
 * workspace (w4a8_mxfp4_prepare's layout, after the decode band's split-K
 * counters, which it leaves untouched), then runs the tile kernel of
 * w4a8_mxfp4_gemm_prepared (value identical to it); other M > 64 the
 * LDS-tiled kernel on this layout.  Errors: INVALID_ARG, UNSUPPORTED_SHAPE,
 * WORKSPACE, HIP. */
w4a8_status w4a8_mxfp4_gemm(
    const uint8_t *d_x_fp8, const float *d_x_scale,
    const uint8_t *d_w_packed, const uint8_t *d_w_e8m0, uint16_t *d_out,
    int64_t M, int64_t N, int64_t K, void *d_ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * MXFP4 weights in matrix-core fragment order (load time) and the GEMM on them.
 * Source: "vllm-radiance (MXFP4)", How the MXFP4 path works: the W4A8 kernel
 * consumes weights repacked at load time into the order of its matrix
 * instructions.  Here the order is that of the gfx950 16x16x128 block-scaled
 * MFMA with the weight as its e2m1 operand: per 16-row tile and 128-wide K step
 * one 1 KiB block (lane L = n + 16g holds row 16t+n, packed bytes 64s+16g..+16),
 * tiles major; e8m0 as one 256-byte block per tile and 4-step chunk (lane L's
 * dword byte u = e8m0 of row 16t+n, K-block 4(4c+u)+g).  Rows are padded to a
 * multiple of 16 and steps to a multiple of 4 (zero codes, e8m0 127).  The GEMM
 * result is identical in value to w4a8_mxfp4_gemm on the plain layout (same
 * products, fp32 accumulation; summation order may differ).
 *   w4a8_mxfp4_prepared_bytes: sizes of the two prepared buffers (host).
 *   w4a8_mxfp4_prepare: d_w_packed [N, K/2], d_w_e8m0 [N, K/32] -> d_w_prepared,
 *     d_s_prepared (caller-allocated, sizes above; 16- and 4-byte aligned).
 *   w4a8_mxfp4_gemm_prepared: as w4a8_mxfp4_gemm on prepared weights, any
 *     M >= 1.  Small M on narrow layers (fewer than 64 column tiles of 256)
 *     runs the split-K decode kernel to M = 8 and the register-streamed tiles
 *     for 9 <= M <= 40; wide layers (at least 1536 16-row tiles on 256 CUs, at
 *     most 16 per CU) at M <= 64 the spread tiles (one workgroup per CU, all
 *     of K, no workspace); larger M the tiled
 *     kernel (64/128/256 x 128/256 output tiles), which splits K across
 *     workgroups when it has fewer than 128 tiles (fp32 partials in the
 *     workspace, then a reduction kernel); 256 x 256 tiles that fill four or
 *     more whole rounds of workgroups but leave a part round run in two
 *     launches, the leading columns in whole rounds and the rest on
 *     narrower tiles (the same value per output).  A workspace sized
 *     with W4A8_WEIGHT_MXFP4_PREPARED for the largest M covers every case
 *     (many tiles need none).  Above the split-K decode kernel's range K must
 *     be < 2^24 (UNSUPPORTED_SHAPE): those kernels address a 256-row
 *     activation block with 32-bit offsets.
 * K % 128 == 0 (else UNSUPPORTED_SHAPE).  Errors: INVALID_ARG, UNSUPPORTED_SHAPE,
 * WORKSPACE, HIP. */
w4a8_status w4a8_mxfp4_prepared_bytes(int64_t N, int64_t K, size_t *h_w_bytes, size_t *h_s_bytes);
w4a8_status w4a8_mxfp4_prepare(const uint8_t *d_w_packed, const uint8_t *d_w_e8m0, int64_t N,
                               int64_t K, uint8_t *d_w_prepared, uint8_t *d_s_prepared, void *stream);
w4a8_status w4a8_mxfp4_gemm_prepared(const uint8_t *d_x_fp8, const float *d_x_scale,
                                     const uint8_t *d_w_prepared, const uint8_t *d_s_prepared,
                                     uint16_t *d_out, int64_t M, int64_t N, int64_t K, void *d_ws,
                                     size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * int4 group-128 symmetric (AutoGPTQ layout), load-time preparation.
 * Source: "radiance_autoround.py", module docstring and
 * AutoRoundLinearMethod.process_weights_after_loading: every qzeros word must
 * be 0x77777777 (zero point 8, so code c means c - 8); the weight is transposed
 * from the checkpoint's [K/8, N] to [N, K/8] so one row of N is contiguous.
 *   d_qweight_kn  device int32 [K/8, N]     nibble j of word i is k = 8i + j
 *   d_qzeros      device int32 [K/128, N/8]
 *   d_qweight_nk  device int32 [N, K/8]     out (unspecified on ASYMMETRIC)
 *   N % 8 == 0, K % 128 == 0, N >= 8, K >= 128
 * Synchronizes `stream` (the check result is read back).  Errors:
 * INVALID_ARG, UNSUPPORTED_SHAPE, ASYMMETRIC, HIP. */
w4a8_status w4a8_int4g128_prepare(
    const int32_t *d_qweight_kn, const int32_t *d_qzeros, int64_t N, int64_t K,
    int32_t *d_qweight_nk, void *stream);

/* int4 g128 W4A8 GEMM:
 *   out[m,n] = bf16_RNE( s_m * sum_k e4m3(x8[m,k]) * (c[n,k] - 8) * fp16(scales[k/128, n]) )
 * Source: "radiance_autoround.py", _exact_ref and autoround_linear (the same
 * launch convention as the MXFP4 GEMM; c - 8 is exact in e4m3, so the product
 * runs on the fp8 matrix cores with the group scale applied per 128-K group in
 * fp32).  Deterministic.
 *   d_qweight_nk  device int32 [N, K/8]  (from w4a8_int4g128_prepare)
 *   d_scales_f16  device uint16 [K/128, N]  fp16 bits
 *   others as w4a8_mxfp4_gemm; N % 8 == 0, K % 128 == 0; workspace sized with
 *   W4A8_WEIGHT_INT4G128.  M <= 64: the decode kernel on this layout; M > 64
 *   (K < 2^24): each call repacks the weight into fragment order inside the
 *   workspace (w4a8_int4g128_prepare_fragments' layout, after the decode
 *   band's split-K counters, which it leaves untouched), then runs the tile
 *   kernel of w4a8_int4g128_gemm_prepared (value identical to it).
 *   Errors: INVALID_ARG, UNSUPPORTED_SHAPE, WORKSPACE, HIP. */
w4a8_status w4a8_int4g128_gemm(
    const uint8_t *d_x_fp8, const float *d_x_scale,
    const int32_t *d_qweight_nk, const uint16_t *d_scales_f16, uint16_t *d_out,
    int64_t M, int64_t N, int64_t K, void *d_ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * W4A4: MXFP4 activations x MXFP4 weights (prepared by w4a8_mxfp4_prepare) on
 * the fp4 x fp4 block-scaled matrix instructions.  Source: "vllm-radiance
 * (MXFP4)", the Quark MXFP4 checkpoints' declared numerics (MXFP4 weights and
 * activations, group 32, e8m0 scales) that the page's W4A8 kernel departs
 * from.  Activations are quantized per token and 32-block by the OCP rule:
 * w4a8_quant_bf16_to_mxfp4 with W4A8_EXP_OCP on the [M, K] bf16 activations
 * (the pages do not print the activation quantizer; this is the OCP MX
 * reading).
 *   out[m, n] = bf16( sum_k e2m1(x[m,k]) 2^(Ex[m,k/32]-127) e2m1(w[n,k]) 2^(Ew[n,k/32]-127) )
 * with fp32 accumulation (summation order differs from a sequential sum).
 *   d_x_fp4   device uint8 [M, K/2] e2m1 codes (even k low nibble), 16-byte aligned
 *   d_x_e8m0  device uint8 [M, K/32], 4-byte aligned
 *   d_w_prepared, d_s_prepared: from w4a8_mxfp4_prepare
 *   d_out     device bf16 [M, N], 8-byte aligned
 * Any M >= 1; K % 128 == 0 and K < 2^24 (else UNSUPPORTED_SHAPE).  Wide
 * layers (at least 1536 16-row tiles on 256 CUs, at most 16 per CU) at
 * M <= 64: the spread tiles (one workgroup per CU over all of K, no
 * workspace).  Otherwise M <= 32: the split-K decode kernel
 * (weights streamed once, activations resident in LDS, K split across
 * workgroups when they do not fit); above, a tiled kernel (128- or 256-row
 * tiles, 256 wide), K split across workgroups when its tiles are fewer than
 * 128.  A split writes fp32 partials to the workspace (size it
 * with W4A8_W4A4_PREPARED for the largest M), then a reduction.  Errors:
 * INVALID_ARG, UNSUPPORTED_SHAPE, WORKSPACE, HIP. */
w4a8_status w4a8_w4a4_gemm_prepared(const uint8_t *d_x_fp4, const uint8_t *d_x_e8m0,
                                    const uint8_t *d_w_prepared, const uint8_t *d_s_prepared, uint16_t *d_out,
                                    int64_t M, int64_t N, int64_t K, void *d_ws, size_t ws_bytes, void *stream);

/* int4 g128 weights in matrix-core fragment order (load time) and the GEMM on
 * them.  Source: "radiance_autoround.py", as w4a8_int4g128_gemm above, with the
 * load-time repack of "vllm-radiance (MXFP4)", How the MXFP4 path works.  The
 * layout is the MXFP4 fragment order: one 1 KiB block per 16-row tile t and
 * 128-wide K step s, tiles major; lane L = n + 16g holds 16 bytes of codes of
 * row 16t+n: words 16s+4g .. 16s+4g+3 of the checkpoint layout (k = 128s+32g
 * .. +31, nibble j of a word is k = 8i + j).  Row scales: fp16 [tile][4-step
 * chunk][row / 4][step][row % 4] (128 B per tile and chunk; the 16 lanes
 * that share four output rows read 32 contiguous bytes).  Rows are padded to 16 and steps to a multiple of
 * 4 (code 8, scale 0).  The result equals
 * w4a8_int4g128_gemm's in value (fp32 accumulation; summation order may
 * differ).
 *   w4a8_int4g128_prepared_bytes: sizes of the two buffers (host).
 *   w4a8_int4g128_prepare_fragments: checkpoint qweight [K/8, N], qzeros
 *     [K/128, N/8] (all 0x77777777, else ASYMMETRIC), scales [K/128, N] fp16
 *     -> d_w_prepared (16-byte aligned), d_s_prepared (16-byte aligned).
 *     Synchronizes `stream` (the check result is read back).
 *   w4a8_int4g128_gemm_prepared: as w4a8_int4g128_gemm, any M >= 1, with the
 *     kernels of w4a8_mxfp4_gemm_prepared (on wide layers for 9 <= M <= 64
 *     the spread tiles, each code taken as two e2m1 halves; else the split-K
 *     decode kernel for M <= 32 on every layer, and 256-row tiles from 128 of
 *     them on) and its workspace rules (size it with
 *     W4A8_WEIGHT_INT4G128_PREPARED).
 * N % 8 == 0, K % 128 == 0 (else UNSUPPORTED_SHAPE).  Errors: INVALID_ARG,
 * UNSUPPORTED_SHAPE, WORKSPACE, ASYMMETRIC (prepare), HIP. */
w4a8_status w4a8_int4g128_prepared_bytes(int64_t N, int64_t K, size_t *h_w_bytes, size_t *h_s_bytes);
w4a8_status w4a8_int4g128_prepare_fragments(const int32_t *d_qweight_kn, const int32_t *d_qzeros,
                                            const uint16_t *d_scales_f16, int64_t N, int64_t K,
                                            uint8_t *d_w_prepared, uint8_t *d_s_prepared, void *stream);
w4a8_status w4a8_int4g128_gemm_prepared(const uint8_t *d_x_fp8, const float *d_x_scale,
                                        const uint8_t *d_w_prepared, const uint8_t *d_s_prepared,
                                        uint16_t *d_out, int64_t M, int64_t N, int64_t K, void *d_ws,
                                        size_t ws_bytes, void *stream);

/* int4 g128 with a zero point per group and column (asymmetric), in
 * matrix-core fragment order.  Source: "vllm-radiance (MXFP4)", ParoQuant
 * (int4 W4A8 and int5 W5A8): int4 group-128 asymmetric weights on the W4A8
 * path, the zero point folded into the GEMM as a row-sum correction rather
 * than dequantized into the matmul; the checkpoint layout and the zero
 * convention (stored zero - 1) of "radiance_autoround.py", module docstring.
 *   out[m,n] = bf16_RNE( s_m * sum_k e4m3(x8[m,k]) * (c[n,k] - z[k/128,n]) * fp16(scales[k/128,n]) )
 * with c = nibble k % 8 of qweight[k/8, n] and z - 1 = nibble n % 8 of
 * qzeros[k/128, n/8] (fp32 accumulation; summation order may differ).  The
 * products run against c - 8 as in the symmetric form, and (8 - z) times the
 * group's activation sum is added per group before its scale.
 *   w4a8_int4g128_zp_prepared_bytes: sizes of the two buffers (host): the
 *     codes as w4a8_int4g128_prepare_fragments; per 16-row tile and 4-step
 *     chunk one 256-byte record of fp16 scales, bytes 16 - z (both in
 *     lane-group order [row / 4][step][row % 4]) and padding.
 *   w4a8_int4g128_zp_prepare_fragments: qweight [K/8, N], qzeros [K/128, N/8],
 *     scales [K/128, N] fp16 -> d_w_prepared (16-byte aligned), d_s_prepared
 *     (16-byte aligned).  Any zero points; asynchronous.
 *   w4a8_int4g128_zp_gemm_prepared: as w4a8_int4g128_gemm_prepared (routes,
 *     workspace rules, any M >= 1), the workspace sized with
 *     W4A8_WEIGHT_INT4G128_ZP_PREPARED.
 * N % 8 == 0, K % 128 == 0 (else UNSUPPORTED_SHAPE).  Errors: INVALID_ARG,
 * UNSUPPORTED_SHAPE, WORKSPACE, HIP. */
w4a8_status w4a8_int4g128_zp_prepared_bytes(int64_t N, int64_t K, size_t *h_w_bytes, size_t *h_s_bytes);
w4a8_status w4a8_int4g128_zp_prepare_fragments(const int32_t *d_qweight_kn, const int32_t *d_qzeros,
                                               const uint16_t *d_scales_f16, int64_t N, int64_t K,
                                               uint8_t *d_w_prepared, uint8_t *d_s_prepared, void *stream);
w4a8_status w4a8_int4g128_zp_gemm_prepared(const uint8_t *d_x_fp8, const float *d_x_scale,
                                           const uint8_t *d_w_prepared, const uint8_t *d_s_prepared,
                                           uint16_t *d_out, int64_t M, int64_t N, int64_t K, void *d_ws,
                                           size_t ws_bytes, void *stream);

/* int5 g128 (W5A8) in matrix-core fragment order.  Source: "vllm-radiance
 * (MXFP4)", int5 (W5A8): 5-bit codes on the W4A8 path, c - 16 (-16..15) exact
 * in e4m3, the zero point folded as for int4, the low nibbles in the int4
 * word layout and the fifth bit in a plane of its own.  The pages print no
 * checkpoint layout; the one read here:
 *   qweight [K/8, N] int32   the low four bits of each code, as the int4 layout
 *   qweight_hi [K/32, N] int32  the fifth bits: bit k % 32 of word [k/32, n]
 *   qzeros [K/128, N] uint8  z - 1 per group and column (0..31)
 *   scales [K/128, N] fp16
 *   out[m,n] = bf16_RNE( s_m * sum_k e4m3(x8[m,k]) * (c[n,k] - z[k/128,n]) * fp16(scales[k/128,n]) )
 * (fp32 accumulation; summation order may differ).  The split-K decode
 * kernel takes x . (c - 16) as four block-scaled fp4 x fp8 products per step
 * (two 2-bit halves of the low nibble, the fifth bit, a constant -16 term)
 * and adds (16 - z) times the group's activation sum before its scale.  The
 * tile kernel widens c - 16 to e4m3 and adds the zero-point term per 4-step
 * chunk from per-token, per-step activation sums that a pre-pass writes into
 * the workspace.
 *   w4a8_int5g128_prepared_bytes: sizes of the three buffers (host): codes as
 *     the int4 fragment order, the fifth-bit plane (one word per 16-row tile,
 *     step and lane, [tile][4-step chunk][lane][step]: the lane's 32
 *     checkpoint bits with their 2-bit units transposed as a 4 x 4 array), 256-byte scale and zero records per
 *     tile and 4-step chunk.
 *   w4a8_int5g128_prepare_fragments: the checkpoint tensors -> the three
 *     buffers (16-byte aligned).  Asynchronous.
 *   w4a8_int5g128_gemm_prepared: any M >= 1; on wide layers (at least 1536
 *     16-row tiles on 256 CUs, at most 16 per CU) for 9 <= M <= 64 the spread
 *     tiles (no workspace); else M <= 32 the split-K decode kernel, larger M
 *     the tile kernel (64-, 128- or 256-row tiles, 128 wide; K split across
 *     workgroups when the tiles are few).  The workspace (sized with
 *     W4A8_WEIGHT_INT5G128_PREPARED) is required for the tile kernel: it
 *     holds the activation sums; calls that overlap on one workspace race.
 * K % 128 == 0 (else UNSUPPORTED_SHAPE).  Errors: INVALID_ARG,
 * UNSUPPORTED_SHAPE, WORKSPACE, HIP. */
w4a8_status w4a8_int5g128_prepared_bytes(int64_t N, int64_t K, size_t *h_w_bytes, size_t *h_w5_bytes,
                                         size_t *h_s_bytes);
w4a8_status w4a8_int5g128_prepare_fragments(const int32_t *d_qweight_kn, const int32_t *d_qweight_hi,
                                            const uint8_t *d_qzeros, const uint16_t *d_scales_f16, int64_t N,
                                            int64_t K, uint8_t *d_w_prepared, uint8_t *d_w5_prepared,
                                            uint8_t *d_s_prepared, void *stream);
w4a8_status w4a8_int5g128_gemm_prepared(const uint8_t *d_x_fp8, const float *d_x_scale,
                                        const uint8_t *d_w_prepared, const uint8_t *d_w5_prepared,
                                        const uint8_t *d_s_prepared, uint16_t *d_out, int64_t M, int64_t N,
                                        int64_t K, void *d_ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * The linear on bf16 activations in one call: per-token fp8 quantization of
 * x (the rule of w4a8_quant_act_fp8_per_token), then the GEMM on prepared
 * weights.  Source: "radiance_nvfp4.py", module docstring (the W4A8 kernel
 * plugin serves an fp8 activation stream) and "vllm-radiance (MXFP4)", NVFP4
 * checkpoints: online requantization to MXFP4 (fp8 residual stream, norm and
 * quant epilogues feeding the next linear): the quantization leaves its own
 * kernel and joins the linear.
 *   d_x_bf16   device bf16 [M, ldx] (ldx >= K elements, 2-byte aligned)
 *   d_x_fp8    device output e4m3 codes [M, K], 16-byte aligned
 *   d_x_scale  device output fp32 token scales [M], 4-byte aligned: the same
 *              bytes as w4a8_quant_act_fp8_per_token writes
 *   others as w4a8_mxfp4_gemm_prepared / w4a8_int4g128_gemm_prepared, the
 *   workspace sized with the same kind.
 * out equals that GEMM on d_x_fp8 / d_x_scale bit for bit (the same kernel
 * plan, the same products in the same order).  With x 16-byte aligned and
 * ldx % 8 == 0 the quantization joins the GEMM kernel in one launch (codes
 * and scales written out by one workgroup): for one token on a wide MXFP4
 * layer (the spread tiles; K a multiple of 1024, at most 8192) in the spread
 * kernel's prologue, the quantized row staying in LDS; otherwise where the
 * split-K decode kernel serves the GEMM with K unsplit, M <= 16 and the bf16
 * slice fits one batch of its registers (M x K/8 <= 8 x its threads), in
 * that kernel's prologue.  Otherwise the quant kernel runs first, then the
 * GEMM; for 17 <= M <= 64 on a wide MXFP4 layer (the spread tiles) the quant
 * kernel also writes the codes step-major ([K/128][M][128], a step's rows
 * contiguous) into the workspace after its split-K counters, and the tiles
 * read that copy (a workspace without room for it: the codes as written).
 * Errors: INVALID_ARG, UNSUPPORTED_SHAPE, WORKSPACE, HIP. */
w4a8_status w4a8_mxfp4_linear_prepared(const uint16_t *d_x_bf16, int64_t ldx, const uint8_t *d_w_prepared,
                                       const uint8_t *d_s_prepared, uint16_t *d_out, int64_t M, int64_t N,
                                       int64_t K, uint8_t *d_x_fp8, float *d_x_scale, void *d_ws,
                                       size_t ws_bytes, void *stream);
w4a8_status w4a8_int4g128_linear_prepared(const uint16_t *d_x_bf16, int64_t ldx, const uint8_t *d_w_prepared,
                                          const uint8_t *d_s_prepared, uint16_t *d_out, int64_t M, int64_t N,
                                          int64_t K, uint8_t *d_x_fp8, float *d_x_scale, void *d_ws,
                                          size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * w4a8_mxfp4_gemm_prepared without a workspace argument.  Its split-K partials
 * go to a static device array of the library (one per GPU, of
 * w4a8_mxfp4_gemm_prepared_noalloc_max_scratch() bytes = 16 MiB, held until
 * the process ends); the call allocates and frees nothing.  The caller passes
 * inputs and outputs as for w4a8_mxfp4_gemm_prepared, on the device current at
 * the call (the first call on a device looks the array's address up on it).
 * Every call on one GPU uses that GPU's array, so calls that overlap on one
 * GPU (concurrent streams) race; calls ordered on a stream do not.  Results
 * are identical to w4a8_mxfp4_gemm_prepared's.  Errors as that call, and
 * WORKSPACE when the call's split-K partials need more than the array
 * (sizes: w4a8_gemm_workspace_bytes with kind MXFP4_PREPARED). */
w4a8_status w4a8_mxfp4_gemm_prepared_noalloc(const uint8_t *d_x_fp8, const float *d_x_scale,
                                             const uint8_t *d_w_prepared, const uint8_t *d_s_prepared,
                                             uint16_t *d_out, int64_t M, int64_t N, int64_t K, void *stream);
size_t      w4a8_mxfp4_gemm_prepared_noalloc_max_scratch(void);

/* ---------------------------------------------------------------------------
 * Decode band with an explicit plan, for tile-size sweeps (the two GEMM entry
 * points above pick these parameters themselves).  Computes exactly what
 * w4a8_mxfp4_gemm (kind MXFP4: d_w = packed codes, d_w_scale = e8m0) or
 * w4a8_int4g128_gemm (kind INT4G128: d_w = qweight [N, K/8], d_w_scale = fp16
 * scales) computes, for 1 <= M <= 64, with
 *   rt  16-row weight tiles per wavefront (1, 2 or 4; 4 waves per workgroup),
 *   u   128-wide K steps per prefetched chunk (1, 2 or 4; 1 if K % 128 != 0),
 *   ks  requested K splits (>= 1; rounded so each split holds whole chunks).
 * Kind MXFP4_PREPARED (prepared weights) selects one of the kernels that
 * w4a8_mxfp4_gemm_prepared chooses among, with the plan given here:
 *   rt = 0        split-K decode kernel (M <= 32), the entry point's tiles per
 *                 workgroup and K splits; u = register ring depth in 512-wide
 *                 chunks (2, 3 or 4), ks = K parts per tile inside a workgroup
 *                 (clamped to 16 waves per workgroup and to the split's chunks);
 *   rt = 100 + t  the same kernel with t tiles per workgroup (t * ks <= 16), K
 *                 split across workgroups only as far as the activation slice
 *                 needs to fit 160 KB of LDS;
 *   rt = -r       register-streamed tiles (M <= 64): r = 1, 2 or 4 tiles per
 *                 wave, u = 4, 8 or 16 waves per workgroup, ks = K splits
 *                 across workgroups;
 *   rt = -100     the LDS-tiled kernel with K split in ks parts (any M);
 *   rt = -200     spread tiles (M <= 64): one workgroup per CU, each over all
 *                 of K, ks = weight ring depth in 128-wide steps (4 or 8, 0 =
 *                 the entry point's choice; UNSUPPORTED_SHAPE unless it
 *                 divides the padded step count), u ignored; no workspace.
 * w4a8_decode_plan_workspace_bytes: workspace for that plan (0 = none needed, or
 * invalid arguments; rt = 0, rt > 100 and rt < 0 select the prepared-weight
 * plans above).  Errors as the GEMMs, INVALID_ARG for a bad plan. */
size_t      w4a8_decode_plan_workspace_bytes(int64_t M, int64_t N, int64_t K, int rt, int u, int ks);
w4a8_status w4a8_decode_with_plan(w4a8_weight_kind kind, const uint8_t *d_x_fp8,
                                  const float *d_x_scale, const void *d_w, const void *d_w_scale,
                                  uint16_t *d_out, int64_t M, int64_t N, int64_t K, int rt, int u,
                                  int ks, void *d_ws, size_t ws_bytes, void *stream);

/* Static strings; never NULL. */
const char *w4a8_status_string(w4a8_status s);
const char *w4a8_version(void);

#ifdef __cplusplus
}
#endif
#endif /* W4A8_H */
