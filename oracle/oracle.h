/*
 * oracle.h -- CPU oracle for the MXFP4 W4A8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library (w4a8_gemm_amd/) includes,
 * links, loads or calls this code; only tests/, the smoke check in
 * __graft_entry__.py and the cpu_baseline leg of bench.py do.  It shares no
 * source, table or helper with the HIP path.
 *
 * Plain, slow, obviously correct C: scalar loops, IEEE fp32 where the pages
 * compute in fp32 (the requant), fp64 for the GEMM reference.  Built with
 * gcc -O2 -ffp-contract=off (no fused multiply-add, no fast-math), OpenMP over
 * independent rows only (results do not depend on the thread count).
 *
 * Sources (cited by page title and section, never by line):
 *   [P1] "radiance_nvfp4.py" -- unpack_e2m1, dequant_nvfp4, e2m1_index,
 *        _block_exponent, _encode_blocks, quant_mxfp4, dequant_mxfp4,
 *        requant_rows, RadianceNvfp4ToMxfp4.process_weights_after_loading,
 *        RadianceBf16ToMxfp4 and RadianceFp8ChannelToMxfp4
 *        .process_weights_after_loading.
 *   [P2] "vllm-radiance (MXFP4)" -- How the MXFP4 path works: The W4A8
 *        fp8-WMMA kernel; NVFP4 checkpoints: online requantization to MXFP4.
 *   [P3] "radiance_autoround.py" -- module docstring (int4 format),
 *        _exact_ref, autoround_linear, process_weights_after_loading.
 */
#ifndef W4A8_ORACLE_H
#define W4A8_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_OCP = 0, ORC_NOCLIP = 1, ORC_MSE = 2 };

/* --- number formats ------------------------------------------------------ */
float   orc_e2m1_value(int code);            /* [P1] unpack_e2m1 */
double  orc_e4m3_value(uint8_t b);           /* OCP E4M3FN; NaN for 0x7F/0xFF */
float   orc_bf16_value(uint16_t h);
uint8_t orc_e4m3_encode(float y);            /* RNE, saturate at 448, sign kept */
int     orc_e2m1_index(float a);             /* [P1] e2m1_index (argmin, even ties) */
int     orc_block_exponent(float amax, int mode); /* [P1] _block_exponent */

/* --- MXFP4 encoding of fp32 rows ([P1] quant_mxfp4) ----------------------- */
float   orc_encode_block(const float *w32, int e, uint8_t *idx32);  /* _encode_blocks */
int     orc_quant_block(const float *w32, int mode, uint8_t *code32, float *err);
void    orc_quant_mxfp4(const float *w, int64_t rows, int64_t K, int mode,
                        uint8_t *packed, uint8_t *e8m0, float *block_err,
                        double *err_sum, double *ssq);
void    orc_dequant_mxfp4(const uint8_t *packed, const uint8_t *e8m0,
                          int64_t rows, int64_t K, float *w);

/* --- NVFP4 -> MXFP4 ([P1] dequant_nvfp4, requant_rows, process_weights) --- */
void    orc_dequant_nvfp4(const uint8_t *packed, const uint8_t *scale_e4m3,
                          int64_t rows, int64_t K, float divisor, float *w);
int     orc_requant_nvfp4_to_mxfp4(const uint8_t *nv_packed, const uint8_t *nv_scale,
                                   const int64_t *part_rows, const float *part_divisor,
                                   int n_parts, int64_t K, int mode, int64_t row_chunk,
                                   uint8_t *mx_packed, uint8_t *mx_e8m0, double *stats);

/* --- bf16 / fp8 per-channel -> MXFP4 ([P1] RadianceBf16ToMxfp4,
 *     RadianceFp8ChannelToMxfp4) ------------------------------------------ */
int     orc_quant_bf16_to_mxfp4(const uint16_t *w_bf16, int64_t rows, int64_t K, int mode,
                                uint8_t *mx_packed, uint8_t *mx_e8m0, double *stats);
int     orc_quant_fp8ch_to_mxfp4(const uint8_t *w_e4m3, const float *row_scale, int64_t rows,
                                 int64_t K, int mode, uint8_t *mx_packed, uint8_t *mx_e8m0,
                                 double *stats);

/* --- per-token fp8 activations ------------------------------------------- */
int     orc_quant_act_fp8(const uint16_t *x_bf16, int64_t M, int64_t K, int64_t ldx,
                          uint8_t *x8, float *x_scale);

/* --- GEMM references ([P3] _exact_ref, adapted to MXFP4) ------------------ */
void    orc_mxfp4_gemm(const uint8_t *x8, const float *x_scale, const uint8_t *w_packed,
                       const uint8_t *w_e8m0, int64_t M, int64_t N, int64_t K,
                       const int64_t *mi, const int64_t *ni, int64_t count, double *ref);
void    orc_w4a4_gemm(const uint8_t *x_packed, const uint8_t *x_e8m0, const uint8_t *w_packed,
                      const uint8_t *w_e8m0, int64_t M, int64_t N, int64_t K,
                      const int64_t *mi, const int64_t *ni, int64_t count, double *ref);
int     orc_int4_prepare(const int32_t *qweight_kn, const int32_t *qzeros,
                         int64_t N, int64_t K, int32_t *qweight_nk);
void    orc_int4_gemm(const uint8_t *x8, const float *x_scale, const int32_t *qweight_nk,
                      const uint16_t *scales_f16, int64_t M, int64_t N, int64_t K,
                      const int64_t *mi, const int64_t *ni, int64_t count, double *ref);
void    orc_int4_zp_gemm(const uint8_t *x8, const float *x_scale, const int32_t *qweight_kn,
                         const int32_t *qzeros, const uint16_t *scales_f16, int64_t M, int64_t N, int64_t K,
                         const int64_t *mi, const int64_t *ni, int64_t count, double *ref);
void    orc_int5_gemm(const uint8_t *x8, const float *x_scale, const int32_t *qweight_kn,
                      const int32_t *qweight_hi, const uint8_t *qzeros, const uint16_t *scales_f16,
                      int64_t M, int64_t N, int64_t K, const int64_t *mi, const int64_t *ni, int64_t count,
                      double *ref);
double  orc_f16_value(uint16_t h);

/* array forms (loops over the scalar functions) */
void    orc_e2m1_index_array(const float *a, int64_t n, uint8_t *out);
void    orc_block_exponent_array(const float *amax, int64_t n, int mode, int32_t *out);
void    orc_e4m3_encode_array(const float *y, int64_t n, uint8_t *out);

#ifdef __cplusplus
}
#endif
/* threads of the parallel loops (timing only) */
void orc_set_threads(int n);
int orc_max_threads(void);

#endif
