// w4a8_internal.h -- shared declarations of libw4a8's kernels and launchers.
//
// Device helpers here are the library's own number-format code (bit-level, exact);
// nothing in this tree is shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "w4a8.h"

namespace w4a8 {

// ---------------------------------------------------------------------------
// exact format conversions
// ---------------------------------------------------------------------------

// OCP E4M3FN byte -> fp32 (exact; the NaN codes never reach these kernels).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t E = (b >> 3) & 15u, m = b & 7u;
    const float mag = E ? __uint_as_float(((E + 120u) << 23) | (m << 20))
                        : (float)m * 0x1p-9f;
    return (b & 0x80u) ? -mag : mag;
}

// e2m1 magnitude index 0..7 -> {0, .5, 1, 1.5, 2, 3, 4, 6}: the index placed in
// the top of the fp32 exponent/mantissa field is that value times 2^-126 (a
// subnormal for indices 0 and 1), so one exact multiply rebiases it.  Needs fp32
// denormals preserved (the library is built without flush-to-zero).
__device__ __forceinline__ float e2m1_mag(uint32_t idx) {
    return __uint_as_float(idx << 22) * 0x1p126f;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// fp32 -> E4M3FN, round to nearest even, magnitudes at or above 448 saturate to
// 448 (0x7E), sign bit kept (so -0 and negative values that round to zero give
// 0x80).  Integer rounding on the fp32 bits for the normal range, an exact
// scaling plus rint for the subnormal range.
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// A 16-byte load with the non-temporal hint: the fragment-order decode
// kernel reads each weight (and scale) byte once per launch, and keeping it
// out of the caches' reuse (gfx950 `nt`) measured 3-8 % faster on its weight
// stream (gate_up M = 1: 18.8 -> 18.0 us; with the scale loads too, 17.8).
// The tile kernels' copies keep the default policy (the hint slowed the
// K-split down_proj tiles, M = 64: 24 -> 27 us), and so do the row-major
// decode kernels (gate_up M = 1: 25 -> 29 us with it).
__device__ __forceinline__ uint4 load_stream16(const uint4* p) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Eight int4 codes (one word, nibble j = k j) -> eight e4m3 bytes of (c - 8) in
// k order.  Codes 0..7 map to -8..-1 and 8..15 to 0..7; each half is an 8-byte
// table indexed by c & 7, and bit 3 picks the half.
// The same with the two 8-byte halves of the table given: lo = e4m3 of codes
// 0..7, hi = codes 8..15 (for a zero point z: e4m3(c - z), exact for
// c - z in [-16, 14]).
__device__ __forceinline__ uint2 int4x8_to_e4m3_tab(uint32_t w, uint32_t lo0, uint32_t lo1, uint32_t hi0,
                                                    uint32_t hi1) {
    const uint32_t ev = w & 0x0F0F0F0Fu;
    const uint32_t od = (w >> 4) & 0x0F0F0F0Fu;
    const uint32_t se = ev & 0x07070707u, so = od & 0x07070707u;
    const uint32_t ne = __builtin_amdgcn_perm(lo1, lo0, se);
    const uint32_t pe = __builtin_amdgcn_perm(hi1, hi0, se);
    const uint32_t no = __builtin_amdgcn_perm(lo1, lo0, so);
    const uint32_t po = __builtin_amdgcn_perm(hi1, hi0, so);
    const uint32_t me = ((ev >> 1) & 0x04040404u) | 0x03020100u;
    const uint32_t mo = ((od >> 1) & 0x04040404u) | 0x03020100u;
    const uint32_t e = __builtin_amdgcn_perm(pe, ne, me);
    const uint32_t o = __builtin_amdgcn_perm(po, no, mo);
    return make_uint2(__builtin_amdgcn_perm(o, e, 0x05010400u), __builtin_amdgcn_perm(o, e, 0x07030602u));
}

__device__ __forceinline__ uint2 int4x8_to_e4m3(uint32_t w) {
    const uint32_t kNegLo = 0xCACCCED0u, kNegHi = 0xB8C0C4C8u;  // -8 -7 -6 -5 | -4 -3 -2 -1
    const uint32_t kPosLo = 0x44403800u, kPosHi = 0x4E4C4A48u;  //  0  1  2  3 |  4  5  6  7
    const uint32_t ev = w & 0x0F0F0F0Fu;          // k = 0, 2, 4, 6
    const uint32_t od = (w >> 4) & 0x0F0F0F0Fu;   // k = 1, 3, 5, 7
    const uint32_t se = ev & 0x07070707u, so = od & 0x07070707u;
    const uint32_t ne = __builtin_amdgcn_perm(kNegHi, kNegLo, se);
    const uint32_t pe = __builtin_amdgcn_perm(kPosHi, kPosLo, se);
    const uint32_t no = __builtin_amdgcn_perm(kNegHi, kNegLo, so);
    const uint32_t po = __builtin_amdgcn_perm(kPosHi, kPosLo, so);
    const uint32_t me = ((ev >> 1) & 0x04040404u) | 0x03020100u;  // byte i -> i, or i+4 if c >= 8
    const uint32_t mo = ((od >> 1) & 0x04040404u) | 0x03020100u;
    const uint32_t e = __builtin_amdgcn_perm(pe, ne, me);
    const uint32_t o = __builtin_amdgcn_perm(po, no, mo);
    return make_uint2(__builtin_amdgcn_perm(o, e, 0x05010400u), __builtin_amdgcn_perm(o, e, 0x07030602u));
}

__device__ __forceinline__ uint32_t f32_to_e4m3_rne_sat(float y) {
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fminf(fabsf(y), 448.0f);
    uint32_t code;
    if (a < 0x1p-6f) {
        code = (uint32_t)rintf(a * 512.0f);  // 0..8; 8 is the smallest normal
    } else {
        const uint32_t b = __float_as_uint(a);
        code = (b - (120u << 23) + 0x7FFFFu + ((b >> 20) & 1u)) >> 20;
    }
    return sign | code;
}

// ---------------------------------------------------------------------------
// launchers (host side; each returns a hipError_t from the launch)
// ---------------------------------------------------------------------------

// NVFP4 -> MXFP4 over n_parts consecutive partitions (part_blocks[i] 32-element
// blocks each, divisor part_divisor[i]; host arrays), one launch; stats: per
// partition {sum err, sum w^2} accumulated into stats[2i], stats[2i + 1]
hipError_t launch_requant(const uint8_t* nv_packed, const uint8_t* nv_scale, const int64_t* part_blocks,
                          const float* part_divisor, int n_parts, int mode, uint8_t* mx_packed,
                          uint8_t* mx_e8m0, double* stats, hipStream_t stream);
int requant_max_parts();   // partitions one launch_requant call takes
// bf16 / fp8-per-channel weights -> MXFP4 (the requant encoder, other input stages)
hipError_t launch_quant_bf16(const uint16_t* w, int64_t rows, int64_t K, int mode, uint8_t* mx_packed,
                             uint8_t* mx_e8m0, double* stats, hipStream_t stream);
hipError_t launch_quant_fp8ch(const uint8_t* w, const float* row_scale, int64_t rows, int64_t K, int mode,
                              uint8_t* mx_packed, uint8_t* mx_e8m0, double* stats, hipStream_t stream);
// the same encoders writing the fragment order of w4a8_mxfp4_prepare directly
// (K % 128 == 0; wt / st sized by prepared_sizes(rows, K); no statistics)
hipError_t launch_requant_prepared(const uint8_t* nv_packed, const uint8_t* nv_scale, const int64_t* part_blocks,
                                   const float* part_divisor, int n_parts, int64_t rows, int64_t K, int mode,
                                   uint8_t* wt, uint8_t* st, hipStream_t stream);
hipError_t launch_quant_bf16_prepared(const uint16_t* w, int64_t rows, int64_t K, int mode, uint8_t* wt,
                                      uint8_t* st, hipStream_t stream);
hipError_t launch_quant_fp8ch_prepared(const uint8_t* w, const float* row_scale, int64_t rows, int64_t K, int mode,
                                       uint8_t* wt, uint8_t* st, hipStream_t stream);
hipError_t launch_fill_zero_f64(double* p, int64_t n, hipStream_t stream);
hipError_t launch_fill_zero_u32(uint32_t* p, int64_t n, hipStream_t stream);

hipError_t launch_act_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* x8,
                            float* xs, hipStream_t stream);
// the same codes also written step-major to x8s ([K/128][M][128], 16-byte
// aligned), where the single-pass kernel serves the shape (act_quant_sm_fits)
bool act_quant_sm_fits(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint8_t* x8);
hipError_t launch_act_quant_sm(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* x8, float* xs,
                               uint8_t* x8s, hipStream_t stream);

// GEMM plans: the host picks the band, the tile and the K split.
struct GemmPlan {
    int band;       // 0 decode (weights streamed, split K), 1 prefill (LDS tiles)
    int mt;         // decode: 16-wide activation tiles (1..4)
    int rt;         // decode: 16-row weight tiles per wave
    int u;          // decode: 128-wide K steps per prefetched chunk
    int ks;         // decode: K splits (1 = no workspace traffic)
    int s_per;      // decode: 128-wide K steps per split
    int64_t tiles;  // decode: row blocks of the weight
    int kw;         // prepared decode: K parts per tile inside a workgroup
    int ab;         // prepared decode: activation loads per thread and batch (4 or 8)
};
GemmPlan make_decode_plan(int64_t M, int64_t N, int64_t K, int rt, int u, int ks_hint);
GemmPlan plan_mxfp4(int64_t M, int64_t N, int64_t K);
GemmPlan plan_int4(int64_t M, int64_t N, int64_t K);
size_t plan_workspace_bytes(const GemmPlan& p, int64_t M, int64_t N);

hipError_t launch_mxfp4_gemm(const GemmPlan& p, const uint8_t* x8, const float* xs,
                             const uint8_t* wq, const uint8_t* we, uint16_t* out, int64_t M,
                             int64_t N, int64_t K, void* ws, hipStream_t stream);

// MXFP4 weights in fragment order (gemm_prepared.hip)
void prepared_sizes(int64_t N, int64_t K, size_t* w_bytes, size_t* s_bytes);
hipError_t launch_prepare(const uint8_t* wq, const uint8_t* we, int64_t N, int64_t K, uint8_t* wt,
                          uint8_t* st, hipStream_t stream);
// split-K decode plan on prepared weights; depth 0 = the plan's own ring depth
GemmPlan plan_prepared(int64_t M, int64_t N, int64_t K, int ks_hint, int depth, bool a4, bool int4);
size_t prepared_lds_bytes(const GemmPlan& p, int64_t M, bool a4 = false);
GemmPlan plan_prepared_explicit(int64_t M, int64_t N, int64_t K, int tw, int kw, int depth);
// zp: int4 weights with zero points (prepared by launch_prepare_i4z)
hipError_t launch_prepared_decode(const GemmPlan& p, const uint8_t* x8, const float* xs,
                                  const uint8_t* wt, const uint8_t* st, uint16_t* out, int64_t M,
                                  int64_t N, int64_t K, void* ws, hipStream_t stream, bool int4, bool zp);
// Which kernel serves a GEMM on prepared weights: the split-K decode kernel
// (M <= 32 on narrow layers and for int4 weights; on wide MXFP4 layers up to
// M = 16 while the activation slice of all of K fits one workgroup's LDS) or
// the tiled kernel (K split across workgroups when its tiles are few).
// DTile: the register-streamed tiles (narrow MXFP4 layers, 9 to 40 rows).
// Spread: the spread tiles (wide layers, M <= 64; int4 and its zero-point
// form from 9 rows).
enum class PreparedRoute { Decode, Tiled, DTile, Spread };
PreparedRoute prepared_route(int64_t M, int64_t N, int64_t K, bool int4);
// force_ks > 1: K split in that many parts where the shape rules would not (tuning)
size_t tiled_workspace_bytes(int64_t M, int64_t N, int64_t K, bool int4, int force_ks = 0);
// The linear on bf16 activations with the per-token fp8 quantization fused
// into the split-K decode kernel's prologue (one launch), where the plan
// allows it (plan_prepared_fused); codes and scales also written to x8_out /
// xs_out by one workgroup.
bool plan_prepared_fused(int64_t M, int64_t N, int64_t K, bool int4, GemmPlan* out);
hipError_t launch_prepared_linear_fused(const GemmPlan& p, const uint16_t* xb, int64_t ldx, const uint8_t* wt,
                                        const uint8_t* st, uint16_t* out, int64_t M, int64_t N, int64_t K,
                                        uint8_t* x8_out, float* xs_out, hipStream_t stream, bool int4);
// W4A4 (MXFP4 activations, prepared MXFP4 weights): the split-K decode
// kernel's W4A4 variant where w4a4_decode_route says so, else the fp4 x fp4
// tile kernel
bool w4a4_decode_route(int64_t M, int64_t N);
size_t w4a4_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_prepared_w4a4(const uint8_t* x4, const uint8_t* xe, const uint8_t* wt, const uint8_t* st,
                                uint16_t* out, int64_t M, int64_t N, int64_t K, void* ws, hipStream_t stream);
hipError_t launch_prepared_tiled(const uint8_t* x8, const float* xs, const uint8_t* wt,
                                 const uint8_t* st, uint16_t* out, int64_t M, int64_t N, int64_t K,
                                 void* ws, hipStream_t stream, bool int4, bool zp, int force_ks = 0);
// int4 g128 in fragment order (same weight geometry as MXFP4; row scales
// [tile][chunk][step][16] fp16)
void prepared_i4_sizes(int64_t N, int64_t K, size_t* w_bytes, size_t* s_bytes);
// int4 with zero points: codes as launch_prepare_i4, scales and zeros in 256-byte records
void prepared_i4z_sizes(int64_t N, int64_t K, size_t* w_bytes, size_t* s_bytes);
hipError_t launch_prepare_i4z(const int32_t* qkn, const int32_t* qz, const uint16_t* sc, int64_t N, int64_t K,
                              uint8_t* wt, uint8_t* st, hipStream_t stream);
// int5: codes' low bits as launch_prepare_i4, a fifth-bit plane, records as int4 with zero points
void prepared_i5_sizes(int64_t N, int64_t K, size_t* w_bytes, size_t* w5_bytes, size_t* s_bytes);
hipError_t launch_prepare_i5(const int32_t* qkn, const int32_t* qhi, const uint8_t* qz, const uint16_t* sc,
                             int64_t N, int64_t K, uint8_t* wt, uint8_t* w5, uint8_t* st, hipStream_t stream);
// the split-K decode kernel on int5 weights, M <= 32
size_t i5_tiled_workspace_bytes(int64_t M, int64_t N, int64_t K);
bool i5_tiled_fits(int64_t M, int64_t K);
hipError_t launch_prepared_tiled_i5(const uint8_t* x8, const float* xs, const uint8_t* wt, const uint8_t* w5,
                                    const uint8_t* st, uint16_t* out, int64_t M, int64_t N, int64_t K, void* ws,
                                    hipStream_t stream);
hipError_t launch_prepared_decode_i5(const uint8_t* x8, const float* xs, const uint8_t* wt, const uint8_t* w5,
                                     const uint8_t* st, uint16_t* out, int64_t M, int64_t N, int64_t K, void* ws,
                                     hipStream_t stream);
hipError_t launch_prepare_i4(const int32_t* qkn, const uint16_t* sc, int64_t N, int64_t K, uint8_t* wt,
                             uint8_t* st, hipStream_t stream);
// the same from the transposed [N, K/8] codes (w4a8_int4g128_gemm's layout)
hipError_t launch_prepare_i4_nk(const int32_t* qnk, const uint16_t* sc, int64_t N, int64_t K, uint8_t* wt,
                                uint8_t* st, hipStream_t stream);
// Register-streamed tiles on prepared MXFP4 weights (decode band, M <= 64):
// R 16-row tiles per wave, W waves per workgroup, K split across ks
// workgroups (h_per two-step units each).
struct DtPlan {
    int mt, r, w, ks, h_per;
    int64_t tiles, groups;
};
DtPlan plan_dtile(int64_t M, int64_t N, int64_t K, int R, int W, int ks);
DtPlan plan_dtile_route(int64_t M, int64_t N, int64_t K);
size_t dtile_workspace_bytes(const DtPlan& p, int64_t M, int64_t N);
hipError_t launch_dtile(const DtPlan& p, const uint8_t* x8, const float* xs, const uint8_t* wt, const uint8_t* st,
                        uint16_t* out, int64_t M, int64_t N, int64_t K, void* ws, hipStream_t stream);
// Spread tiles on prepared MXFP4 weights (wide layers, M <= 64): one
// workgroup of eight waves per CU, the 16-row tiles dealt out evenly (at most
// R per wave), all of K per workgroup; D = weight ring depth in steps (0:
// the default for the shape).
struct SpPlan {
    int mt, r, d, cs;     // cs: e8m0 dwords once per 4-step chunk (ring depth 4, padded steps a multiple of 8)
    int64_t tiles, groups;
};
SpPlan plan_spread(int64_t M, int64_t N, int64_t K, int D, int CS);
bool spread_fits(int64_t M, int64_t N, int64_t K);
bool spread_plain_fits(int64_t M, int64_t N, int64_t K);
// the linear on one bf16 token (16-byte aligned row) with the quantization
// fused into the spread tiles; x8_out / xs_out receive the codes and the scale
bool spread_fq_fits(int64_t M, int64_t N, int64_t K);
hipError_t launch_spread_fq(const uint16_t* xb, const uint8_t* wt, const uint8_t* st, uint16_t* out,
                            uint8_t* x8_out, float* xs_out, int64_t N, int64_t K, hipStream_t stream);
// plain: wt / st are the plain layout ([N, K/2] codes, [N, K/32] e8m0, both
// 16-byte aligned, K / 128 a multiple of 8) instead of fragment order;
// x_step_major: the codes x8 in step-major order [K/128][M][128] (a step's
// rows contiguous) instead of [M, K]
hipError_t launch_spread(const SpPlan& p, const uint8_t* x8, const float* xs, const uint8_t* wt, const uint8_t* st,
                         uint16_t* out, int64_t M, int64_t N, int64_t K, hipStream_t stream, bool plain = false,
                         bool x_step_major = false);
// int4 / int5 g128 fragment-order weights on the spread tiles (wt codes, st
// the row-scale records per tile and chunk: 128 bytes, or 256 with the zero
// bytes; w5 the int5 fifth-bit planes, else null); x8 row-major.  wf: 1 int4,
// 3 int4 with zero points, 4 int5
hipError_t launch_spread_i4(const uint8_t* x8, const float* xs, const uint8_t* wt, const uint8_t* st, uint16_t* out,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream, int wf, const uint8_t* w5);
// W4A4 (e2m1 codes x4 [M, K/2], e8m0 xe [M, K/32]) on the spread tiles
bool spread_a4_fits(int64_t M, int64_t N, int64_t K);
hipError_t launch_spread_a4(const uint8_t* x4, const uint8_t* xe, const uint8_t* wt, const uint8_t* st,
                            uint16_t* out, int64_t M, int64_t N, int64_t K, hipStream_t stream);
constexpr int64_t kPreparedDecodeMaxM = 32;
// largest K of the tiled kernel on prepared weights (32-bit buffer offsets
// into a 256-row activation block: 256 * K < 2^32)
constexpr int64_t kPreparedTiledMaxK = (1 << 24) - 128;

hipError_t launch_int4_check_transpose(const int32_t* qw_kn, const int32_t* qzeros, int64_t N,
                                       int64_t K, int32_t* qw_nk, uint32_t* bad_count,
                                       hipStream_t stream);
hipError_t launch_int4_gemm(const GemmPlan& p, const uint8_t* x8, const float* xs,
                            const int32_t* qw_nk, const uint16_t* scales, uint16_t* out,
                            int64_t M, int64_t N, int64_t K, void* ws, hipStream_t stream);

// out[m, n] = bf16(s_m * sum_j partials[j, m, n]) in split order (decode split K)
hipError_t launch_splitk_reduce(const float* partials, const float* xs, int64_t M, int64_t N,
                                int ks, uint16_t* out, hipStream_t stream);

// Split-K workspace layout: a 256-byte-aligned header region (one arrival
// counter per 16-row tile or group of tiles, zero between calls), then fp32
// partials [ks][M][N].
inline size_t ws_counter_bytes(int64_t tiles) {
    return (size_t)((tiles * 4 + 255) / 256 * 256);
}

// ---------------------------------------------------------------------------
// Split-K reduced in place by the last split to arrive ("vllm-radiance
// (MXFP4)", How the MXFP4 path works, The W4A8 fp8-WMMA kernel: the K splits
// of an output block race on a counter, and the one that arrives last adds
// the partials, with no second launch).
//
// The eight XCDs of an MI355X have L2 caches of their own, and the splits of
// one block run on any of them.  Partials are therefore written and read with
// device-scope relaxed atomic accesses: on gfx950 ordinary loads and stores
// carrying the sc1 bit, which go to the device's coherence point instead of
// staying in (or being served from) the XCD's L2.  A split waits for its
// stores to complete (vmcnt(0)) before its workgroup barrier, and one thread
// then increments the block's counter (a device-scope atomic); the split that
// reads ks - 1 is the last, resets the counter to zero for the next call and
// sums the ks partials in split order, so the output is bit-identical to the
// separate reduction kernel's.  No release or acquire fence is needed (at
// device scope those write back or invalidate the whole L2), and no split
// waits for another: the splits that are not last simply end.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void sk_put(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float sk_get(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte forms for four consecutive columns: buffer accesses with the same
// sc1 bit (cache-policy operand 16), addressed by a 32-bit byte offset from
// the partials' base (the host keeps ks x M x N x 4 below 2^31)
typedef int32_t sk_i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t sk_rsrc(const float* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ void sk_put4(__amdgpu_buffer_rsrc_t r, uint32_t off, float a, float b, float c, float d) {
    const sk_i32x4 v = {__float_as_int(a), __float_as_int(b), __float_as_int(c), __float_as_int(d)};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 16);
}
__device__ __forceinline__ sk_i32x4 sk_get4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 16);
}
// Every thread of the workgroup calls it (after its partial stores); true in
// the last split of the block.  flag: one word of LDS.
__device__ __forceinline__ bool sk_arrive(uint32_t* counter, int ks, uint32_t* flag) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = old == (uint32_t)(ks - 1);
        if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = last ? 1u : 0u;
    }
    __syncthreads();
    return *flag != 0u;
}
// Host: whether a K split of ks parts over an M x N output reduces in place
// (partials addressed with 32-bit byte offsets).
inline bool sk_inplace_fits(int64_t ks, int64_t M, int64_t N) {
    return ks >= 2 && ks * M * N * 4 < ((int64_t)1 << 31);
}

// The last split's sum over rows m < M and columns [n_lo, n_hi): out = bf16(s_m
// x (p_0 + p_1 + ... + p_{ks-1})) in split order (xs null: no token scale).
// Atomic loads keep their program order, so each thread issues a batch of
// loads (up to kSkBatch splits of its outputs) before the batch's adds: one
// memory latency per batch instead of one per partial, in 32 registers.  With
// N, n_lo and n_hi multiples of 4 the loads are 16 bytes (four columns) each.
constexpr int kSkBatch = 8;
__device__ __forceinline__ void sk_reduce(const float* partials, const float* xs, int M, int N, int ks, int n_lo,
                                          int n_hi, uint16_t* out, int tid, int nthreads) {
    const int64_t plane = (int64_t)M * N;
    const int w = n_hi - n_lo;
    if ((N & 3) == 0 && (n_lo & 3) == 0 && (w & 3) == 0) {
        const __amdgpu_buffer_rsrc_t r = sk_rsrc(partials);
        const int w4 = w >> 2, total = M * w4;
        for (int i = tid; i < total; i += nthreads) {
            const int m = i / w4;
            const uint32_t o = (uint32_t)((int64_t)m * N + n_lo + 4 * (i - m * w4));
            float t0 = 0.f, t1 = 0.f, t2 = 0.f, t3 = 0.f;
            for (int j0 = 0; j0 < ks; j0 += kSkBatch) {
                sk_i32x4 v[kSkBatch];
#pragma unroll
                for (int j = 0; j < kSkBatch; ++j)
                    if (j0 + j < ks) v[j] = sk_get4(r, 4u * (uint32_t)((j0 + j) * plane + o));
#pragma unroll
                for (int j = 0; j < kSkBatch; ++j)
                    if (j0 + j < ks) {
                        if (j0 + j == 0) {
                            t0 = __int_as_float(v[j][0]); t1 = __int_as_float(v[j][1]);
                            t2 = __int_as_float(v[j][2]); t3 = __int_as_float(v[j][3]);
                        } else {
                            t0 = t0 + __int_as_float(v[j][0]); t1 = t1 + __int_as_float(v[j][1]);
                            t2 = t2 + __int_as_float(v[j][2]); t3 = t3 + __int_as_float(v[j][3]);
                        }
                    }
            }
            const float sm = xs ? xs[m] : 1.0f;
            const uint32_t h0 = f32_to_bf16_rne(sm * t0) | (f32_to_bf16_rne(sm * t1) << 16);
            const uint32_t h1 = f32_to_bf16_rne(sm * t2) | (f32_to_bf16_rne(sm * t3) << 16);
            *reinterpret_cast<uint2*>(out + o) = make_uint2(h0, h1);
        }
        return;
    }
    const int total = M * w;
    for (int i = tid; i < total; i += nthreads) {
        const int m = i / w;
        const int64_t o = (int64_t)m * N + n_lo + (i - m * w);
        float t = 0.f;
        for (int j0 = 0; j0 < ks; j0 += kSkBatch) {
            float v[kSkBatch];
#pragma unroll
            for (int j = 0; j < kSkBatch; ++j)
                if (j0 + j < ks) v[j] = sk_get(partials + (j0 + j) * plane + o);
#pragma unroll
            for (int j = 0; j < kSkBatch; ++j)
                if (j0 + j < ks) t = j0 + j == 0 ? v[j] : t + v[j];
        }
        const float sm = xs ? xs[m] : 1.0f;
        out[o] = (uint16_t)f32_to_bf16_rne(sm * t);
    }
}

}  // namespace w4a8
